// C ABI of the relative-position-bias attention library: argument validation
// (pure host code, before any HIP call) and dispatch to the gfx950 kernels.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "relbias_attn.h"
#include "rba_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return RBA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

constexpr int kMaxBiasRange = 1 << 20;

// Checks shared by prefill and decode.  Returns RBA_OK or an error code.
int check_common(const char* fn, int dtype, int Hq, int Hkv, int D, int window, int bias_range,
                 int mode, const float* table, const void* r, const float* E, int R, float scale) {
  if (dtype != RBA_F32 && dtype != RBA_BF16) return fail(RBA_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (Hq < 1 || Hkv < 1) return fail(RBA_EINVAL, "%s: Hq=%d and Hkv=%d must be >= 1", fn, Hq, Hkv);
  if (Hq % Hkv) return fail(RBA_EINVAL, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (window < 0) return fail(RBA_EINVAL, "%s: window=%d must be >= 0 (0 = full causal)", fn, window);
  if (mode != RBA_BIAS_NONE && mode != RBA_BIAS_TABLE && mode != RBA_BIAS_RPROJ &&
      mode != RBA_BIAS_RPROJ_SHARED)
    return fail(RBA_EINVAL, "%s: unknown bias mode %d", fn, mode);
  if (!std::isfinite(scale)) return fail(RBA_EINVAL, "%s: scale is not finite", fn);
  if (dtype == RBA_BF16 && D != 64 && D != 128)
    return fail(RBA_ENOTSUP, "%s: bf16 supports head_dim 64 or 128, got %d", fn, D);
  if (dtype == RBA_F32 && D != 32 && D != 64 && D != 128)
    return fail(RBA_ENOTSUP, "%s: f32 supports head_dim 32, 64 or 128, got %d", fn, D);
  if (mode != RBA_BIAS_NONE) {
    if (bias_range < 1) return fail(RBA_EINVAL, "%s: bias_range=%d must be >= 1 with a bias", fn, bias_range);
    if (bias_range > kMaxBiasRange)
      return fail(RBA_ENOTSUP, "%s: bias_range=%d exceeds %d", fn, bias_range, kMaxBiasRange);
  }
  if (mode == RBA_BIAS_TABLE) {
    if (!table) return fail(RBA_EINVAL, "%s: table mode needs a table pointer", fn);
    if (!aligned_to(table, 4)) return fail(RBA_EINVAL, "%s: table is not 4-byte aligned", fn);
  }
  if (mode == RBA_BIAS_RPROJ || mode == RBA_BIAS_RPROJ_SHARED) {
    if (R < 1 || R > 16) return fail(RBA_ENOTSUP, "%s: R=%d outside 1..16", fn, R);
    if (!r || !E) return fail(RBA_EINVAL, "%s: rproj mode needs r and E pointers", fn);
    if (!aligned_to(E, 4)) return fail(RBA_EINVAL, "%s: E is not 4-byte aligned", fn);
    if (!aligned_to(r, dtype == RBA_F32 ? 4 : 2)) return fail(RBA_EINVAL, "%s: r is misaligned", fn);
  }
  return RBA_OK;
}

// temp_len: 0 (no context-length temperature) or the visible-key count beyond which it grows.
int check_temp(const char* fn, int temp_len) {
  if (temp_len < 0 || temp_len == 1)
    return fail(RBA_EINVAL, "%s: temp_len=%d must be 0 (no temperature) or >= 2", fn, temp_len);
  return RBA_OK;
}
// Host-side geometry of a paged cache: pool and table sizes, the launch bound max_kv_len, and
// the block table and length pointers (their device values are clamped by the kernel).
int check_paged(const char* fn, int num_pages, int page_size, int max_pages, int max_kv_len,
                const int* block_table, const int* kv_lens) {
  if (page_size < 16 || page_size % 16)
    return fail(RBA_ENOTSUP, "%s: page_size=%d must be a positive multiple of 16", fn, page_size);
  if (num_pages < 1 || max_pages < 1)
    return fail(RBA_EINVAL, "%s: num_pages=%d and max_pages=%d must be >= 1", fn, num_pages, max_pages);
  if (max_kv_len < 1 || static_cast<long long>(max_kv_len) > static_cast<long long>(max_pages) * page_size)
    return fail(RBA_EINVAL, "%s: need 1 <= max_kv_len (%d) <= max_pages * page_size (%lld)", fn,
                max_kv_len, static_cast<long long>(max_pages) * page_size);
  if (static_cast<long long>(num_pages) * page_size >= (1LL << 31))
    return fail(RBA_ENOTSUP, "%s: page pool too large (rows must fit in int32)", fn);
  if (!block_table || !kv_lens) return fail(RBA_EINVAL, "%s: block_table and kv_lens must be non-NULL", fn);
  if (!aligned_to(block_table, 4) || !aligned_to(kv_lens, 4))
    return fail(RBA_EINVAL, "%s: block_table and kv_lens must be 4-byte aligned", fn);
  return RBA_OK;
}

// A caller workspace of `need` bytes (none needed when need is 0).
int check_workspace(const char* fn, size_t need, const void* workspace, size_t workspace_bytes) {
  if (need == 0) return RBA_OK;
  if (!workspace) return fail(RBA_EINVAL, "%s: workspace of %zu bytes required, got NULL", fn, need);
  if (workspace_bytes < need)
    return fail(RBA_EINVAL, "%s: workspace too small (%zu < %zu bytes)", fn, workspace_bytes, need);
  if (!aligned_to(workspace, 4)) return fail(RBA_EINVAL, "%s: workspace is not 4-byte aligned", fn);
  return RBA_OK;
}

float temp_inv_log2(int temp_len) {
  return temp_len > 0 ? static_cast<float>(1.0 / std::log2(static_cast<double>(temp_len))) : 0.f;
}

// The kernels know three bias modes; the shared bank is r.E with a head stride of 0 for E.
int kernel_mode(int mode) { return mode == RBA_BIAS_RPROJ_SHARED ? RBA_BIAS_RPROJ : mode; }
long long e_head_stride(int mode, int R, int bias_range) {
  return mode == RBA_BIAS_RPROJ ? static_cast<long long>(R) * bias_range : 0;
}
bool is_rproj(int mode) { return mode == RBA_BIAS_RPROJ || mode == RBA_BIAS_RPROJ_SHARED; }

// Kernel arguments of a bf16 prefill (the launch geometry is the launcher's).
rba::FwdArgs bf16_fwd_args(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int S, int Hq, int Hkv, int window, int bias_range, int mode,
                           const float* table, const void* r, const float* E, int R, float scale,
                           int temp_len) {
  rba::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.table = table;
  a.r = static_cast<const uint16_t*>(r);
  a.E = E;
  a.B = B;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.window = window;
  a.bias_range = mode == RBA_BIAS_NONE ? 0 : bias_range;
  a.R = is_rproj(mode) ? R : 0;
  a.e_hs = e_head_stride(mode, R, bias_range);
  a.c_qk = scale * rba::kLog2e;
  a.temp_len = temp_len;
  a.temp_inv_log2 = temp_inv_log2(temp_len);
  return a;
}

// Kernel arguments of a bf16 decode over a contiguous cache (L_max > 0) or a paged pool
// (L_max = 0; the caller adds the page table); kv_len is the cache length or the launch bound.
rba::DecodeArgs bf16_decode_args(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const float* table, const void* r, const float* E,
                                 void* workspace, int B, int L_max, int kv_len, int Hq, int Hkv,
                                 int window, int bias_range, int mode, int R, float scale,
                                 int temp_len) {
  rba::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.table = table;
  a.r = static_cast<const uint16_t*>(r);
  a.E = E;
  a.ws = static_cast<float*>(workspace);
  a.B = B;
  a.L_max = L_max;
  a.kv_len = kv_len;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.window = window;
  a.bias_range = mode == RBA_BIAS_NONE ? 0 : bias_range;
  a.R = is_rproj(mode) ? R : 0;
  a.e_hs = e_head_stride(mode, R, bias_range);
  a.key_begin = window ? (kv_len > window ? kv_len - window : 0) : 0;
  rba::decode_split(B, Hkv, kv_len, window, &a.n_split, &a.keys_per_wave);
  a.c_qk = scale * rba::kLog2e;
  a.temp_len = temp_len;
  a.temp_inv_log2 = temp_inv_log2(temp_len);
  return a;
}

// Reads of a paged pool: sequence b's row j is row j % page_size of page block_table[b][j /
// page_size]; lengths and the first visible key come from kv_lens per sequence.
void set_pages(rba::DecodeArgs& a, const int* block_table, const int* kv_lens, int num_pages,
               int page_size, int max_pages) {
  a.key_begin = 0;
  a.block_table = block_table;
  a.kv_lens = kv_lens;
  a.page_size = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
}

// Checks of a decode over MXFP4 caches (contiguous or paged) that do not depend on the layout.
int check_fp4(const char* fn, const void* q, const void* k_codes, const void* k_scales,
              const void* v_codes, const void* v_scales, const void* o, const float* lse, int B,
              int Hq, int Hkv, int D, int window, int bias_range, int mode, const float* table,
              const void* r, const float* E, int R, float scale, int temp_len) {
  if (B < 0) return fail(RBA_EINVAL, "%s: B=%d must be >= 0", fn, B);
  int st = check_common(fn, RBA_BF16, Hq, Hkv, D, window, bias_range, mode, table, r, E, R, scale);
  if (st == RBA_OK) st = check_temp(fn, temp_len);
  if (st != RBA_OK) return st;
  if (D != 64 && D != 128)
    return fail(RBA_ENOTSUP, "%s: MXFP4 caches are supported for head_dim 64 or 128, got %d", fn, D);
  const int G = Hq / Hkv;
  if (G > 32) return fail(RBA_ENOTSUP, "%s: MXFP4 caches support Hq/Hkv <= 32, got %d", fn, G);
  if (B == 0) return RBA_OK;
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !o)
    return fail(RBA_EINVAL, "%s: q, codes, scales and o must be non-NULL", fn);
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(o))
    return fail(RBA_EINVAL, "%s: q, codes and o must be 16-byte aligned", fn);
  if (lse && !aligned_to(lse, 4)) return fail(RBA_EINVAL, "%s: lse is not 4-byte aligned", fn);
  return RBA_OK;
}

// Decode against a contiguous cache.  noalloc: the split partials go to the library's fixed
// per-GPU scratch (relbias_attn_decode_noalloc) instead of the caller's workspace.
int decode_impl(const char* fn, int dtype, const void* q, const void* k_cache, const void* v_cache,
                void* o, float* lse, int B, int L_max, int kv_len, int Hq, int Hkv, int D,
                int window, int bias_range, int mode, const float* table, const void* r,
                const float* E, int R, float scale, int temp_len, void* workspace,
                size_t workspace_bytes, void* stream, bool noalloc) {
  if (B < 0) return fail(RBA_EINVAL, "%s: B=%d must be >= 0", fn, B);
  if (noalloc && dtype != RBA_BF16) return fail(RBA_ENOTSUP, "%s: supported for bf16 only", fn);
  int st = check_common(fn, dtype, Hq, Hkv, D, window, bias_range, mode, table, r, E, R, scale);
  if (st == RBA_OK) st = check_temp(fn, temp_len);
  if (st != RBA_OK) return st;
  if (B == 0) return ok();
  if (L_max < 1 || kv_len < 1 || kv_len > L_max)
    return fail(RBA_EINVAL, "%s: need 1 <= kv_len (%d) <= L_max (%d)", fn, kv_len, L_max);
  if (!q || !k_cache || !v_cache || !o)
    return fail(RBA_EINVAL, "%s: q, k_cache, v_cache and o must be non-NULL", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(RBA_EINVAL, "%s: q, caches and o must be 16-byte aligned", fn);
  if (lse && !aligned_to(lse, 4)) return fail(RBA_EINVAL, "%s: lse is not 4-byte aligned", fn);
  const int G = Hq / Hkv;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == RBA_BF16) {
    if (G > 32) return fail(RBA_ENOTSUP, "%s: bf16 decode supports Hq/Hkv <= 32, got %d", fn, G);
    if (Hkv > 65535 || B > 65535) return fail(RBA_ENOTSUP, "%s: grid too large", fn);
    const size_t need = relbias_attn_decode_workspace_size(B, Hq, Hkv, D, kv_len, window);
    if (noalloc) {
      if (need > static_cast<size_t>(RBA_DECODE_NOALLOC_SCRATCH_BYTES))
        return fail(RBA_ENOTSUP,
                    "%s: these sizes need %zu bytes of split scratch, more than the %d bytes the "
                    "library holds per GPU; use relbias_attn_decode with a caller workspace",
                    fn, need, RBA_DECODE_NOALLOC_SCRATCH_BYTES);
      workspace = nullptr;
      if (need > 0) {
        // the scratch copy of the device the stream runs on, which must be the current one
        int cur = 0, sdev = 0;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && hs != nullptr) e = hipStreamGetDevice(hs, &sdev);
        else sdev = cur;
        if (e != hipSuccess) return fail(RBA_EHIP, "%s: HIP error %s", fn, hipGetErrorString(e));
        if (sdev != cur)
          return fail(RBA_EINVAL, "%s: the stream belongs to device %d but device %d is current", fn,
                      sdev, cur);
        e = rba::decode_noalloc_scratch(&workspace);
        if (e != hipSuccess) return fail(RBA_EHIP, "%s: HIP error %s", fn, hipGetErrorString(e));
      }
    } else {
      st = check_workspace(fn, need, workspace, workspace_bytes);
      if (st != RBA_OK) return st;
    }
    const rba::DecodeArgs a = bf16_decode_args(q, k_cache, v_cache, o, lse, table, r, E, workspace,
                                               B, L_max, kv_len, Hq, Hkv, window, bias_range, mode,
                                               R, scale, temp_len);
    e = rba::launch_decode_bf16(a, D, kernel_mode(mode), hs);
  } else {
    rba::F32Args a{};
    a.q = static_cast<const float*>(q);
    a.k = static_cast<const float*>(k_cache);
    a.v = static_cast<const float*>(v_cache);
    a.o = static_cast<float*>(o);
    a.lse = lse;
    a.table = table;
    a.r = static_cast<const float*>(r);
    a.E = E;
    a.B = B;
    a.Sq = 1;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.D = D;
    a.kv_rows = L_max;
    a.Lk = kv_len;
    a.q_pos0 = kv_len - 1;
    a.window = window;
    a.bias_range = mode == RBA_BIAS_NONE ? 0 : bias_range;
    a.mode = kernel_mode(mode);
    a.R = is_rproj(mode) ? R : 0;
    a.e_hs = e_head_stride(mode, R, bias_range);
    a.scale = scale;
    a.temp_len = temp_len;
    a.temp_inv_log2 = temp_inv_log2(temp_len);
    e = rba::launch_attn_f32(a, hs);
  }
  if (e != hipSuccess) return fail(RBA_EHIP, "%s: HIP error %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* relbias_attn_last_error(void) { return g_err.c_str(); }

const char* relbias_attn_version(void) { return "relbias_attn 0.1 gfx950"; }

size_t relbias_attn_fwd_workspace_size(int dtype, int B, int S, int Hq, int Hkv, int D,
                                       int window, int bias_range, int mode, int R, float scale) {
  if (dtype != RBA_BF16 || B <= 0 || S <= 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || window < 0) return 0;
  if (!(D == 64 || D == 128) || !std::isfinite(scale)) return 0;
  if (mode != RBA_BIAS_NONE && (bias_range < 1 || bias_range > kMaxBiasRange)) return 0;
  if (is_rproj(mode) && (R < 1 || R > 16)) return 0;
  if (mode < RBA_BIAS_NONE || mode > RBA_BIAS_RPROJ_SHARED) return 0;
  const rba::FwdArgs a = bf16_fwd_args(nullptr, nullptr, nullptr, nullptr, nullptr, B, S, Hq, Hkv,
                                       window, bias_range, mode, nullptr, nullptr, nullptr, R, scale, 0);
  return static_cast<size_t>(rba::fwd_bf16_workspace(a, D, kernel_mode(mode)));
}

int relbias_attn_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int S, int Hq, int Hkv, int D, int window, int bias_range, int mode,
                     const float* table, const void* r, const float* E, int R, float scale,
                     int temp_len, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "relbias_attn_fwd";
  if (B < 0 || S < 0) return fail(RBA_EINVAL, "%s: B=%d and S=%d must be >= 0", fn, B, S);
  int st = check_common(fn, dtype, Hq, Hkv, D, window, bias_range, mode, table, r, E, R, scale);
  if (st == RBA_OK) st = check_temp(fn, temp_len);
  if (st != RBA_OK) return st;
  if (B == 0 || S == 0) return ok();
  if (!q || !k || !v || !o) return fail(RBA_EINVAL, "%s: q, k, v and o must be non-NULL", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(RBA_EINVAL, "%s: q, k, v and o must be 16-byte aligned", fn);
  if (lse && !aligned_to(lse, 4)) return fail(RBA_EINVAL, "%s: lse is not 4-byte aligned", fn);
  const long long rows = static_cast<long long>(B) * S;
  if (rows * Hq * D >= (1LL << 40)) return fail(RBA_ENOTSUP, "%s: problem too large", fn);
  if (static_cast<long long>(S) * 1 > (1LL << 30)) return fail(RBA_ENOTSUP, "%s: S too large", fn);

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == RBA_BF16) {
    const int G = Hq / Hkv;
    const int hpw = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
    const long long rows_wg = 32LL * (4 / hpw);
    const long long nblk = ((S + rows_wg - 1) / rows_wg) * (Hq / hpw) * static_cast<long long>(B);
    if (nblk > 0x7fffffffLL) return fail(RBA_ENOTSUP, "%s: grid too large", fn);
    (void)G;
    const rba::FwdArgs a = bf16_fwd_args(q, k, v, o, lse, B, S, Hq, Hkv, window, bias_range, mode,
                                         table, r, E, R, scale, temp_len);
    const long long need = rba::fwd_bf16_workspace(a, D, kernel_mode(mode));
    if (need > 0) {
      if (!workspace) return fail(RBA_EINVAL, "%s: workspace of %lld bytes required, got NULL", fn, need);
      if (workspace_bytes < static_cast<size_t>(need))
        return fail(RBA_EINVAL, "%s: workspace too small (%zu < %lld bytes)", fn, workspace_bytes, need);
      if (!aligned16(workspace)) return fail(RBA_EINVAL, "%s: workspace is not 16-byte aligned", fn);
    }
    e = rba::launch_fwd_bf16(a, D, kernel_mode(mode), workspace, hs);
  } else {
    rba::F32Args a{};
    a.q = static_cast<const float*>(q);
    a.k = static_cast<const float*>(k);
    a.v = static_cast<const float*>(v);
    a.o = static_cast<float*>(o);
    a.lse = lse;
    a.table = table;
    a.r = static_cast<const float*>(r);
    a.E = E;
    a.B = B;
    a.Sq = S;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.D = D;
    a.kv_rows = S;
    a.Lk = S;
    a.q_pos0 = 0;
    a.window = window;
    a.bias_range = mode == RBA_BIAS_NONE ? 0 : bias_range;
    a.mode = kernel_mode(mode);
    a.R = is_rproj(mode) ? R : 0;
    a.e_hs = e_head_stride(mode, R, bias_range);
    a.scale = scale;
    a.temp_len = temp_len;
    a.temp_inv_log2 = temp_inv_log2(temp_len);
    e = rba::launch_attn_f32(a, hs);
  }
  if (e != hipSuccess) return fail(RBA_EHIP, "%s: HIP error %s", fn, hipGetErrorString(e));
  return ok();
}

size_t relbias_attn_decode_workspace_size(int B, int Hq, int Hkv, int D, int kv_len, int window) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || kv_len <= 0 || window < 0) return 0;
  int ns = 1, kpw = 0;
  rba::decode_split(B, Hkv, kv_len, window, &ns, &kpw);
  if (ns <= 1) return 0;
  return static_cast<size_t>(B) * Hq * ns * (D + 2) * sizeof(float);
}

int relbias_attn_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                        void* o, float* lse, int B, int L_max, int kv_len, int Hq, int Hkv, int D,
                        int window, int bias_range, int mode, const float* table, const void* r,
                        const float* E, int R, float scale, int temp_len, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return decode_impl("relbias_attn_decode", dtype, q, k_cache, v_cache, o, lse, B, L_max, kv_len, Hq,
                     Hkv, D, window, bias_range, mode, table, r, E, R, scale, temp_len, workspace,
                     workspace_bytes, stream, false);
}

int relbias_attn_decode_noalloc(int dtype, const void* q, const void* k_cache, const void* v_cache,
                                void* o, float* lse, int B, int L_max, int kv_len, int Hq, int Hkv,
                                int D, int window, int bias_range, int mode, const float* table,
                                const void* r, const float* E, int R, float scale, int temp_len,
                                void* stream) {
  return decode_impl("relbias_attn_decode_noalloc", dtype, q, k_cache, v_cache, o, lse, B, L_max,
                     kv_len, Hq, Hkv, D, window, bias_range, mode, table, r, E, R, scale, temp_len,
                     nullptr, 0, stream, true);
}

size_t relbias_attn_decode_paged_workspace_size(int B, int Hq, int Hkv, int D, int max_kv_len,
                                                int window) {
  return relbias_attn_decode_workspace_size(B, Hq, Hkv, D, max_kv_len, window);
}

int relbias_attn_decode_paged(int dtype, const void* q, const void* k_pages, const void* v_pages,
                              const int* block_table, const int* kv_lens, void* o, float* lse,
                              int B, int num_pages, int page_size, int max_pages, int max_kv_len,
                              int Hq, int Hkv, int D, int window, int bias_range, int mode,
                              const float* table, const void* r, const float* E, int R,
                              float scale, int temp_len, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const char* fn = "relbias_attn_decode_paged";
  if (B < 0) return fail(RBA_EINVAL, "%s: B=%d must be >= 0", fn, B);
  int st = check_common(fn, dtype, Hq, Hkv, D, window, bias_range, mode, table, r, E, R, scale);
  if (st == RBA_OK) st = check_temp(fn, temp_len);
  if (st != RBA_OK) return st;
  if (B == 0) return ok();
  if (dtype != RBA_BF16) return fail(RBA_ENOTSUP, "%s: paged caches are supported for bf16 only", fn);
  st = check_paged(fn, num_pages, page_size, max_pages, max_kv_len, block_table, kv_lens);
  if (st != RBA_OK) return st;
  if (!q || !k_pages || !v_pages || !o)
    return fail(RBA_EINVAL, "%s: q, k_pages, v_pages and o must be non-NULL", fn);
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o))
    return fail(RBA_EINVAL, "%s: q, page pools and o must be 16-byte aligned", fn);
  if (lse && !aligned_to(lse, 4)) return fail(RBA_EINVAL, "%s: lse is not 4-byte aligned", fn);
  const int G = Hq / Hkv;
  if (G > 32) return fail(RBA_ENOTSUP, "%s: bf16 decode supports Hq/Hkv <= 32, got %d", fn, G);
  st = check_workspace(fn, relbias_attn_decode_paged_workspace_size(B, Hq, Hkv, D, max_kv_len, window),
                       workspace, workspace_bytes);
  if (st != RBA_OK) return st;
  if (Hkv > 65535 || B > 65535) return fail(RBA_ENOTSUP, "%s: grid too large", fn);
  rba::DecodeArgs a = bf16_decode_args(q, k_pages, v_pages, o, lse, table, r, E, workspace, B, 0,
                                       max_kv_len, Hq, Hkv, window, bias_range, mode, R, scale,
                                       temp_len);
  set_pages(a, block_table, kv_lens, num_pages, page_size, max_pages);
  hipError_t e = rba::launch_decode_bf16(a, D, kernel_mode(mode), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RBA_EHIP, "%s: HIP error %s", fn, hipGetErrorString(e));
  return ok();
}

int relbias_attn_kv_quantize_fp4(const void* x, void* codes, void* scales, long long rows, int D,
                                 void* stream) {
  const char* fn = "relbias_attn_kv_quantize_fp4";
  if (rows < 0) return fail(RBA_EINVAL, "%s: rows=%lld must be >= 0", fn, rows);
  if (D < 32 || D % 32) return fail(RBA_EINVAL, "%s: D=%d must be a positive multiple of 32", fn, D);
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(RBA_EINVAL, "%s: x, codes and scales must be non-NULL", fn);
  if (!aligned16(x) || !aligned16(codes))
    return fail(RBA_EINVAL, "%s: x and codes must be 16-byte aligned", fn);
  if (rows > (1LL << 40) / D) return fail(RBA_ENOTSUP, "%s: problem too large", fn);
  hipError_t e = rba::launch_quantize_fp4(static_cast<const uint16_t*>(x), static_cast<uint8_t*>(codes),
                                          static_cast<uint8_t*>(scales), rows * (D / 32),
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RBA_EHIP, "%s: HIP error %s", fn, hipGetErrorString(e));
  return ok();
}

int relbias_attn_decode_fp4(const void* q, const void* k_codes, const void* k_scales,
                            const void* v_codes, const void* v_scales, void* o, float* lse, int B,
                            int L_max, int kv_len, int Hq, int Hkv, int D, int window,
                            int bias_range, int mode, const float* table, const void* r,
                            const float* E, int R, float scale, int temp_len, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const char* fn = "relbias_attn_decode_fp4";
  int st = check_fp4(fn, q, k_codes, k_scales, v_codes, v_scales, o, lse, B, Hq, Hkv, D, window,
                     bias_range, mode, table, r, E, R, scale, temp_len);
  if (st != RBA_OK || B == 0) return st == RBA_OK ? ok() : st;
  if (L_max < 1 || kv_len < 1 || kv_len > L_max)
    return fail(RBA_EINVAL, "%s: need 1 <= kv_len (%d) <= L_max (%d)", fn, kv_len, L_max);
  st = check_workspace(fn, relbias_attn_decode_workspace_size(B, Hq, Hkv, D, kv_len, window),
                       workspace, workspace_bytes);
  if (st != RBA_OK) return st;
  if (Hkv > 65535 || B > 65535) return fail(RBA_ENOTSUP, "%s: grid too large", fn);
  rba::DecodeArgs a = bf16_decode_args(q, k_codes, v_codes, o, lse, table, r, E, workspace, B, L_max,
                                       kv_len, Hq, Hkv, window, bias_range, mode, R, scale, temp_len);
  a.k_scale = static_cast<const uint8_t*>(k_scales);
  a.v_scale = static_cast<const uint8_t*>(v_scales);
  hipError_t e = rba::launch_decode_fp4(a, D, kernel_mode(mode), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RBA_EHIP, "%s: HIP error %s", fn, hipGetErrorString(e));
  return ok();
}

int relbias_attn_decode_fp4_paged(const void* q, const void* k_codes, const void* k_scales,
                                  const void* v_codes, const void* v_scales,
                                  const int* block_table, const int* kv_lens, void* o, float* lse,
                                  int B, int num_pages, int page_size, int max_pages,
                                  int max_kv_len, int Hq, int Hkv, int D, int window,
                                  int bias_range, int mode, const float* table, const void* r,
                                  const float* E, int R, float scale, int temp_len,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "relbias_attn_decode_fp4_paged";
  int st = check_fp4(fn, q, k_codes, k_scales, v_codes, v_scales, o, lse, B, Hq, Hkv, D, window,
                     bias_range, mode, table, r, E, R, scale, temp_len);
  if (st != RBA_OK || B == 0) return st == RBA_OK ? ok() : st;
  st = check_paged(fn, num_pages, page_size, max_pages, max_kv_len, block_table, kv_lens);
  if (st != RBA_OK) return st;
  st = check_workspace(fn, relbias_attn_decode_paged_workspace_size(B, Hq, Hkv, D, max_kv_len, window),
                       workspace, workspace_bytes);
  if (st != RBA_OK) return st;
  if (Hkv > 65535 || B > 65535) return fail(RBA_ENOTSUP, "%s: grid too large", fn);
  rba::DecodeArgs a = bf16_decode_args(q, k_codes, v_codes, o, lse, table, r, E, workspace, B, 0,
                                       max_kv_len, Hq, Hkv, window, bias_range, mode, R, scale,
                                       temp_len);
  a.k_scale = static_cast<const uint8_t*>(k_scales);
  a.v_scale = static_cast<const uint8_t*>(v_scales);
  set_pages(a, block_table, kv_lens, num_pages, page_size, max_pages);
  hipError_t e = rba::launch_decode_fp4(a, D, kernel_mode(mode), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RBA_EHIP, "%s: HIP error %s", fn, hipGetErrorString(e));
  return ok();
}

size_t relbias_attn_bwd_workspace_size(int B, int S, int Hq, int mode, int bias_range) {
  if (B <= 0 || S <= 0 || Hq <= 0) return 0;
  const size_t rows = static_cast<size_t>(B) * S * Hq;
  size_t n = (rows * sizeof(float) + 255) / 256 * 256;       // rowsum(dout * o)
  if (is_rproj(mode) && bias_range > 0)                      // E as bf16 high and low parts (R <= 16)
    n += static_cast<size_t>(rba::e2_bytes(mode == RBA_BIAS_RPROJ_SHARED ? 1 : Hq, bias_range, 32));
  return n;
}

int relbias_attn_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     float* dtable, void* dr, float* dE, int B, int S, int Hq, int Hkv, int D,
                     int window, int bias_range, int mode, const float* table, const void* r,
                     const float* E, int R, float scale, int temp_len, void* workspace,
                     size_t workspace_bytes, void* stream) {
  const char* fn = "relbias_attn_bwd";
  if (B < 0 || S < 0) return fail(RBA_EINVAL, "%s: B=%d and S=%d must be >= 0", fn, B, S);
  int st = check_common(fn, dtype, Hq, Hkv, D, window, bias_range, mode, table, r, E, R, scale);
  if (st == RBA_OK) st = check_temp(fn, temp_len);
  if (st != RBA_OK) return st;
  if (B == 0 || S == 0) return ok();
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(RBA_EINVAL, "%s: q, k, v, o, lse, dout, dq, dk and dv must be non-NULL", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(RBA_EINVAL, "%s: q, k, v, o, dout, dq, dk and dv must be 16-byte aligned", fn);
  if (!aligned_to(lse, 4)) return fail(RBA_EINVAL, "%s: lse is not 4-byte aligned", fn);
  if (mode == RBA_BIAS_TABLE && (!dtable || !aligned_to(dtable, 4)))
    return fail(RBA_EINVAL, "%s: table mode needs a 4-byte aligned dtable", fn);
  if (is_rproj(mode) && (!dr || !dE || !aligned_to(dr, dtype == RBA_F32 ? 4 : 2) || !aligned_to(dE, 4)))
    return fail(RBA_EINVAL, "%s: rproj modes need aligned dr and dE", fn);
  const long long rows = static_cast<long long>(B) * S;
  if (rows * Hq * D >= (1LL << 40)) return fail(RBA_ENOTSUP, "%s: problem too large", fn);
  if (dtype == RBA_BF16 && rba::bwd_lds_bytes(D, kernel_mode(mode), bias_range, is_rproj(mode) ? R : 0) < 0)
    return fail(RBA_ENOTSUP, "%s: bias_range=%d needs more LDS than the kernels have", fn, bias_range);
  const size_t need = relbias_attn_bwd_workspace_size(B, S, Hq, mode, bias_range);
  if (!workspace) return fail(RBA_EINVAL, "%s: workspace of %zu bytes required, got NULL", fn, need);
  if (workspace_bytes < need)
    return fail(RBA_EINVAL, "%s: workspace too small (%zu < %zu bytes)", fn, workspace_bytes, need);
  if (!aligned_to(workspace, 16)) return fail(RBA_EINVAL, "%s: workspace is not 16-byte aligned", fn);
  const int G = Hq / Hkv;
  const long long nq = ((S + 31) / 32) * static_cast<long long>(Hq) * B;
  if (nq > 0x7fffffffLL) return fail(RBA_ENOTSUP, "%s: grid too large", fn);
  if (dtype == RBA_F32) {
    rba::BwdF32Args f{};
    f.q = static_cast<const float*>(q);
    f.k = static_cast<const float*>(k);
    f.v = static_cast<const float*>(v);
    f.o = static_cast<const float*>(o);
    f.dout = static_cast<const float*>(dout);
    f.lse = lse;
    f.dq = static_cast<float*>(dq);
    f.dk = static_cast<float*>(dk);
    f.dv = static_cast<float*>(dv);
    f.dr = static_cast<float*>(dr);
    f.dE = dE;
    f.dtable = dtable;
    f.table = table;
    f.r = static_cast<const float*>(r);
    f.E = E;
    f.e_hs = e_head_stride(mode, R, bias_range);
    f.dsum = static_cast<float*>(workspace);
    f.B = B;
    f.S = S;
    f.Hq = Hq;
    f.Hkv = Hkv;
    f.G = G;
    f.D = D;
    f.window = window;
    f.bias_range = mode == RBA_BIAS_NONE ? 0 : bias_range;
    f.mode = kernel_mode(mode);
    f.R = is_rproj(mode) ? R : 0;
    f.scale = scale;
    f.temp_len = temp_len;
    f.temp_inv_log2 = temp_inv_log2(temp_len);
    hipError_t e = rba::launch_bwd_f32(f, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(RBA_EHIP, "%s: HIP error %s", fn, hipGetErrorString(e));
    return ok();
  }
  rba::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.dr = static_cast<uint16_t*>(dr);
  a.dE = dE;
  a.dtable = dtable;
  a.table = table;
  a.r = static_cast<const uint16_t*>(r);
  a.E = E;
  a.e_hs = e_head_stride(mode, R, bias_range);
  a.dsum = static_cast<float*>(workspace);
  a.e2 = is_rproj(mode)
      ? reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(workspace) +
                                    (static_cast<size_t>(B) * S * Hq * sizeof(float) + 255) / 256 * 256)
      : nullptr;
  a.B = B;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.window = window;
  a.bias_range = mode == RBA_BIAS_NONE ? 0 : bias_range;
  a.R = is_rproj(mode) ? R : 0;
  a.c_qk = scale * rba::kLog2e;
  a.scale = scale;
  a.temp_len = temp_len;
  a.temp_inv_log2 = temp_inv_log2(temp_len);
  hipError_t e = rba::launch_bwd_bf16(a, D, kernel_mode(mode), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RBA_EHIP, "%s: HIP error %s", fn, hipGetErrorString(e));
  return ok();
}

}  // extern "C"
