// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Not installed; the public interface is include/relbias_attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

namespace rba {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// E converted for the MFMA curve blocks (split prefill and backward): distance-major rows of a
// bf16 high and low part of E * inv_scale, [heads][bias_range + 2 kE2Pad + 1][e2_width(R)],
// zero at the kE2Pad padding distances on each side (and one more row), zero past feature R.
constexpr int kE2Pad = 64;
inline int e2_width(int R) { return R > 8 ? 32 : 16; }
inline long long e2_bytes(int heads, int bias_range, int width) {
  return static_cast<long long>(heads) * (bias_range + 2 * kE2Pad + 1) * width * 2;
}

// Context-length temperature of a query that sees n keys: 1 while n <= temp_len, then
// log(n) / log(temp_len), a factor on both the q.k term and the bias ("Thinking Machines
// dropped RoPE", section "The temperature scale is dependent on context length": flat up to
// 128k visible keys, logarithmic growth beyond).  temp_len == 0: no temperature.
// inv_log2_len = 1 / log2(temp_len).
__host__ __device__ inline float temp_factor(int n, int temp_len, float inv_log2_len) {
#ifdef __HIP_DEVICE_COMPILE__
  return (temp_len > 0 && n > temp_len) ? __builtin_amdgcn_logf(static_cast<float>(n)) * inv_log2_len : 1.f;
#else
  return (temp_len > 0 && n > temp_len) ? static_cast<float>(std::log2(static_cast<double>(n))) * inv_log2_len : 1.f;
#endif
}

// Keys a query at position `pos` sees when keys 0..pos exist (window 0: all of them).
__host__ __device__ inline int visible_keys(int pos, int window) {
  return window ? (pos + 1 < window ? pos + 1 : window) : pos + 1;
}

// Prefill arguments (bf16 MFMA path).  Strides are implied by the dense shapes
// q/o [B,S,Hq,D], k/v [B,S,Hkv,D], r [B,S,Hq,R], lse [B,Hq,S].
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const float* table;   // [Hq, bias_range]
  const uint16_t* r;    // [B, S, Hq, R]
  const float* E;       // [Hq, R, bias_range], head h at E + h * e_hs
  long long e_hs;       // head stride of E in floats (R * bias_range, or 0 for one shared bank)
  int B, S, Hq, Hkv, G;
  int window;           // 0 = full causal
  int bias_range;
  int R;
  int hpw;              // query heads per workgroup (they share one kv head)
  int rows_wg;          // query rows per workgroup
  int n_qtiles;         // ceil(S / rows_wg)
  int n_hgroups;        // Hq / hpw
  int longest_first;    // schedule query tiles with the most keys first
  float c_qk;           // scale * log2(e)
  int temp_len;         // context-length temperature threshold (0: none)
  float temp_inv_log2;  // 1 / log2(temp_len)
};

// Generic fp32 attention (VALU): queries at positions q_pos0 + i, keys at
// positions 0..Lk-1 read from rows of a [B, kv_rows, Hkv, D] buffer.
struct F32Args {
  const float* q;       // [B, Sq, Hq, D]
  const float* k;       // [B, kv_rows, Hkv, D]
  const float* v;
  float* o;             // [B, Sq, Hq, D]
  float* lse;           // [B, Hq, Sq] or null
  const float* table;
  const float* r;       // [B, Sq, Hq, R]
  const float* E;
  long long e_hs;       // head stride of E in floats (0: one bank for all heads)
  int B, Sq, Hq, Hkv, G, D;
  int kv_rows;          // row count of the k/v buffers per batch entry (L_max or S)
  int Lk;               // keys 0..Lk-1 exist
  int q_pos0;           // position of query 0
  int window, bias_range, mode, R;
  float scale;
  int temp_len;         // context-length temperature threshold (0: none)
  float temp_inv_log2;  // 1 / log2(temp_len)
};

// Decode arguments (bf16 MFMA path).
struct DecodeArgs {
  const uint16_t* q;    // [B, Hq, D]
  const uint16_t* k;    // [B, L_max, Hkv, D]
  const uint16_t* v;
  uint16_t* o;          // [B, Hq, D]
  float* lse;           // [B, Hq] or null
  const float* table;
  const uint16_t* r;    // [B, Hq, R]
  const float* E;
  long long e_hs;       // head stride of E in floats (0: one bank for all heads)
  float* ws;            // partials [B, Hq, n_part, D + 2] (unnormalised acc, m, l) or null
  int B, L_max, kv_len, Hq, Hkv, G;
  int window, bias_range, R;
  int key_begin;        // first visible key (kv_len - window, clamped at 0); per sequence when paged
  // paged cache: k/v are page pools [num_pages, page_size, Hkv, D]; row j of sequence b lives
  // in page block_table[b * max_pages + j / page_size] at slot j % page_size; the cache length
  // of sequence b is kv_lens[b] (kv_len is then the upper bound the split was sized for)
  const uint8_t* k_scale;   // MXFP4 caches: E8M0 scales [B, L_max, Hkv, D / 32] (k / v then
  const uint8_t* v_scale;   // hold the packed codes [B, L_max, Hkv, D / 2]); null for bf16
  const int* block_table;   // null: contiguous caches [B, L_max, Hkv, D]
  const int* kv_lens;
  int page_size, max_pages, num_pages;
  int n_split;          // workgroups per (b, kv head); each has 4 waves
  int keys_per_wave;    // multiple of 64
  float c_qk;
  int temp_len;         // context-length temperature threshold (0: none)
  float temp_inv_log2;  // 1 / log2(temp_len)
};

// Backward arguments (bf16 MFMA path).  Shapes as in FwdArgs; dq like q, dk / dv like k / v,
// dr like r (bf16), dE like E and dtable like table (fp32, accumulated; zeroed by the pre pass).
struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;     // [B, Hq, S] natural-log sum-exp of the forward
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dr;         // [B, S, Hq, R]
  float* dE;            // head h at dE + h * e_hs
  float* dtable;        // [Hq, bias_range]
  const float* table;
  const uint16_t* r;
  const float* E;
  long long e_hs;       // head stride of E and dE in floats (0: one shared bank)
  float* dsum;          // workspace [B, Hq, S]: rowsum(dout * o)
  uint16_t* e2;         // workspace (r.E): E in the curve-block format (kE2Pad, e2_width(R)), scale 1
  int B, S, Hq, Hkv, G;
  int window, bias_range, R;
  float c_qk;           // scale * log2(e)
  float scale;
  int temp_len;
  float temp_inv_log2;
};

// Backward arguments (fp32 vector-ALU path): the tensors of BwdArgs in fp32 (dr like r).
struct BwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* dout;
  const float* lse;     // [B, Hq, S] natural-log sum-exp of the forward
  float* dq;
  float* dk;
  float* dv;
  float* dr;            // [B, S, Hq, R]
  float* dE;            // head h at dE + h * e_hs
  float* dtable;        // [Hq, bias_range]
  const float* table;
  const float* r;
  const float* E;
  long long e_hs;       // head stride of E and dE in floats (0: one shared bank)
  float* dsum;          // workspace [B, Hq, S]: rowsum(dout * o)
  int B, S, Hq, Hkv, G, D;
  int window, bias_range, mode, R;
  float scale;
  int temp_len;
  float temp_inv_log2;
};

// Raise a kernel's dynamic-LDS limit to `bytes` (no-op up to 64 KB) on the device of stream s,
// once per (kernel, device); thread-safe.
hipError_t set_max_lds(const void* fn, int bytes, hipStream_t s);

hipError_t launch_fwd_bf16(const FwdArgs& a, int D, int mode, void* workspace, hipStream_t s);
// Workspace bytes the bf16 prefill of this shape takes (0: none); the size query and the launch
// share it, so both pick the same kernel.
long long fwd_bf16_workspace(const FwdArgs& a, int D, int mode);
// Split prefill (two workgroups per CU): workspace bytes it needs (the converted E of r.E bias),
// or -1 outside its domain; and its launcher.
long long fwd_split_workspace(int D, int G, int mode, int bias_range, int R, int e_shared, int Hq, float scale);
hipError_t launch_fwd_bf16_split(const FwdArgs& a, int mode, void* workspace, hipStream_t s);
// The conversion of E into that format (heads rows of E at head stride e_hs).
hipError_t launch_e2_convert(const float* E, long long e_hs, int R, int bias_range, float inv_scale, int heads,
                             uint16_t* e2, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, int D, int mode, hipStream_t s);
// fp32 backward (D = 32, 64 or 128; mode 0 none, 1 table, 2 r.E)
hipError_t launch_bwd_f32(const BwdF32Args& a, hipStream_t s);
// LDS bytes of the largest backward kernel for this shape, or -1 when it does not fit.
int bwd_lds_bytes(int D, int mode, int bias_range, int R);
hipError_t launch_attn_f32(const F32Args& a, hipStream_t s);
hipError_t launch_decode_bf16(DecodeArgs a, int D, int mode, hipStream_t s);
// Decode over MXFP4 caches (D = 64 or 128, G <= 32) and the MXFP4 quantiser of bf16 rows
// (nblk blocks of 32 elements: 16 code bytes and one scale byte each).
hipError_t launch_decode_fp4(DecodeArgs a, int D, int mode, hipStream_t s);
hipError_t launch_quantize_fp4(const uint16_t* x, uint8_t* codes, uint8_t* scales, long long nblk, hipStream_t s);

// Device address of the allocation-free decode's fixed scratch (RBA_DECODE_NOALLOC_SCRATCH_BYTES)
// on the current device.
hipError_t decode_noalloc_scratch(void** ptr);

// Decode split policy, shared by the workspace-size query and the launcher.
void decode_split(int B, int Hkv, int kv_len, int window, int* n_split, int* keys_per_wave);

}  // namespace rba
