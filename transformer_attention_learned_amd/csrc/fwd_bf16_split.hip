// Prefill for head_dim 128 and GQA groups of 4k query heads, two workgroups per CU (gfx950).
//
// Same operation as the other prefill kernels (scaled q.k plus a bias read at the distance
// i - j, zero at and beyond the range, causal / sliding window; "Thinking Machines dropped
// RoPE", steps 3-5 and the kernel-cost section), organised so that two workgroups share a CU:
//
//   * workgroup = 4 waves = the 4 query heads of one GQA group over the same 32 query rows,
//     one wave per SIMD; a second workgroup on the CU supplies the other wave of each SIMD, so
//     one workgroup's barriers and start-up overlap the other's key loop;
//   * K/V tiles of 32 keys (one key step) in a ring of three LDS buffers: the tile of step j + 2
//     is loaded while steps j (P.V) and j + 1 (scores) read theirs, so one barrier per step
//     covers both hazards; the loads go straight from memory into LDS (16 bytes per lane, no
//     registers, no stores), K and V row-major with the 16-byte chunks of a row XOR-swizzled so
//     that the fragment reads are conflict-free; V^T fragments come from row-major V with the
//     LDS transpose read (ds_read_b64_tr_b16);
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: each lane owns one query row,
//     P stays in registers; the key loop is a two-stage software pipeline (S MFMAs of step j + 1
//     beside the exp of step j, P.V MFMAs of step j beside the row max of step j + 1), unrolled
//     by three so that every iteration's ring buffer is a compile-time constant (fragment reads
//     are a per-lane register offset plus an immediate); per-step flags (edge, band) are
//     compares against thresholds computed once per workgroup;
//   * bias and masks enter through the S accumulator's start values; lazy rescaling of O;
//   * table bias: the group's table rows in LDS, zero-padded, read with immediate offsets;
//   * input-dependent bias r_i . E[h, :, delta]: E in accumulator units split into a bf16 high
//     and low part (about 16 mantissa bits), distance-major rows of EW = 16 or 32 entries
//     (converted once per call into the caller's workspace), so that a curve block's operand is
//     one 16-byte load per lane and MFMA; the high and low parts of R <= 8 features share one
//     MFMA (they fill its two K halves).  The curves of a step (MFMAs over the features for its
//     64 distances, fp32) go through the wave's LDS curve buffer in fp32 and are formed one step
//     ahead of their use, their E rows one step before that; with the window inside the range
//     every step is in band and this path has no branches.

#include <algorithm>
#include <type_traits>

#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

constexpr int D = 128;
constexpr int BN = 32;            // keys per tile (= per step)
constexpr int NC = D / 16;        // K = 16 chunks of the head dim
constexpr int NDB = D / 32;       // 32-wide head-dim blocks of O^T
constexpr int NBUF = 3;           // tile ring
constexpr int PAD = kE2Pad;       // zero distances on each side of the bias range (table rows, E rows)
constexpr int ROWS_WG = 32;       // query rows per workgroup
constexpr int NT = 256;           // threads per workgroup
constexpr float kRescale = 8.f;   // lazy rescale threshold (log2 units)

constexpr int KT_BYTES = BN * D * 2;   // K tile: 32 rows of 256 bytes
constexpr int VT_BYTES = BN * D * 2;   // V tile: 32 rows of 256 bytes
constexpr int BUF_BYTES = KT_BYTES + VT_BYTES;
constexpr int CURVE_FLOATS = 32 * 36;   // per wave: 32 skewed fp32 rows of 36 entries
constexpr int CURVE_BYTES = CURVE_FLOATS * 4;
constexpr int TILE_BYTES = NBUF * BUF_BYTES;
static_assert(4 * ROWS_WG * D * 2 <= TILE_BYTES, "the epilogue stages the four waves' rows in the ring");

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) float lds_float;

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at dst + 16 l
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, 0, 0, 0);
}
// LDS transpose read: within each group of 16 lanes, lane i receives 16-bit element i % 4 of the
// 8-byte pieces addressed by lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4
__device__ __forceinline__ u32x2 tr_read(const void* p) {
  const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(u32x2, x);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// E (fp32 [heads, R, Rb], head h at E + h * e_hs) -> bf16 rows [heads][Rb + 2 PAD + 1][EW] of a
// high and a low part: with x = E[h, f, d] / scale in fp32, entry (h, PAD + d, f) = bf16(x) and
// entry (h, PAD + d, EW / 2 + f) = bf16(x - bf16(x)) for 0 <= d < Rb and f < R, zero elsewhere
// (the pads and the features past R), so that every read of the kernels below is in range and
// unguarded and the pair carries about 16 mantissa bits of x.  One thread per (head, row) and 8
// features: two 16-byte stores; grid.y = head, grid.z = feature octet (EW / 16 of them).
__global__ void e2_convert_kernel(const float* __restrict__ E, long long e_hs, int R, int Rb,
                                  float inv_scale, int EW, uint16_t* __restrict__ e2) {
  const int rows = Rb + 2 * PAD + 1;
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= rows) return;
  const int h = blockIdx.y;
  const int f0 = 8 * blockIdx.z;
  const int d = p - PAD;
  const bool live = d >= 0 && d < Rb;
  // all 8 loads issued unconditionally (distance and feature clamped into range) and masked
  // afterwards as integers, so that none waits behind its own branch
  const float* eh = E + h * e_hs + min(max(d, 0), Rb - 1);
  uint32_t raw[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) raw[q] = __float_as_uint(eh[static_cast<long long>(min(f0 + q, R - 1)) * Rb]);
  uint32_t whi[4], wlo[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint16_t hb[2], lb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int f = f0 + 2 * k + u;
      const uint32_t keep = (live && f < R) ? ~0u : 0u;
      const float x = __uint_as_float(__float_as_uint(__uint_as_float(raw[2 * k + u]) * inv_scale) & keep);
      hb[u] = f32_to_bf16(x);
      lb[u] = f32_to_bf16(x - bf16_to_f32(hb[u]));
    }
    whi[k] = static_cast<uint32_t>(hb[0]) | (static_cast<uint32_t>(hb[1]) << 16);
    wlo[k] = static_cast<uint32_t>(lb[0]) | (static_cast<uint32_t>(lb[1]) << 16);
  }
  uint16_t* row = e2 + (static_cast<size_t>(h) * rows + p) * EW;
  st16(row + f0, u32x4{whi[0], whi[1], whi[2], whi[3]});
  st16(row + EW / 2 + f0, u32x4{wlo[0], wlo[1], wlo[2], wlo[3]});
}

// MODE 0 none, 1 table, 2 r.E (EW = 16 or 32 entries per E row: the high and low parts of up
// to 8 or 16 features); ALLBAND: every visible key is inside the bias range (window <= range),
// so every step of MODE 2 is in band.
template <int MODE, int EW, bool ALLBAND>
__global__ __launch_bounds__(NT, 2) void fwd_split_kernel(FwdArgs a, const uint16_t* __restrict__ e2g) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: geometry stays scalar
  const int ln = lane & 31;
  const int lh = lane >> 5;

  const int per_q = a.n_hgroups * a.B;
  int qt = blockIdx.x / per_q;
  const int rem = blockIdx.x - qt * per_q;
  const int hg = rem % a.n_hgroups;
  const int b = rem / a.n_hgroups;
  if (a.longest_first) qt = a.n_qtiles - 1 - qt;

  const int S = a.S;
  const int W = a.window;
  const int Rb = a.bias_range;
  const int i0 = qt * ROWS_WG;                 // first query row (all four waves)
  const int h = hg * 4 + wave;
  const int hkv = h / a.G;
  const int row_last = min(S, i0 + ROWS_WG) - 1;
  const int kmin = W ? max(0, i0 - W + 1) : 0;
  const int t_begin = kmin / BN;
  const int nsteps = row_last / BN - t_begin + 1;

  const float cqk = a.c_qk;              // scale * log2(e)
  const float inv_scale = kLog2e / cqk;  // bias -> accumulator units (bias / scale)
  // scale * log2(e) times the row's context-length temperature, which multiplies the q.k term
  // and the bias alike (both sit in the accumulator)
  const float cqk_r = cqk * temp_factor(visible_keys(i0 + ln, W), a.temp_len, a.temp_inv_log2);

  const size_t q_row = static_cast<size_t>(a.Hq) * D;
  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const uint16_t* kbase = a.k + static_cast<size_t>(b) * S * kv_row + static_cast<size_t>(hkv) * D;
  const uint16_t* vbase = a.v + static_cast<size_t>(b) * S * kv_row + static_cast<size_t>(hkv) * D;

  // ---- K/V tiles, 32 keys x 128 dims each, loaded straight into LDS: one load moves 1 KB (4 rows
  // of 256 bytes); wave w loads the K and the V row blocks 2w and 2w + 1.  The 16-byte chunk c of
  // row r sits at slot c ^ (r % 16) of the row in the K tile and at slot c ^ 4 (r % 4) in the V
  // tile, so that the fragment reads below hit distinct banks.  Rows at or past S read as zeros
  // through the buffer range (rows - r0) * row bytes - head offset, which every in-range chunk
  // fits below.
  const int kv_row_b = a.Hkv * D * 2;
  const int head_b = hkv * D * 2;
  int kvo[2], vvo[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 4 * (2 * wave + q) + (lane >> 4);
    const int sl = lane & 15;
    kvo[q] = r * kv_row_b + 16 * (sl ^ (r & 15));
    vvo[q] = r * kv_row_b + 16 * (sl ^ (4 * (r & 3)));
  }
  auto dma_tile = [&](int t, unsigned char* buf) {   // tile t of the step sequence
    const int tk0 = (t_begin + t) * BN;
    const int left = S - tk0;
    const int nrec = left > 0 ? left * kv_row_b - head_b : 0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + static_cast<size_t>(tk0) * kv_row, nrec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + static_cast<size_t>(tk0) * kv_row, nrec);
    unsigned char* kdst = buf + 2 * wave * 1024;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      dma16(rk, kdst + q * 1024, kvo[q]);
      dma16(rv, kdst + KT_BYTES + q * 1024, vvo[q]);
    }
  };
  // this wave's loads into LDS have landed (they are its only vector-memory writes to LDS; the
  // barrier that follows publishes them)
  auto dma_wait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)
  // the same inside the key loop when the only loads issued after the awaited tile are the
  // 2 NEF E-row loads of a later step: vector-memory loads complete in issue order, so
  // vmcnt(2 NEF) leaves those in flight instead of waiting out their latency before the barrier
  auto dma_wait_but_e = [&]() {
    if (EW == 32) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0F72);            // vmcnt(2)
  };

  // tiles 0 and 1 in flight first (HBM), then the query rows
  dma_tile(0, smem);
  if (nsteps > 1) dma_tile(1, smem + BUF_BYTES);
  // ---- table rows of the group (MODE 1), in accumulator units, PAD zero distances each side
  // (requested behind the first two tiles, whose latency their first wait then overlaps)
  const int Rp = Rb + 2 * PAD;
  if (MODE == 1) {
    float* tab = reinterpret_cast<float*>(smem + TILE_BYTES);
    const float* tg = a.table + static_cast<size_t>(hg) * 4 * Rb;
    auto dist = [&](int i, int& hw) {
      hw = static_cast<int>(i >= Rp) + static_cast<int>(i >= 2 * Rp) + static_cast<int>(i >= 3 * Rp);
      return i - hw * Rp - PAD;
    };
    stage_batched(tid, NT, 4 * Rp,
        [&](int i) {
          int hw;
          const int d = dist(i, hw);
          return __float_as_uint(tg[hw * Rb + min(max(d, 0), Rb - 1)]);
        },
        [&](int i, uint32_t w) {
          int hw;
          const int d = dist(i, hw);
          const uint32_t keep = (d >= 0 && d < Rb) ? ~0u : 0u;
          tab[i] = __uint_as_float(__float_as_uint(__uint_as_float(w) * inv_scale) & keep);
        });
  }


  bf16x8 qf[NC];
  {
    const int row = i0 + ln;
    const uint16_t* qp = a.q + (static_cast<size_t>(b) * S + row) * q_row + static_cast<size_t>(h) * D + 8 * lh;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < S) v = ld16(qp + 16 * c);
      qf[c] = as_bf16x8(v);
    }
  }
  // r fragment (B operand of the curve MFMAs): with EW = 16 both lane halves hold features 0..7
  // (they meet the high and the low part of E), with EW = 32 lane half lh holds features 8 lh ..
  // 8 lh + 7 (the high and the low part take one MFMA each)
  bf16x8 rf;
  const uint16_t* e2h = nullptr;   // this head's E rows at distance 0
  if (MODE == 2) {
    const int row = i0 + ln;
    const uint16_t* rp = a.r + ((static_cast<size_t>(b) * S + row) * a.Hq + h) * a.R;
    const int f0 = (EW == 32) ? 8 * lh : 0;
    const bool live = row < S;
    if (a.R == EW / 2 && (reinterpret_cast<uintptr_t>(a.r) & 15) == 0) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (live) v = ld16(rp + f0);
      rf = as_bf16x8(v);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int f = f0 + 2 * jj;
        const uint32_t lo = (live && f < a.R) ? rp[f] : 0u;
        const uint32_t hi = (live && f + 1 < a.R) ? rp[f + 1] : 0u;
        w[jj] = lo | (hi << 16);
      }
      rf = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
    }
    e2h = e2g + (static_cast<size_t>(a.e_hs ? h : 0) * (Rp + 1) + PAD) * EW;
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  const float NEG_INF = -INFINITY;
  const float* tabw = (MODE == 1) ? reinterpret_cast<const float*>(smem + TILE_BYTES) + wave * Rp + PAD : nullptr;
  float* cbuf = (MODE == 2) ? reinterpret_cast<float*>(smem + TILE_BYTES) + wave * CURVE_FLOATS : nullptr;

  // Step js covers keys j0 .. j0 + 31 with j0 = (t_begin + js) * BN; delta = c + n - m with
  // c = i0 - j0, n the lane's row, m the key within the step.  For js >= 0 the step has visible
  // keys exactly when js < nsteps; it crosses the diagonal only as the last step (c = 0), the
  // window's far edge only among the first js_w steps (c + 31 >= W), and it is in band from
  // step js_band on (c - 31 < Rb).  The thresholds are computed once, so that the per-step
  // flags are single compares.
  auto step_c = [&](int js) { return i0 - (t_begin + js) * BN; };
  const int c_first = i0 - t_begin * BN;
  const int js_w = (W && c_first + 31 >= W) ? (c_first + 31 - W) / BN + 1 : 0;
  const int js_band = (c_first - 31 < Rb) ? 0 : (c_first - 31 - Rb) / BN + 1;
  auto step_on = [&](int js) { return js < nsteps; };
  auto step_inband = [&](int js) { return MODE != 0 && js < nsteps && js >= js_band; };
  auto step_edge = [&](int js) { return js >= nsteps - 1 || js < js_w; };

  // ---- r.E curves: E rows of step js are loaded one step before its curves are formed
  constexpr int NEF = EW / 16;   // curve MFMAs per 32 distances (high and low part of E)
  u32x4 ef[2][NEF];              // [distance block][MFMA]
#pragma unroll
  for (int u = 0; u < 2 * NEF; ++u) ef[u / NEF][u % NEF] = u32x4{0u, 0u, 0u, 0u};
  float cr[16];                  // the bias of this lane's 16 keys of the step, accumulator units
#pragma unroll
  for (int i = 0; i < 16; ++i) cr[i] = 0.f;
  auto curve_c = [&](int js) {
    // a step outside the band is fully masked (ALLBAND) or skipped: clamp its offset so that
    // the E rows read stay inside the padded rows (distances -PAD .. Rb + PAD)
    return min(max(step_c(js), -33), Rb + 31);
  };
  auto e_fetch_to = [&](int js, u32x4 (&e)[2][NEF]) {
    // A operand: E row of distance c - 31 + ln (block 0) or c + 1 + ln (block 1); MFMA u takes
    // entries 16 u + 8 lh .. + 7 of the row
    const uint16_t* ep = e2h + (curve_c(js) - 31 + ln) * EW + 8 * lh;
#pragma unroll
    for (int u = 0; u < NEF; ++u) {
      e[0][u] = ld16(ep + 16 * u);
      e[1][u] = ld16(ep + 32 * EW + 16 * u);
    }
  };
  auto e_fetch = [&](int js) { e_fetch_to(js, ef); };
  // curves of step js from the fetched E rows: MFMAs over the features give the 64 distances
  // c - 31 .. c + 32 for every query row, in fp32 (curve_mfma): lane (n, lh) holds row n at
  // t = 8 g + 4 lh + k (block 0) and 32 + the same (block 1), t = distance - (c - 31).
  // curve_store writes them to the wave's buffer and reads back the lane's diagonal
  // t = 31 + n - m for its keys m = 8 g + 4 lh + k.  Row n keeps only the t it reads,
  // n .. n + 31, as entries t - 4 (n / 4) in 0..35 of a 36-entry row.  With n = 4 j + e the row
  // sits in slot ((3 j + sigma(e)) % 8) + 8 e, sigma = (0, 1, 4, 5): then the dword reads of
  // each half-wave (32 lanes) hit 32 distinct banks and the 16-byte writes of each group of 8
  // lanes 8 distinct 4-bank groups (the LDS serves dword reads as 32 banks, half a wave per
  // clock).  Chunks a row does not read are not written (a per-lane constant predicate).
  const int cj = ln >> 2, ce = ln & 3;
  const int cslot = ((3 * cj + (ce & 1) + 4 * (ce >> 1)) & 7) + 8 * ce;
  const int cbase = 36 * cslot - 4 * cj;
  bool cwrite[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int ts = 32 * (u >> 2) + 8 * (u & 3) + 4 * lh;
    cwrite[u] = ts + 3 >= ln && ts <= ln + 31;
  }
  const lds_float* crd = nullptr;
  if (MODE == 2) {
    crd = (const lds_float*)(cbuf + cbase + 4 + ln - 4 * lh);
    // an opaque register: the reads below then use it as their base with immediate offsets,
    // instead of one address computation each (the LDS offset of the buffer is too large for
    // the pair-read offset field)
    asm volatile("" : "+v"(crd));
  }
  auto curve_mfma = [&](f32x16& lo, f32x16& hi) {
    const f32x16 zero = {};
    lo = mfma32(as_bf16x8(ef[0][0]), rf, zero);
    hi = mfma32(as_bf16x8(ef[1][0]), rf, zero);
#pragma unroll
    for (int u = 1; u < NEF; ++u) {
      lo = mfma32(as_bf16x8(ef[0][u]), rf, lo);
      hi = mfma32(as_bf16x8(ef[1][u]), rf, hi);
    }
  };
  auto curve_store = [&](const f32x16& lo, const f32x16& hi) {
    float* wp = cbuf + cbase + 4 * lh;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (__builtin_expect(cwrite[g], 1)) st16(wp + 8 * g, __builtin_bit_cast(u32x4, f32x4{lo[4 * g], lo[4 * g + 1], lo[4 * g + 2], lo[4 * g + 3]}));
      if (__builtin_expect(cwrite[4 + g], 1)) st16(wp + 32 + 8 * g, __builtin_bit_cast(u32x4, f32x4{hi[4 * g], hi[4 * g + 1], hi[4 * g + 2], hi[4 * g + 3]}));
    }
    wave_sync_lds();
    // key m = 8 g + 4 lh + k at entry cbase + 31 + n - m (crd: entry cbase + 4 + n - 4 lh, so
    // that the 16 reads are one base register and dword offsets 0..27, paired into ds_read2_b32)
#pragma unroll
    for (int i = 0; i < 16; ++i) cr[i] = crd[27 - 8 * (i >> 2) - (i & 3)];
  };
  auto curve_issue = [&](int js) {
    f32x16 lo, hi;
    curve_mfma(lo, hi);
    curve_store(lo, hi);
  };
  // the curve work of step js (when it has any), and the E rows of step js + 1
  auto curve_step = [&](int js) {
    if (MODE != 2) return;
    if (ALLBAND) {
      curve_issue(js);
      e_fetch(js + 1);
    } else {
      if (step_inband(js)) curve_issue(js);
      if (step_inband(js + 1)) e_fetch(js + 1);
    }
  };

  // Whether step js starts from something other than zero; uniform across the wave.
  auto step_special = [&](int js) -> bool {
    if (MODE == 2 && ALLBAND) return true;
    return step_edge(js) || step_inband(js);
  };
  // Accumulator start values: bias / scale where the key is visible and in band, 0 where
  // visible and beyond the band, -inf elsewhere.
  auto step_init = [&](int js) -> f32x16 {
    f32x16 init;
#pragma unroll
    for (int i = 0; i < 16; ++i) init[i] = 0.f;
    const int c = step_c(js);
    const bool on = step_on(js);
    const bool inband = step_inband(js);
    if (MODE == 1 && inband) {
      asm volatile("; in-band step: table bias" ::: "memory");
      const float* tb = tabw + (c + ln - 4 * lh - 27);
#pragma unroll
      for (int i = 0; i < 16; ++i) init[i] = tb[27 - 8 * (i >> 2) - (i & 3)];
    }
    if (MODE == 2 && (ALLBAND || inband)) {
      asm volatile("; in-band step: r.E bias" ::: "memory");
#pragma unroll
      for (int i = 0; i < 16; ++i) init[i] = cr[i];
    }
    if (step_edge(js)) {
      asm volatile("; edge step: mask" ::: "memory");
      // visible iff 0 <= d < W (d >= 0 without a window): one unsigned compare per element
      const int dbase = c + ln - 4 * lh;
      const unsigned lim = !on ? 0u : (W ? static_cast<unsigned>(W) : 0x80000000u);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = dbase - (8 * (i >> 2) + (i & 3));
        if (static_cast<unsigned>(d) >= lim) init[i] = NEG_INF;
      }
    }
    return init;
  };

  // K fragment of chunk c (dims 16 c + 8 lh .. + 7 of key ln): slot (2 c + lh) ^ (ln % 16)
  int kaddr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) kaddr[c] = ln * 256 + 16 * ((2 * c + lh) ^ (ln & 15));
  // V^T fragment (dims 32 db + ln, keys of slot e = 16 kk + 4 lh + e % 4 + 8 (e / 4), the P
  // layout): two transpose reads of 4 keys each; lane t = 4 j + q of a 16-lane group addresses
  // key row 16 kk + 4 lh + j (+ 8), dims 32 db + 16 gq + 4 q .. + 3, i.e. half q % 2 of chunk
  // 4 db + 2 gq + q / 2, whose slot is that chunk ^ 4 j (row % 4 = j)
  int vaddr[NDB];
  {
    const int t16 = lane & 15, j = t16 >> 2, q = t16 & 3, gq = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vaddr[db] = (4 * lh + j) * 256 + 16 * ((4 * db + 2 * gq + (q >> 1)) ^ (4 * j)) + 8 * (q & 1);
  }
  // (buf: the tile's LDS buffer)
  auto k_frag = [&](const unsigned char* buf, int c) -> bf16x8 { return as_bf16x8(ld16(buf + kaddr[c])); };
  auto v_frag = [&](const unsigned char* buf, int idx) -> bf16x8 {   // idx = 2 * db + kk
    const unsigned char* vb = buf + KT_BYTES + vaddr[idx >> 1] + 16 * (idx & 1) * 256;
    const u32x2 lo = tr_read(vb), hi = tr_read(vb + 8 * 256);
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
  auto step_scores = [&](const unsigned char* buf, f32x16& acc, auto spec_c) {
    constexpr bool SPEC = decltype(spec_c)::value;
    bf16x8 kf = k_frag(buf, 0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 kn = kf;
      if (c + 1 < NC) kn = k_frag(buf, c + 1);
      if (c == 0 && !SPEC) {
        const f32x16 zero = {};
        acc = mfma32(kf, qf[0], zero);
      } else {
        acc = mfma32(kf, qf[c], acc);
      }
      kf = kn;
    }
  };
  auto step_pv = [&](const unsigned char* buf, const bf16x8 (&pf)[2]) {
    bf16x8 vf[2 * NDB];
#pragma unroll
    for (int idx = 0; idx < 2 * NDB; ++idx) vf[idx] = v_frag(buf, idx);
#pragma unroll
    for (int idx = 0; idx < 2 * NDB; ++idx) oacc[idx >> 1] = mfma32(vf[idx], pf[idx & 1], oacc[idx >> 1]);
    // V fragments read one head-dim block ahead of the MFMAs that consume them (left alone,
    // the scheduler reuses one set of registers and waits out each read)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  auto step_probs = [&](const f32x16& acc, float m_use, bf16x8 (&pf)[2]) {
    float psum = l_run;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float p0 = fast_exp2(fmaf(acc[8 * kk + 2 * jj], cqk_r, -m_use));
        const float p1 = fast_exp2(fmaf(acc[8 * kk + 2 * jj + 1], cqk_r, -m_use));
        w[jj] = pack_bf16x2(p0, p1);
        psum = sum_bf16x2(w[jj], psum);
      }
      pf[kk] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
    }
    l_run = psum;
  };
  auto step_rowmax = [&](const f32x16& acc) -> float {
    float v = fmaxf(fmaxf(acc[0], acc[1]), acc[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) v = fmaxf(fmaxf(v, acc[i]), acc[i + 1]);
    v = fmaxf(v, acc[15]);
    return pair_max(v) * cqk_r;
  };
  auto rescale = [&](float mx) {
    const bool need = mx > m_run + kRescale;
    if (__any(need)) {
      float alpha = need ? fast_exp2(m_run - mx) : 1.f;
      asm volatile("; rare path: rescale O" : "+v"(alpha));
      if (need) m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
  };

  using false_t = std::integral_constant<bool, false>;
  using true_t = std::integral_constant<bool, true>;

  // ---- prologue: tiles 0 and 1, the query rows and the E rows of steps 0 and 1 requested
  // together (one memory round trip), then the curves and scores of step 0 ---------------------
  u32x4 ef1[2][NEF];
#pragma unroll
  for (int u = 0; u < 2 * NEF; ++u) ef1[u / NEF][u % NEF] = u32x4{0u, 0u, 0u, 0u};
  if (MODE == 2 && (ALLBAND || step_inband(0))) e_fetch(0);
  if (MODE == 2 && (ALLBAND || step_inband(1))) e_fetch_to(1, ef1);
  dma_wait();
  __syncthreads();

  f32x16 sa, sb;
  {
    if (MODE == 2 && (ALLBAND || step_inband(0))) curve_issue(0);
#pragma unroll
    for (int u = 0; u < 2 * NEF; ++u) ef[u / NEF][u % NEF] = ef1[u / NEF][u % NEF];
    if (step_special(0)) {
      sa = step_init(0);
      step_scores(smem, sa, true_t{});
    } else {
      step_scores(smem, sa, false_t{});
    }
    const float mx = step_rowmax(sa);
    curve_step(1);
    rescale(mx);
  }

  // ---- key loop: iteration js consumes the scores of step js and produces those of js + 1 ----
  // One iteration on three distinct buffers (restrict: the compiler then knows that the loads
  // into dbuf do not feed the reads of tiles js and js + 1, and does not wait for them there).
  // INNER: step js + 2 is known to exist (inside the unrolled loop), so the tile load and the
  // curve step are unconditional and the compiler counts the loads in flight exactly (a
  // conditional load makes it wait for all of them before the next use of the E rows).
  auto iteration_body = [&](int js, f32x16& scur, f32x16& snxt, unsigned char* __restrict__ dbuf,
                            const unsigned char* __restrict__ cbuf_t, const unsigned char* __restrict__ nbuf_t,
                            auto inner_c) {
    constexpr bool INNER = decltype(inner_c)::value;
    const bool more = INNER || js + 2 < nsteps;
    if (more) dma_tile(js + 2, dbuf);

    const float m_use = (m_run == NEG_INF) ? 0.f : m_run;
    bf16x8 pf[2];
    auto fence_stage1 = [&]() {
      asm volatile("" : "+v"(snxt));
      asm volatile("" : "+v"(pf[0]), "+v"(pf[1]));
    };
    // stage 1: S MFMAs of step js + 1 beside the exp / pack of step js
    if (step_special(js + 1)) {
      snxt = step_init(js + 1);
      step_scores(nbuf_t, snxt, true_t{});
      step_probs(scur, m_use, pf);
      fence_stage1();
    } else {
      step_scores(nbuf_t, snxt, false_t{});
      step_probs(scur, m_use, pf);
      fence_stage1();
    }
    // stage 2: P.V MFMAs of step js beside the row max of step js + 1, then the curves of
    // step js + 2.  In the branch-free loop the two curve MFMAs go in ahead of the P.V MFMAs
    // (pinned there: the compiler would otherwise sink them to their use), so that their
    // results are ready when the conversions and LDS writes that follow the P.V MFMAs need them.
    if (MODE == 2 && ALLBAND && INNER) {
      f32x16 clo, chi;
      curve_mfma(clo, chi);
      asm volatile("" : "+v"(clo), "+v"(chi), "+v"(pf[0]), "+v"(pf[1]));
      __builtin_amdgcn_sched_barrier(0);
      step_pv(cbuf_t, pf);
      const float mx = step_rowmax(snxt);
#pragma unroll
      for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(oacc[db]));
      curve_store(clo, chi);
      e_fetch(js + 3);
      rescale(mx);
    } else {
      step_pv(cbuf_t, pf);
      const float mx = step_rowmax(snxt);
#pragma unroll
      for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(oacc[db]));
      if (more) curve_step(js + 2);
      rescale(mx);
    }
  };
  // tile js + 1 (loaded a step ago) is in LDS once every wave's loads have landed; every wave
  // is then also done with tile js - 1, whose buffer takes tile js + 2.  The loads issued after
  // tile js + 1 are the E rows of step js + 2 when that step is in band (the curve step of
  // js + 1 fetched them), nothing else.
  auto iteration_wait = [&](int js) {
    if (MODE == 2 && (ALLBAND || step_inband(js + 2)))
      dma_wait_but_e();
    else
      dma_wait();
    __syncthreads();
  };
  // Tile t sits in ring buffer t % 3.  In the unrolled loop the buffer of each iteration is a
  // compile-time constant (SL = js % 3), so every fragment read addresses LDS as a per-lane
  // offset plus an immediate, with no address arithmetic per step.
  auto iteration_at = [&](int js, f32x16& scur, f32x16& snxt, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    iteration_wait(js);
    iteration_body(js, scur, snxt, smem + ((SL + 2) % NBUF) * BUF_BYTES, smem + SL * BUF_BYTES,
                   smem + ((SL + 1) % NBUF) * BUF_BYTES, true_t{});
  };
  auto iteration = [&](int js, f32x16& scur, f32x16& snxt) {
    iteration_wait(js);
    const int sl = js % NBUF;
    iteration_body(js, scur, snxt, smem + ((sl + 2) % NBUF) * BUF_BYTES, smem + sl * BUF_BYTES,
                   smem + ((sl + 1) % NBUF) * BUF_BYTES, false_t{});
  };
  int js = 0;
  for (; js + 4 < nsteps; js += 3) {
    iteration_at(js, sa, sb, std::integral_constant<int, 0>{});
    iteration_at(js + 1, sb, sa, std::integral_constant<int, 1>{});
    iteration_at(js + 2, sa, sb, std::integral_constant<int, 2>{});
    sa = sb;   // the scores of step js + 3 back in the first set
  }
  for (; js + 1 < nsteps; ++js) {
    iteration(js, sa, sb);
    sa = sb;
  }

  // ---- last step ------------------------------------------------------------------------------
  {
    const float m_use = (m_run == NEG_INF) ? 0.f : m_run;
    bf16x8 pf[2];
    step_probs(sa, m_use, pf);
    step_pv(smem + (js % NBUF) * BUF_BYTES, pf);
  }

  // ---- epilogue -------------------------------------------------------------------------------
  // O^T holds 4-dim pieces of each row in the two lanes of that row; the rows go through the
  // ring's LDS (8 KB per wave, once every wave is done with the last tile) so that each store
  // instruction writes four whole 256-byte rows instead of 16 bytes of 32 rows.  Chunk c (16
  // bytes) of row r sits at slot c ^ (r % 16), which keeps both the writes and the reads
  // spread over the banks.
  const int row = i0 + ln;
  const float lt = pair_sum(l_run);
  const float inv = 1.f / lt;
  unsigned char* ot = smem + wave * (ROWS_WG * D * 2);
  __syncthreads();
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int chunk = (4 * db + g4) ^ (ln & 15);
      const f32x16& acc = oacc[db];
      *reinterpret_cast<u32x2*>(ot + ln * (D * 2) + chunk * 16 + 8 * lh) =
          u32x2{pack_bf16x2(acc[4 * g4] * inv, acc[4 * g4 + 1] * inv),
                pack_bf16x2(acc[4 * g4 + 2] * inv, acc[4 * g4 + 3] * inv)};
    }
  if (a.lse && lh == 0 && row < S)
    a.lse[(static_cast<size_t>(b) * a.Hq + h) * S + row] = (m_run + fast_log2(lt)) * kLn2;
  wave_sync_lds();
#pragma unroll
  for (int it = 0; it < ROWS_WG / 4; ++it) {
    const int r = 4 * it + (lane >> 4);
    const int c = lane & 15;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ot + r * (D * 2) + ((c ^ (r & 15)) * 16));
    if (i0 + r < S) st16(a.o + (static_cast<size_t>(b) * S + i0 + r) * q_row + static_cast<size_t>(h) * D + 8 * c, v);
  }
}

constexpr int kMaxLdsPerWg = 80 * 1024;   // two workgroups per CU

int split_lds(int mode, int Rb) {
  if (mode == 1) return TILE_BYTES + 4 * (Rb + 2 * PAD) * 4;
  if (mode == 2) return TILE_BYTES + 4 * CURVE_BYTES;
  return TILE_BYTES;
}

template <int MODE, int EW, bool ALLBAND>
hipError_t launch_split(FwdArgs a, const float* E, void* workspace, hipStream_t s) {
  a.hpw = 4;
  a.rows_wg = ROWS_WG;
  a.n_qtiles = (a.S + ROWS_WG - 1) / ROWS_WG;
  a.n_hgroups = a.Hq / 4;
  a.longest_first = (a.window == 0 || a.window > ROWS_WG) ? 1 : 0;
  const long long nblk = static_cast<long long>(a.n_qtiles) * a.n_hgroups * a.B;
  if (nblk <= 0) return hipSuccess;
  const int lds = split_lds(MODE, a.bias_range);
  // every check that can fail comes before the first launch
  hipError_t e = set_max_lds(reinterpret_cast<const void*>(&fwd_split_kernel<MODE, EW, ALLBAND>), lds, s);
  if (e != hipSuccess) return e;
  uint16_t* e2 = static_cast<uint16_t*>(workspace);
  if (MODE == 2) {
    e = launch_e2_convert(E, a.e_hs, a.R, a.bias_range, kLog2e / a.c_qk, a.e_hs ? a.Hq : 1, e2, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((fwd_split_kernel<MODE, EW, ALLBAND>), dim3(static_cast<unsigned>(nblk)), dim3(NT), lds, s, a, e2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_e2_convert(const float* E, long long e_hs, int R, int Rb, float inv_scale, int heads,
                             uint16_t* e2, hipStream_t s) {
  const int EW = e2_width(R);
  const int rows = Rb + 2 * PAD + 1;
  hipLaunchKernelGGL(e2_convert_kernel, dim3((rows + 255) / 256, heads, EW / 16), dim3(256), 0, s, E, e_hs, R, Rb,
                     inv_scale, EW, e2);
  return hipGetLastError();
}

// Workspace bytes the split prefill needs (the converted E of r.E bias), or -1 when the shape
// is outside its domain (head_dim 128, GQA groups of 4k heads, positive scale, LDS per
// workgroup within half the CU).
long long fwd_split_workspace(int D_, int G, int mode, int Rb, int R, int e_shared, int Hq, float scale) {
  if (D_ != D || G % 4 != 0 || !(scale > 0.f) || Hq > 65535) return -1;
  if (mode != 0 && Rb % 4 != 0) return -1;
  if (split_lds(mode, Rb) > kMaxLdsPerWg) return -1;
  if (mode != 2) return 0;
  return e2_bytes(e_shared ? 1 : Hq, Rb, e2_width(R));
}

hipError_t launch_fwd_bf16_split(const FwdArgs& a, int mode, void* workspace, hipStream_t s) {
  if (mode == 0) return launch_split<0, 16, false>(a, nullptr, nullptr, s);
  if (mode == 1) return launch_split<1, 16, false>(a, nullptr, nullptr, s);
  const bool allband = a.window != 0 && a.window <= a.bias_range;
  if (a.R > 8)
    return allband ? launch_split<2, 32, true>(a, a.E, workspace, s) : launch_split<2, 32, false>(a, a.E, workspace, s);
  return allband ? launch_split<2, 16, true>(a, a.E, workspace, s) : launch_split<2, 16, false>(a, a.E, workspace, s);
}

}  // namespace rba
