// Prefill, fast path for head_dim 128 and GQA groups of 4k query heads (gfx950).
//
// Same operation as the generic prefill kernel (scaled q.k plus a bias read at
// the distance i - j, zero at and beyond the range, causal / sliding window;
// "Thinking Machines dropped RoPE", steps 3-5 and the kernel-cost section),
// organised for MFMA throughput:
//
//   * workgroup = 4 waves = the 4 query heads of one GQA group over the same
//     64 query rows; each wave owns 64 rows (two 32-row MFMA blocks), so every
//     16-byte K or V fragment read from LDS feeds two MFMAs (8 LDS bytes per
//     logit for K and V together);
//   * K/V tiles of 64 keys, double-buffered in LDS; the tile after next is
//     fetched into registers while the current one is in use (V transposed on
//     its way to LDS);
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: each lane owns
//     one query row, P stays in registers;
//   * the key loop is a two-stage software pipeline over 32-key steps: the
//     S MFMAs of step j+1 are issued next to the exp / pack of step j, and the
//     P.V MFMAs of step j next to the row max of step j+1, so the matrix cores
//     and the vector ALUs work at the same time;
//   * bias and mask enter through the MFMA accumulator: the S accumulator of a
//     step starts at bias / scale (or -inf where a key is not visible), so
//     scale * (q.k + bias / scale) = scale * q.k + bias comes out of the MFMA
//     and the softmax needs no per-element fix-up; steps with neither bias nor
//     mask start at zero;
//   * online softmax with lazy rescaling: the running max only moves when a
//     row's max grows by more than 2^8, so the O rescale is rare;
//   * table bias: the group's table rows sit in LDS, padded with zero distances on both sides,
//     and each lane reads its 16 distances from one base with immediate offsets;
//   * input-dependent bias r_i . E[h, :, delta]: E (bf16, zero-padded the same way) for the
//     group's heads is staged in LDS once per workgroup; the curves of a 32x32 block over its
//     64 distances are two MFMAs (K = the R features) stored unskewed to a per-wave buffer
//     (row = query, column = distance), and each lane reads its diagonal delta = c + n - m with
//     aligned dword reads and v_perm; when E does not fit in LDS the curve MFMA reads it from
//     global memory and consecutive key blocks share curve blocks through a skewed ring;
//   * steps outside the window are skipped by the mask; steps beyond the bias
//     range are content-only (the NoPE tail of global layers).

#ifndef RBA_FORCE_GLOBAL_E
#define RBA_FORCE_GLOBAL_E 0
#endif

#include <type_traits>

#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

constexpr int D = 128;
constexpr int BN = 64;            // keys per tile
constexpr int NC = D / 16;        // K = 16 chunks of the head dim
constexpr int NDB = D / 32;       // 32-wide head-dim blocks of O^T
constexpr int KST = D + 8;        // K tile row stride (bf16)
constexpr int VST = BN + 8;       // V^T tile row stride (bf16)
constexpr int RST = 68;           // ring curve buffer row stride (bf16), E read from global memory
constexpr int CBW = 72;           // curve buffer row stride (bf16), staged E: 64 slots + pad
constexpr int PAD = 64;           // zero distances staged on each side of the bias range
constexpr int ROWS_WG = 64;       // query rows per workgroup
constexpr float kRescale = 8.f;   // lazy rescale threshold (log2 units)

constexpr int KS_BYTES = BN * KST * 2;
constexpr int VT_BYTES = D * VST * 2;
constexpr int BUF_BYTES = KS_BYTES + VT_BYTES;
constexpr int RING_BYTES_PER_QB = 32 * RST * 2;
constexpr int CURVE_BYTES_PER_QB = 32 * CBW * 2;

// QB 32-row query blocks per wave; 8 / QB waves = 4 heads x (2 / QB) row halves.

__device__ __forceinline__ int vt_pos(int x) {
  return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// MODE 0 none, 1 table, 2 r.E; EF = features per distance in the staged E (8 or 16);
// RING: one curve buffer per query block, shared by consecutive key blocks.
// ESTAGE: E is staged in LDS (bf16); otherwise the curve MFMA reads fp32 E from global memory.
// ALLBAND: every visible key is inside the bias range (window <= range, local layers), so every
// step carries the bias; with staged E its curves are then formed a step ahead, without branches.
template <int MODE, int EF, bool RING, int QB, bool ESTAGE, bool ALLBAND>
__global__ __launch_bounds__(512 / QB, 1) void fwd_fast_kernel(FwdArgs a, int bias_off, int ring_off) {
  constexpr int NT = 512 / QB;      // threads per workgroup
  // staged-E curves formed one step ahead of their use
  constexpr bool PIPE = MODE == 2 && ESTAGE && ALLBAND;
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
  const int i0 = qt * ROWS_WG;
  const int h = hg * 4 + (wave & 3);
  const int i0w = i0 + 32 * QB * (wave >> 2);   // first row of this wave
  const int hkv = h / a.G;
  const int row_last = min(S, i0 + ROWS_WG) - 1;
  const int kmin = W ? max(0, i0 - W + 1) : 0;
  const int t_begin = kmin / BN;
  const int ntiles = row_last / BN - t_begin + 1;
  const int nsteps = 2 * ntiles;

  const float cqk = a.c_qk;              // scale * log2(e)
  const float inv_scale = kLog2e / cqk;  // bias -> accumulator units (bias / scale)
  // per query row: scale * log2(e) times the row's context-length temperature, which
  // multiplies the q.k term and the bias alike (both sit in the accumulator)
  float cqk_r[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
    cqk_r[qb] = cqk * temp_factor(visible_keys(i0w + 32 * qb + ln, W), a.temp_len, a.temp_inv_log2);

  const size_t q_row = static_cast<size_t>(a.Hq) * D;
  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const uint16_t* kbase = a.k + static_cast<size_t>(b) * S * kv_row + static_cast<size_t>(hkv) * D;
  const uint16_t* vbase = a.v + static_cast<size_t>(b) * S * kv_row + static_cast<size_t>(hkv) * D;

  // ---- K/V staging: 64 keys x 128 dims of K and of V per tile.  K: 1024 chunks of 16 B,
  // row-major; V: 256 items of 4 keys x 8 dims, transposed.  With 256 threads each thread
  // takes 4 K chunks and one V item; with 512 threads half take K, half take V.
  // staging registers: with 512 threads a thread stages either K or V, so both share one set
  constexpr int VR0 = (NT == 512) ? 0 : 4;
  u32x4 sreg[VR0 + 4];
  const bool v_thread = (NT == 256) || (wave >= 4);
  const bool k_thread = (NT == 256) || (wave < 4);
  const int vt_id = tid & 255;
  const int v_kg = vt_id & 15;
  const int v_dg = vt_id >> 4;
  // Byte offsets inside a tile; rows at or past S read as zeros through the buffer range
  // (rows - r0) * row bytes - head offset, which every in-range 16-byte chunk fits below.
  const int kv_row_b = a.Hkv * D * 2;
  const int head_b = hkv * D * 2;
  const int k_voff = (vt_id >> 4) * kv_row_b + 16 * (vt_id & 15);
  const int v_voff = 4 * v_kg * kv_row_b + 16 * v_dg;
  auto rows_rsrc = [&](const uint16_t* base, int r0) {
    const int left = S - r0;
    return make_rsrc(base + static_cast<size_t>(r0) * kv_row, left > 0 ? left * kv_row_b - head_b : 0);
  };
  auto load_tile = [&](int tk0) {
    if (k_thread) {
#pragma unroll
      for (int it = 0; it < 4; ++it) sreg[it] = buf_ld16(rows_rsrc(kbase, tk0 + 16 * it), k_voff);
    }
    if (v_thread) {
#pragma unroll
      for (int s = 0; s < 4; ++s) sreg[VR0 + s] = buf_ld16(rows_rsrc(vbase, tk0 + s), v_voff);
    }
    if (QB == 2) {   // 1 wave per SIMD: park the staged tile in the accumulation registers
#pragma unroll
      for (int it = 0; it < VR0 + 4; ++it) asm volatile("" : "+a"(sreg[it]));
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* Ks = reinterpret_cast<uint16_t*>(smem + buf * BUF_BYTES);
    uint16_t* Vt = reinterpret_cast<uint16_t*>(smem + buf * BUF_BYTES + KS_BYTES);
    if (k_thread) {
#pragma unroll
      for (int it = 0; it < 4; ++it) st16(Ks + (it * 16 + (vt_id >> 4)) * KST + 8 * (vt_id & 15), sreg[it]);
    }
    if (v_thread) {
      const int pos = vt_pos(4 * v_kg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
        const uint32_t p01 = __builtin_amdgcn_perm(sreg[VR0 + 1][w], sreg[VR0 + 0][w], sel);
        const uint32_t p23 = __builtin_amdgcn_perm(sreg[VR0 + 3][w], sreg[VR0 + 2][w], sel);
        st8(Vt + (8 * v_dg + e) * VST + pos, u32x2{p01, p23});
      }
    }
  };

  // ---- bias parameters: the first round of their loads (L2-resident) goes out before the
  // HBM loads of the first tile and the query rows, so that converting them into LDS does not
  // wait for those (loads complete in issue order)
  const int Rp = Rb + 2 * PAD;             // padded row length (distances -PAD .. Rb + PAD - 1)
  constexpr int PRE = 8;                   // float4 loads per thread in the first round
  const int n_pvec = (MODE == 1) ? Rb : (MODE == 2 && ESTAGE) ? EF * Rb : 0;   // float4 per group
  const int per_hw = (MODE == 1) ? Rb / 4 : EF * Rb / 4;                        // float4 per head
  const float* Eg = (MODE == 2) ? a.E + static_cast<size_t>(hg) * 4 * a.e_hs : nullptr;
  // head (0..3 within the group) of float4 number vi, without an integer division
  auto item_head = [&](int vi) -> int {
    return static_cast<int>(vi >= per_hw) + static_cast<int>(vi >= 2 * per_hw) + static_cast<int>(vi >= 3 * per_hw);
  };
  auto pfetch = [&](int vi) -> float4 {    // float4 number vi of the group's bias parameters
    if (MODE == 1)
      return reinterpret_cast<const float4*>(a.table + static_cast<size_t>(hg) * 4 * Rb)[vi];
    // E[h, f, 4q .. 4q+3]; the feature index varies fastest over the lanes so that 8
    // neighbouring lanes fill one 16-byte row e2[(hw, d)][0..7] (2-way bank conflicts)
    const int hw = item_head(vi);
    const int rr = vi - hw * per_hw;
    const int f = rr % EF;
    const int dq = rr / EF;
    if (f >= a.R) return float4{0.f, 0.f, 0.f, 0.f};
    return reinterpret_cast<const float4*>(Eg + static_cast<size_t>(hw) * a.e_hs + static_cast<size_t>(f) * Rb)[dq];
  };
  auto pstore = [&](int vi, float4 v) {    // scaled to accumulator units, into LDS
    const int hw = item_head(vi);
    const int rr = vi - hw * per_hw;
    if (MODE == 1) {
      float* tab = reinterpret_cast<float*>(smem + bias_off);
      *reinterpret_cast<float4*>(tab + hw * Rp + PAD + 4 * rr) =
          float4{v.x * inv_scale, v.y * inv_scale, v.z * inv_scale, v.w * inv_scale};
    } else {
      uint16_t* e2 = reinterpret_cast<uint16_t*>(smem + bias_off);
      const int f = rr % EF;
      const int dq = rr / EF;
      uint16_t* dst = e2 + (hw * (Rp + 1) + PAD + 4 * dq) * EF + f;
      dst[0] = f32_to_bf16(v.x * inv_scale);
      dst[EF] = f32_to_bf16(v.y * inv_scale);
      dst[2 * EF] = f32_to_bf16(v.z * inv_scale);
      dst[3 * EF] = f32_to_bf16(v.w * inv_scale);
    }
  };
  float4 pre[PRE];
  if (n_pvec > 0) {
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
      const int vi = tid + NT * u;
      pre[u] = float4{0.f, 0.f, 0.f, 0.f};
      if (vi < n_pvec) pre[u] = pfetch(vi);
    }
  }

  // first tile in flight while the bias parameters are staged
  load_tile(t_begin * BN);

  // ---- per-wave constants -------------------------------------------------------------------
  bf16x8 qf[QB][NC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = i0w + 32 * qb + ln;
    const uint16_t* qp = a.q + (static_cast<size_t>(b) * S + row) * q_row + static_cast<size_t>(h) * D + 8 * lh;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < S) v = ld16(qp + 16 * c);
      qf[qb][c] = as_bf16x8(v);
    }
  }
  // The query fragments are only ever MFMA operands: keep them in the accumulation
  // registers so the architectural VGPRs stay free for O and the softmax.
  if (QB == 2) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int c = 0; c < NC; ++c) asm volatile("" : "+a"(qf[qb][c]));
  }
  bf16x8 rf[QB];
  const bool r_vec = a.R == EF && (reinterpret_cast<uintptr_t>(a.r) & 15) == 0;
  if (MODE == 2) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = i0w + 32 * qb + ln;
      const uint16_t* rp = a.r + ((static_cast<size_t>(b) * S + row) * a.Hq + h) * a.R;
      const int f0 = (EF == 16) ? 8 * lh : 0;
      const bool live = row < S && (EF == 16 || lh == 0);
      if (r_vec) {
        // rows of exactly EF features, 16-byte aligned: one load, no arithmetic on the value
        // (its first use, the curve MFMA of the first step, waits for it there)
        u32x4 v = {0u, 0u, 0u, 0u};
        if (live) v = ld16(rp + f0);
        rf[qb] = as_bf16x8(v);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int f = f0 + 2 * jj;
          const uint32_t lo = (live && f < a.R) ? rp[f] : 0u;
          const uint32_t hi = (live && f + 1 < a.R) ? rp[f + 1] : 0u;
          w[jj] = lo | (hi << 16);
        }
        rf[qb] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
      }
    }
  }

  // ---- stage the group's bias parameters in LDS, in accumulator units (bias / scale) ------
  // Rows in LDS are padded with PAD zero distances on both sides, so that every in-band step
  // reads its distances c - 62 .. c + 63 without guards: zero below 0 (those keys are masked
  // anyway) and at and beyond the range.
  if (n_pvec > 0) {
#pragma unroll
    for (int u = 0; u < PRE; ++u)
      if (tid + NT * u < n_pvec) pstore(tid + NT * u, pre[u]);
    for (int base = tid + NT * PRE; base < n_pvec; base += NT * PRE) {   // larger ranges
      float4 v[PRE];
#pragma unroll
      for (int u = 0; u < PRE; ++u)
        if (base + NT * u < n_pvec) v[u] = pfetch(base + NT * u);
#pragma unroll
      for (int u = 0; u < PRE; ++u)
        if (base + NT * u < n_pvec) pstore(base + NT * u, v[u]);
    }
  }
  if (MODE == 1) {
    float* tab = reinterpret_cast<float*>(smem + bias_off);
    for (int i = tid; i < 4 * 2 * PAD; i += NT) {
      const int hw = i / (2 * PAD);
      const int k = i - hw * 2 * PAD;
      tab[hw * Rp + (k < PAD ? k : Rb + k)] = 0.f;
    }
  }
  if (MODE == 2 && ESTAGE) {
    // zero pads (one extra distance row at the end for the upper-half lanes' over-read)
    uint32_t* e2u = reinterpret_cast<uint32_t*>(smem + bias_off);
    const int pad_words = (2 * PAD + 1) * EF / 2;
    for (int i = tid; i < 4 * pad_words; i += NT) {
      const int hw = i / pad_words;
      const int k = i - hw * pad_words;
      const int lo_words = PAD * EF / 2;
      e2u[(hw * (Rp + 1)) * EF / 2 + (k < lo_words ? k : Rb * EF / 2 + k)] = 0u;
    }
  }

  float m_run[QB], l_run[QB];
  f32x16 oacc[QB][NDB];
  int ring_lo[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
    ring_lo[qb] = 0x7fffffff;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.f;
  }

  const float NEG_INF = -INFINITY;
  // v_perm selectors for the curve reads: bf16 number r (0..2) of a dword pair into the top
  // half, zero bytes (selector 12) below; r = parity of the lane's row (+1 for sel_b)
  auto perm_sel = [](int r) -> uint32_t {
    return 0x0c0cu | (static_cast<uint32_t>(2 * r) << 16) | (static_cast<uint32_t>(2 * r + 1) << 24);
  };
  const uint32_t sel_a = perm_sel(ln & 1);
  const uint32_t sel_b = perm_sel((ln & 1) + 1);
  // the wave's head row at distance 0
  const float* tabw = (MODE == 1) ? reinterpret_cast<const float*>(smem + bias_off) + (wave & 3) * Rp + PAD : nullptr;
  const uint16_t* e2w = (MODE == 2) ? reinterpret_cast<const uint16_t*>(smem + bias_off) + ((wave & 3) * (Rp + 1) + PAD) * EF : nullptr;
  uint16_t* ring = (MODE == 2) ? reinterpret_cast<uint16_t*>(smem + ring_off) +
                                     wave * QB * 32 * (ESTAGE ? CBW : RST) : nullptr;

  // All-in-band layers, staged E: curves of step js, two MFMAs over the R features give the curves of the 64
  // distances c - 31 .. c + 32 for every query row of the block; they are written unskewed to the
  // wave's curve buffer (row = query, column = distance - (c - 31)) and each lane's diagonal is
  // read back into cr.  Issued one step ahead, so that neither the MFMA nor the LDS round trip
  // sits in front of the step's score MFMAs.
  uint32_t cr[QB][12];
  auto curve_issue = [&](int js) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int j0 = (t_begin + (js >> 1)) * BN + 32 * (js & 1);
      // every visible key is in band, so a step outside the band is fully masked: clamp its
      // offset to keep the reads inside the staged rows (distances -PAD .. Rb + PAD)
      const int c = min(max((i0w + 32 * qb) - j0, -33), Rb + 31);
      uint16_t* cb = ring + (QB > 1 ? qb : 0) * 32 * CBW;
      const uint16_t* ep = e2w + (c - 31 + ln) * EF + 8 * lh;
      const f32x16 zero = {};
      const f32x16 lo = mfma32(as_bf16x8(ld16(ep)), rf[qb], zero);
      const f32x16 hi = mfma32(as_bf16x8(ld16(ep + 32 * EF)), rf[qb], zero);
      uint16_t* wp = cb + ln * CBW + 4 * lh;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        st8(wp + 8 * k, u32x2{pack_bf16x2(lo[4 * k], lo[4 * k + 1]), pack_bf16x2(lo[4 * k + 2], lo[4 * k + 3])});
        st8(wp + 32 + 8 * k, u32x2{pack_bf16x2(hi[4 * k], hi[4 * k + 1]), pack_bf16x2(hi[4 * k + 2], hi[4 * k + 3])});
      }
      wave_sync_lds();
      // dword reads are always aligned; the lane's run of key m0 .. m0 + 3 spans three of them
      const uint32_t* rd = reinterpret_cast<const uint32_t*>(cb) + ln * (CBW / 2) + (ln >> 1) + 2 - 2 * lh;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        cr[qb][3 * g4] = rd[12 - 4 * g4];
        cr[qb][3 * g4 + 1] = rd[13 - 4 * g4];
        cr[qb][3 * g4 + 2] = rd[14 - 4 * g4];
      }
    }
  };

  // Whether step js of query block qb starts from something other than zero (bias in band,
  // or a mask at the window / causal edges); uniform across the wave.
  auto step_special = [&](int js, int qb) -> bool {
    const int j0 = (t_begin + (js >> 1)) * BN + 32 * (js & 1);
    const int c = (i0w + 32 * qb) - j0;
    bool on = (c + 31 >= 0) && (j0 < S) && (i0w + 32 * qb < S);
    if (W) on = on && (c - 31 < W);
    const bool edge = !on || (c - 31 < 0) || (W && c + 31 >= W);
    const bool inband = on && (MODE != 0) && (c - 31 < Rb);
    return edge || inband;
  };
  // Accumulator start values of a special step: bias / scale where the key is visible and
  // in band, 0 where visible and beyond the band, -inf elsewhere.
  auto step_init = [&](int js, int qb) -> f32x16 {
    f32x16 init;
#pragma unroll
    for (int i = 0; i < 16; ++i) init[i] = 0.f;
    const int j0 = (t_begin + (js >> 1)) * BN + 32 * (js & 1);
    const int c = (i0w + 32 * qb) - j0;                // delta = c + n - m
    bool on = (c + 31 >= 0) && (j0 < S) && (i0w + 32 * qb < S);
    if (W) on = on && (c - 31 < W);
    const bool edge = !on || (c - 31 < 0) || (W && c + 31 >= W);
    const bool inband = on && (MODE != 0) && (c - 31 < Rb);
    if (MODE == 1 && inband) {
      asm volatile("; in-band step: table bias" ::: "memory");
      // d = c + n - m with m = 8 g + 4 lh + j: one base per lane, immediate offsets 27 - 8 g - j
      const float* tb = tabw + (c + ln - 4 * lh - 27);
#pragma unroll
      for (int i = 0; i < 16; ++i) init[i] = tb[27 - 8 * (i >> 2) - (i & 3)];
    }
    if (MODE == 2 && ESTAGE && !PIPE && inband) {
      asm volatile("; in-band step: r.E bias" ::: "memory");
      // curves of the 64 distances c - 31 .. c + 32 for every query row of the block (two
      // MFMAs over the R features), written unskewed: row n, column = distance - (c - 31)
      uint16_t* cb = ring + (QB > 1 ? qb : 0) * 32 * CBW;
      const uint16_t* ep = e2w + (c - 31 + ln) * EF + 8 * lh;
      const f32x16 zero = {};
      const f32x16 lo = mfma32(as_bf16x8(ld16(ep)), rf[qb], zero);
      const f32x16 hi = mfma32(as_bf16x8(ld16(ep + 32 * EF)), rf[qb], zero);
      uint16_t* wp = cb + ln * CBW + 4 * lh;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        st8(wp + 8 * k, u32x2{pack_bf16x2(lo[4 * k], lo[4 * k + 1]), pack_bf16x2(lo[4 * k + 2], lo[4 * k + 3])});
        st8(wp + 32 + 8 * k, u32x2{pack_bf16x2(hi[4 * k], hi[4 * k + 1]), pack_bf16x2(hi[4 * k + 2], hi[4 * k + 3])});
      }
      wave_sync_lds();
      // key m of lane n sits at column 31 + n - m: keys m0 .. m0 + 3 (m0 = 8 g + 4 lh) are the
      // four columns from 28 + n - m0, which start on a 2-byte boundary for odd n.  Read the
      // three dwords around them (dword accesses are always aligned) and let v_perm move each
      // bf16 into the top half of an fp32 with zeros below: column 28 + n - m0 + k holds key
      // m0 + 3 - k.
      const uint32_t* rd = reinterpret_cast<const uint32_t*>(cb) + ln * (CBW / 2) + (ln >> 1) + 2 - 2 * lh;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint32_t d0 = rd[12 - 4 * g4], d1 = rd[13 - 4 * g4], d2 = rd[14 - 4 * g4];
        init[4 * g4 + 3] = __uint_as_float(__builtin_amdgcn_perm(d1, d0, sel_a));
        init[4 * g4 + 2] = __uint_as_float(__builtin_amdgcn_perm(d1, d0, sel_b));
        init[4 * g4 + 1] = __uint_as_float(__builtin_amdgcn_perm(d2, d1, sel_a));
        init[4 * g4 + 0] = __uint_as_float(__builtin_amdgcn_perm(d2, d1, sel_b));
      }
      wave_sync_lds();
    }
    if (PIPE) {
      asm volatile("; in-band step: r.E bias, curves read a step ahead" ::: "memory");
      // key m of lane n sits at column 31 + n - m of the curve buffer: keys m0 .. m0 + 3
      // (m0 = 8 g + 4 lh) are the four columns from 28 + n - m0, which start on a 2-byte boundary
      // for odd n.  The three dwords around them were read a step ahead (curve_issue); v_perm
      // moves each bf16 into the top half of an fp32 with zeros below: column 28 + n - m0 + k
      // holds key m0 + 3 - k.
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint32_t d0 = cr[qb][3 * g4], d1 = cr[qb][3 * g4 + 1], d2 = cr[qb][3 * g4 + 2];
        init[4 * g4 + 3] = __uint_as_float(__builtin_amdgcn_perm(d1, d0, sel_a));
        init[4 * g4 + 2] = __uint_as_float(__builtin_amdgcn_perm(d1, d0, sel_b));
        init[4 * g4 + 1] = __uint_as_float(__builtin_amdgcn_perm(d2, d1, sel_a));
        init[4 * g4 + 0] = __uint_as_float(__builtin_amdgcn_perm(d2, d1, sel_b));
      }
    }
    if (MODE == 2 && !ESTAGE && inband) {
      // E from global memory: ring of curve blocks, consecutive key blocks share one
      uint16_t* rg = ring + (RING ? qb : 0) * 32 * RST;
      const int gam = c >> 5;
      auto curve_block = [&](int beta) {
        const int dl = 32 * beta + 1 + ln;
        u32x4 ev = {0u, 0u, 0u, 0u};
        if ((EF == 16 || lh == 0) && dl >= 0 && dl < Rb) {
          // E[h, f, dl] for f = 8 lh .. 8 lh + 7 (coalesced over the lanes' distances)
          const float* ep = a.E + static_cast<size_t>(h) * a.e_hs + static_cast<size_t>(8 * lh) * Rb + dl;
          float e[8];
#pragma unroll
          for (int f = 0; f < 8; ++f) e[f] = (8 * lh + f < a.R) ? ep[static_cast<size_t>(f) * Rb] * inv_scale : 0.f;
          ev = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                     pack_bf16x2(e[6], e[7])};
        }
        f32x16 cacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) cacc[i] = 0.f;
        cacc = mfma32(as_bf16x8(ev), rf[qb], cacc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int sidx = 8 * (i >> 2) + 4 * lh + (i & 3);
          const int col = (32 * beta + 1 + sidx - ln + 3) & 63;
          rg[ln * RST + col] = f32_to_bf16(cacc[i]);
        }
      };
      if (!RING || ring_lo[qb] != gam) curve_block(gam);
      curve_block(gam - 1);
      if (RING) ring_lo[qb] = gam - 1;
      wave_sync_lds();
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int m0 = 8 * g4 + 4 * lh;
        const u32x2 w = ld8(rg + ln * RST + ((c - m0) & 63));
        // element k of the run holds key m0 + 3 - k
        init[4 * g4 + 3] = __uint_as_float(w[0] << 16);
        init[4 * g4 + 2] = __uint_as_float(w[0] & 0xffff0000u);
        init[4 * g4 + 1] = __uint_as_float(w[1] << 16);
        init[4 * g4 + 0] = __uint_as_float(w[1] & 0xffff0000u);
      }
      wave_sync_lds();
    }
    if (edge) {
      asm volatile("; edge step: mask" ::: "memory");          // keep this a branch, not selects
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * lh + (i & 3);
        const int d = c + ln - m;
        if (!on || d < 0 || (W && d >= W)) init[i] = NEG_INF;
      }
    }
    return init;
  };

  auto k_frag = [&](int js, int c) -> bf16x8 {
    const uint16_t* Ks = reinterpret_cast<const uint16_t*>(smem + ((js >> 1) & 1) * BUF_BYTES);
    return as_bf16x8(ld16(Ks + (32 * (js & 1) + ln) * KST + 16 * c + 8 * lh));
  };
  auto v_frag = [&](int js, int idx) -> bf16x8 {   // idx = 2 * db + kk
    const uint16_t* Vt = reinterpret_cast<const uint16_t*>(smem + ((js >> 1) & 1) * BUF_BYTES + KS_BYTES);
    return as_bf16x8(ld16(Vt + (32 * (idx >> 1) + ln) * VST + 32 * (js & 1) + 16 * (idx & 1) + 8 * lh));
  };
  // S^T of step js accumulated onto `acc`; the K fragment of chunk c+1 is read before
  // the MFMAs of chunk c.
  // SPEC false: the step starts from the MFMA's zero operand (no start values in registers).
  auto step_scores = [&](int js, f32x16 (&acc)[QB], auto spec_c) {
    constexpr bool SPEC = decltype(spec_c)::value;
    bf16x8 kf = k_frag(js, 0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 kn = kf;
      if (c + 1 < NC) kn = k_frag(js, c + 1);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (c == 0 && !SPEC) {
          const f32x16 zero = {};
          acc[qb] = mfma32(kf, qf[qb][0], zero);
        } else {
          acc[qb] = mfma32(kf, qf[qb][c], acc[qb]);
        }
      }
      kf = kn;
    }
  };
  // O^T += V^T P^T for step js.
  auto step_pv = [&](int js, const bf16x8 (&pf)[QB][2]) {
    bf16x8 vf = v_frag(js, 0);
#pragma unroll
    for (int idx = 0; idx < 2 * NDB; ++idx) {
      bf16x8 vn = vf;
      if (idx + 1 < 2 * NDB) vn = v_frag(js, idx + 1);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[qb][idx >> 1] = mfma32(vf, pf[qb][idx & 1], oacc[qb][idx >> 1]);
      vf = vn;
    }
  };
  // Probabilities of a step (bf16, packed for the P.V MFMA) and the running row sums.
  auto step_probs = [&](const f32x16 (&acc)[QB], const float (&m_use)[QB], bf16x8 (&pf)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float psum = l_run[qb];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t w[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float p0 = fast_exp2(fmaf(acc[qb][8 * kk + 2 * jj], cqk_r[qb], -m_use[qb]));
          const float p1 = fast_exp2(fmaf(acc[qb][8 * kk + 2 * jj + 1], cqk_r[qb], -m_use[qb]));
          w[jj] = pack_bf16x2(p0, p1);
          psum = sum_bf16x2(w[jj], psum);
        }
        pf[qb][kk] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
      }
      l_run[qb] = psum;
    }
  };
  // Row max of a step in log2 units (both halves of the lane pair).
  auto step_rowmax = [&](const f32x16 (&acc)[QB], float (&mx)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float v = fmaxf(fmaxf(acc[qb][0], acc[qb][1]), acc[qb][2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) v = fmaxf(fmaxf(v, acc[qb][i]), acc[qb][i + 1]);
      v = fmaxf(v, acc[qb][15]);
      mx[qb] = pair_max(v) * cqk_r[qb];
    }
  };
  // Lazy rescale: move the running max only when a row grew by more than 2^kRescale.
  auto rescale = [&](const float (&mx)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const bool need = mx[qb] > m_run[qb] + kRescale;
      if (__any(need)) {
        // rare path; the factor passes through an asm so the O multiply stays inside the branch
        float alpha = need ? fast_exp2(m_run[qb] - mx[qb]) : 1.f;
        asm volatile("; rare path: rescale O" : "+v"(alpha));
        if (need) m_run[qb] = mx[qb];
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[qb][db][i] *= alpha;
      }
    }
  };

  // ---- prologue: tile 0 in buffer 0, tile 1 in flight, scores of step 0 ------------------------
  store_tile(0);
  if (ntiles > 1) load_tile((t_begin + 1) * BN);
  __syncthreads();

  using false_t = std::integral_constant<bool, false>;
  using true_t = std::integral_constant<bool, true>;
  // whether any query block of step js needs start values (the two stage-1 variants)
  auto any_special = [&](int js) {
    if (ALLBAND) return true;
    bool sp = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) sp = sp || step_special(js, qb);
    return sp;
  };

  f32x16 sa[QB], sb[QB];
  if (PIPE) curve_issue(0);
  {
    if (any_special(0)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sa[qb] = step_init(0, qb);
      step_scores(0, sa, true_t{});
    } else {
      step_scores(0, sa, false_t{});
    }
    float mx[QB];
    step_rowmax(sa, mx);
    if (PIPE) curve_issue(1);   // (past the last step: offsets clamped, results unused)
    rescale(mx);
  }

  // ---- steady state: two straight-line stages per 32-key step ----------------------------------
  // One iteration consumes the scores of step js (scur) and produces those of step js+1 (snxt);
  // the loop is unrolled by two so that the two score sets swap roles without copies.
  auto iteration = [&](int js, auto odd_c, f32x16 (&scur)[QB], f32x16 (&snxt)[QB]) {
    constexpr bool ODD = decltype(odd_c)::value;
    const int tl = js >> 1;
    if (!ODD && tl + 1 < ntiles) {
      __syncthreads();                      // everyone is done with the buffer of tile tl-1
      store_tile((tl + 1) & 1);
      if (tl + 2 < ntiles) load_tile((t_begin + tl + 2) * BN);
    }
    if (ODD && tl + 1 < ntiles) __syncthreads();   // tile tl+1 is in LDS

    float m_use[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_use[qb] = (m_run[qb] == NEG_INF) ? 0.f : m_run[qb];

    // stage 1: S MFMAs of step js+1 interleaved with the exp / pack of step js, in a variant
    // with start values (bias, masks) and one that starts from zero
    bf16x8 pf[QB][2];
    // (the empty asm at the end of each variant keeps the compiler from merging their tails,
    // which would pull the exp work out of the MFMA stream)
    auto fence_stage1 = [&]() {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        asm volatile("" : "+v"(snxt[qb]));
        asm volatile("" : "+v"(pf[qb][0]), "+v"(pf[qb][1]));
      }
    };
    if (any_special(js + 1)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) snxt[qb] = step_init(js + 1, qb);
      step_scores(js + 1, snxt, true_t{});
      step_probs(scur, m_use, pf);
      fence_stage1();
    } else {
      step_scores(js + 1, snxt, false_t{});
      step_probs(scur, m_use, pf);
      fence_stage1();
    }

    // stage 2: P.V MFMAs of step js interleaved with the row max of step js+1
    float mx[QB];
    step_pv(js, pf);
    step_rowmax(snxt, mx);
    if (PIPE) curve_issue(js + 2);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(oacc[qb][db]));

    rescale(mx);
  };
  int js = 0;
  for (; js + 2 < nsteps; js += 2) {        // nsteps is even: pairs, then one even step
    iteration(js, false_t{}, sa, sb);
    iteration(js + 1, true_t{}, sb, sa);
  }
  iteration(js, false_t{}, sa, sb);

  // ---- last step (scores in sb) -------------------------------------------------------------------
  {
    float m_use[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_use[qb] = (m_run[qb] == NEG_INF) ? 0.f : m_run[qb];
    bf16x8 pf[QB][2];
    step_probs(sb, m_use, pf);
    step_pv(nsteps - 1, pf);
  }

  // ---- epilogue ------------------------------------------------------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = i0w + 32 * qb + ln;
    const float lt = pair_sum(l_run[qb]);
    if (row >= S) continue;
    const float inv = 1.f / lt;
    uint16_t* op = a.o + (static_cast<size_t>(b) * S + row) * q_row + static_cast<size_t>(h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * lh;
        const f32x16& acc = oacc[qb][db];
        st8(op + d, u32x2{pack_bf16x2(acc[4 * g4] * inv, acc[4 * g4 + 1] * inv),
                          pack_bf16x2(acc[4 * g4 + 2] * inv, acc[4 * g4 + 3] * inv)});
      }
    if (a.lse && lh == 0)
      a.lse[(static_cast<size_t>(b) * a.Hq + h) * S + row] = (m_run[qb] + fast_log2(lt)) * kLn2;
  }
}

int bias_bytes(int mode, int Rb, int R) {
  if (mode == 1) return 4 * (Rb + 2 * PAD) * 4;
  if (mode == 2) return 4 * (Rb + 2 * PAD + 1) * (R > 8 ? 16 : 8) * 2;
  return 0;
}

// curve buffers, one per (wave, query block): 8 in all
int ring_bytes(int mode, bool estage) {
  return mode == 2 ? 8 * (estage ? CURVE_BYTES_PER_QB : RING_BYTES_PER_QB) : 0;
}

constexpr int kMaxLds = 160 * 1024;

int lds_total(int mode, int Rb, int R, bool estage) {
  return 2 * BUF_BYTES + (estage || mode != 2 ? bias_bytes(mode, Rb, R) : 0) + ring_bytes(mode, estage);
}

template <int MODE, int EF, bool RING, int QB, bool ESTAGE = true, bool ALLBAND = false>
hipError_t launch_fast(FwdArgs a, hipStream_t s) {
  a.hpw = 4;
  a.rows_wg = ROWS_WG;
  a.n_qtiles = (a.S + ROWS_WG - 1) / ROWS_WG;
  a.n_hgroups = a.Hq / 4;
  a.longest_first = (a.window == 0 || a.window > ROWS_WG) ? 1 : 0;
  const int bias_off = 2 * BUF_BYTES;
  const int ring_off = bias_off + ((MODE != 2 || ESTAGE) ? bias_bytes(MODE, a.bias_range, a.R) : 0);
  const int total = ring_off + ring_bytes(MODE, ESTAGE);
  const long long nblk = static_cast<long long>(a.n_qtiles) * a.n_hgroups * a.B;
  if (nblk <= 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_fast_kernel<MODE, EF, RING, QB, ESTAGE, ALLBAND>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((fwd_fast_kernel<MODE, EF, RING, QB, ESTAGE, ALLBAND>), dim3(static_cast<unsigned>(nblk)), dim3(512 / QB), total, s,
                     a, bias_off, ring_off);
  return hipGetLastError();
}

}  // namespace

// LDS bytes the fast kernel needs, or -1 when the shape is outside its domain.
int fwd_fast_lds_bytes(int D_, int G, int mode, int Rb, int R, float scale) {
  if (D_ != D || G % 4 != 0 || !(scale > 0.f)) return -1;
  if (mode != 0 && Rb % 4 != 0) return -1;
  if (mode == 1 && lds_total(1, Rb, R, true) > kMaxLds) return -1;
  return lds_total(mode, Rb, R, mode != 2);
}

hipError_t launch_fwd_bf16_fast(const FwdArgs& a, int mode, hipStream_t s) {
  // 8 waves x 32 query rows; E staged in LDS when it fits next to the K/V tiles and the
  // per-wave curve buffers, else read from global memory by the curve MFMA.
  switch (mode) {
    case 0: return launch_fast<0, 8, false, 1>(a, s);
    case 1: return launch_fast<1, 8, false, 1>(a, s);
    default: {
      const bool stage = !RBA_FORCE_GLOBAL_E && lds_total(2, a.bias_range, a.R, true) <= kMaxLds;
      // every visible key in band (window <= range): branch-free curve steps
      const bool allband = a.window != 0 && a.window <= a.bias_range;
      if (a.R > 8) {
        if (!stage) return launch_fast<2, 16, true, 1, false>(a, s);
        return allband ? launch_fast<2, 16, true, 1, true, true>(a, s) : launch_fast<2, 16, true, 1, true>(a, s);
      }
      if (!stage) return launch_fast<2, 8, true, 1, false>(a, s);
      return allband ? launch_fast<2, 8, true, 1, true, true>(a, s) : launch_fast<2, 8, true, 1, true>(a, s);
    }
  }
}

}  // namespace rba
