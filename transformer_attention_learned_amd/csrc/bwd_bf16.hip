// Backward of causal attention with a learned relative-position bias: bf16 in, fp32 MFMA
// accumulation, for gfx950 (CDNA4).
//
// The bias is a trained part of the layer ("Thinking Machines dropped RoPE": the bank of
// distance functions and the coefficient projection are learned with the model; "Learned
// Relative-Position Bias", section "Standard Relative Bias (T5-style)": the table is a
// learned parameter), so besides dq, dk and dv the pass returns the gradient of the bias
// parameters: dtable, or dr and dE for the input-dependent form.  With P the softmax of the
// forward logits s = tau * (scale * q.k + beta) (tau: context-length temperature, 1 if off):
//     dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),  dZ = tau * dS,
//     dq = scale * dZ K,  dk = scale * dZ^T Q,  dv = P^T dO,
//     d beta = dZ at in-band pairs; dtable[h, d] = sum of d beta along the diagonal at
//     distance d; dr[i, f] = sum_j d beta_ij E[f, i - j]; dE[f, d] = sum_i r[i, f] d beta_(i, i-d).
//
// Three kernels on one stream:
//   * bwd_pre: rowsum(dO * O) per (batch, head, row) into the workspace, and zero dE / dtable.
//   * bwd_dq: one workgroup = 4 waves x 32 query rows of one head (the forward's transposed
//     layout: S^T = K Q^T, so each lane owns one query row and its lse, rowsum and temperature
//     are scalars).  Per 32 x 32 block it recomputes S^T and dP^T = V dO^T, forms dZ^T and
//     accumulates dQ^T += K^T dZ^T (K^T in LDS with the key permutation of the forward's V^T).
//     In-band blocks also write dZ into two wave-private skewed buffers, G[query][distance]
//     and its transpose, over the block's 64-distance window; then
//       dr^T += E G^T            (one MFMA per 16 distances; E rows read from global memory)
//       dE   += r^T G  per 32 distances (A = r^T, held in registers for the wave's rows),
//     and the dE / dtable block goes to global memory with fp32 atomics: each instruction
//     adds 32 consecutive distances of one curve, two cache lines.  dtable uses the same MFMA
//     with r replaced by a ones row.
//   * bwd_dkdv: one workgroup = 4 waves x 32 keys of one kv head, looping over the group's
//     query heads and the query tiles that see its keys.  Untransposed layout S = Q K^T (each
//     lane owns one key), K and V held in registers as B operands; Q, dO and their transposes
//     in LDS; per-row lse, rowsum and temperature from LDS.  dV^T += dO^T P and dK^T += Q^T dZ
//     take P and dZ straight from the registers the score MFMAs left them in.  The bias is
//     recomputed per block: table rows staged in LDS with zero padding, or the r.E curve block
//     by MFMA (as in the forward) shared across the wave through LDS.

#include <algorithm>

#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

constexpr int BN = 64;        // keys per tile (dq kernel), query rows per tile (dk/dv kernel)
constexpr int CST = 68;       // row stride (floats) of the curve scratch: 16-byte rows, and the
                              // diagonal reads (stride CST + 1 = 5 mod 64 banks) do not collide
constexpr int PADT = 64;      // zero distances staged on each side of a table row
constexpr int PADE = 64;      // zero distances staged on each side of E
constexpr int GST = 64 + 8;   // G row stride (bf16): row = query, 64 distances
constexpr int GTS = 32 + 8;   // G^T row stride (bf16): row = distance, 32 queries
constexpr int DQ_WAVES = 4;
constexpr int DKV_WAVES = 4;

// Position of key (or query) x of a 64-row tile inside a transposed LDS row: bits 2 and 3
// swapped, so the 8 rows one lane half feeds to an MFMA over 16 rows are contiguous.
__device__ __forceinline__ int vt_pos(int x) {
  return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row of element i of a 32x32 MFMA output in lane half lh.
__device__ __forceinline__ int out_row(int i, int lh) { return 8 * (i >> 2) + 4 * lh + (i & 3); }

// Rows [r0, r0 + 64) of a [.., ld]-strided bf16 tensor (D columns), in items of 4 rows x 8
// columns: load_rows fetches a thread's items into registers (rows >= nrows read as zero),
// store_rows writes them to LDS twice: row-major (stride D + 8) and, if tr != nullptr,
// transposed with the row permutation vt_pos (stride 64 + 8).  Split so that the loads of
// the next tile are in flight while the current one is used.
template <int D>
constexpr int row_items() { return (BN / 4) * (D / 8); }

template <int D, int NIT>
__device__ __forceinline__ void load_rows(const uint16_t* base, size_t ld, int r0, int nrows,
                                          u32x4 (&pre)[NIT][4], int t, int nt) {
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int it = t + k * nt;
    const int rg = it % (BN / 4);
    const int dg = it / (BN / 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int row = r0 + 4 * rg + s;
      pre[k][s] = u32x4{0u, 0u, 0u, 0u};
      if (it < row_items<D>() && row < nrows) pre[k][s] = ld16(base + static_cast<size_t>(row) * ld + 8 * dg);
    }
  }
}

template <int D, int NIT>
__device__ __forceinline__ void store_rows(const u32x4 (&pre)[NIT][4], uint16_t* rm, uint16_t* tr,
                                           int t, int nt) {
#pragma unroll
  for (int k = 0; k < NIT; ++k) {
    const int it = t + k * nt;
    if (it >= row_items<D>()) continue;
    const int rg = it % (BN / 4);
    const int dg = it / (BN / 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) st16(rm + (4 * rg + s) * (D + 8) + 8 * dg, pre[k][s]);
    if (tr) {
      const int pos = vt_pos(4 * rg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const int sh = (e & 1) * 16;
        const uint32_t x0 = (pre[k][0][w] >> sh) & 0xffffu;
        const uint32_t x1 = (pre[k][1][w] >> sh) & 0xffffu;
        const uint32_t x2 = (pre[k][2][w] >> sh) & 0xffffu;
        const uint32_t x3 = (pre[k][3][w] >> sh) & 0xffffu;
        st8(tr + (8 * dg + e) * (BN + 8) + pos, u32x2{x0 | (x1 << 16), x2 | (x3 << 16)});
      }
    }
  }
}

// A 32x32 MFMA output column into a curve-scratch row: rows 8 g + 4 lh + 0..3 are
// consecutive, one 16-byte store each (dst = row start + 4 lh).
__device__ __forceinline__ void store_curve(const f32x16& v, float* dst) {
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<f32x4*>(dst + 8 * g) = f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
}

// The r.E curve block of 32 query rows q0.. over the 64 distances base .. base + 63, written
// to a wave-private scratch cs[query][distance - base] in log2 units: two MFMAs (32 distances
// each) with A = E^T (row = distance, E split into bf16 high and low parts carried by the two
// lane halves) and B = r of the rows (both halves), as in the forward.
template <int D>
__device__ __forceinline__ void curve_block(const BwdArgs& a, const float* Eh, const bf16x8 (&rf)[2],
                                            int base, float* cs, int ln, int lh) {
  const int nfc = (a.R + 7) / 8;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int dl = base + 32 * half + ln;
    f32x16 cacc = zero16();
    for (int fc = 0; fc < nfc; ++fc) {
      uint32_t w[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float e2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int f = 8 * fc + 2 * jj + u;
          float e = 0.f;
          if (f < a.R && dl >= 0 && dl < a.bias_range) e = Eh[static_cast<size_t>(f) * a.bias_range + dl] * kLog2e;
          const float hi = bf16_to_f32(f32_to_bf16(e));
          e2[u] = lh ? (e - hi) : e;
        }
        w[jj] = pack_bf16x2(e2[0], e2[1]);
      }
      cacc = mfma32(as_bf16x8(u32x4{w[0], w[1], w[2], w[3]}), rf[fc], cacc);
    }
    store_curve(cacc, cs + ln * CST + 32 * half + 4 * lh);
  }
}

// r of one query row (lane column) as the B operand of the curve MFMA: both halves carry
// r[row][8 fc + j].
__device__ __forceinline__ void load_rf(const BwdArgs& a, int b, int row, int h, bf16x8 (&rf)[2]) {
  const uint16_t* rp = a.r + ((static_cast<size_t>(b) * a.S + row) * a.Hq + h) * a.R;
#pragma unroll
  for (int fc = 0; fc < 2; ++fc) {
    uint32_t w[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int f0 = 8 * fc + 2 * jj;
      const uint32_t lo = (row < a.S && f0 < a.R) ? rp[f0] : 0u;
      const uint32_t hi = (row < a.S && f0 + 1 < a.R) ? rp[f0 + 1] : 0u;
      w[jj] = lo | (hi << 16);
    }
    rf[fc] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
  }
}

// E staged in LDS for the curve MFMA: row PADE + distance holds, per chunk of 8 curves, the
// bf16 high parts and then the low parts of E * log2(e) (the A operands of the two lane
// halves), zero outside [0, bias_range) and for curves >= R.  Consecutive threads read
// consecutive distances of one curve.
__device__ __forceinline__ void stage_et(const BwdArgs& a, const float* Eh, uint16_t* et, int nfc,
                                         int t, int nt) {
  const int rows = a.bias_range + 2 * PADE;
  const int n = rows * 8 * nfc;
  for (int x = t; x < n; x += nt) {
    const int row = x % rows;
    const int f = x / rows;                 // 8 fc + j
    const int d = row - PADE;
    float e = 0.f;
    if (f < a.R && d >= 0 && d < a.bias_range) e = Eh[static_cast<size_t>(f) * a.bias_range + d] * kLog2e;
    const uint16_t hi = f32_to_bf16(e);
    const uint16_t lo = f32_to_bf16(e - bf16_to_f32(hi));
    uint16_t* dst = et + row * 16 * nfc + 16 * (f >> 3) + (f & 7);
    dst[0] = hi;
    dst[8] = lo;
  }
}

// The curve block of the forward from the staged E: cs[query][distance - base], log2 units.
__device__ __forceinline__ void curve_block_lds(const uint16_t* et, int nfc, const bf16x8 (&rf)[2],
                                                int base, float* cs, int ln, int lh) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint16_t* er = et + (PADE + base + 32 * half + ln) * 16 * nfc + 8 * lh;
    f32x16 cacc = zero16();
    for (int fc = 0; fc < nfc; ++fc) cacc = mfma32(as_bf16x8(ld16(er + 16 * fc)), rf[fc], cacc);
    store_curve(cacc, cs + ln * CST + 32 * half + 4 * lh);
  }
}

// Bytes of the staged E for the curve MFMA.
__host__ __device__ inline int et_bytes(int bias_range, int R) {
  return (bias_range + 2 * PADE) * 16 * ((R + 7) / 8) * 2;
}
// Row stride (bf16) of E staged curve-major for the dr MFMA, and its bytes.
__host__ __device__ inline int ef_stride(int bias_range) { return (bias_range + 2 * PADE + 7) & ~7; }
__host__ __device__ inline int ef_bytes(int bias_range, int R) { return R * ef_stride(bias_range) * 2; }

// ---- pre pass: rowsum(dO * O) and zeroed parameter gradients ----------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, float* zero_ptr, long long n_zero) {
  const long long nrows = static_cast<long long>(a.B) * a.S * a.Hq;
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; idx < nrows; idx += stride) {
    // idx = (b * S + i) * Hq + h: consecutive threads read consecutive rows
    const uint16_t* op = a.o + idx * D;
    const uint16_t* dp = a.dout + idx * D;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 x = ld16(op + 8 * c);
      const u32x4 y = ld16(dp + 8 * c);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = fmaf(__uint_as_float(x[w] << 16), __uint_as_float(y[w] << 16), acc);
        acc = fmaf(__uint_as_float(x[w] & 0xffff0000u), __uint_as_float(y[w] & 0xffff0000u), acc);
      }
    }
    const long long h = idx % a.Hq;
    const long long bi = idx / a.Hq;
    const long long b = bi / a.S;
    const long long i = bi - b * a.S;
    a.dsum[(b * a.Hq + h) * a.S + i] = acc;
  }
  for (long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; idx < n_zero; idx += stride)
    zero_ptr[idx] = 0.f;
}

// ---- dq (+ dr, dE, dtable): query-parallel -----------------------------------------------------
// LDS: K, V, K^T tiles; per wave the curve scratch (r.E) and the skewed dZ buffers; the table
// row (table mode); E staged for the curve and dr MFMAs when ESTAGE.
template <int D, int MODE>
struct DqLayout {
  static constexpr int KST = D + 8;
  static constexpr int TST = BN + 8;
  static constexpr int TILE_BYTES = (2 * BN * KST + D * TST) * 2;
  static constexpr int CS_BYTES = (MODE == 2) ? 32 * CST * 4 : 0;
  static constexpr int G_BYTES = (MODE == 2) ? 32 * GST * 2 : 0;
  static constexpr int GT_BYTES = (MODE != 0) ? 64 * GTS * 2 : 0;
  static constexpr int WAVE_BYTES = CS_BYTES + G_BYTES + GT_BYTES;
  static constexpr int FIXED = TILE_BYTES + DQ_WAVES * WAVE_BYTES;
  static int bytes(int Rb, int R, bool estage) {
    int n = FIXED;
    if (MODE == 1) n += (Rb + 2 * PADT) * 4;
    if (MODE == 2 && estage) n += et_bytes(Rb, R) + ef_bytes(Rb, R);
    return n;
  }
};

template <int D, int MODE, bool ESTAGE>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a, int n_qtiles, int longest_first) {
  using L = DqLayout<D, MODE>;
  constexpr int KST = L::KST;
  constexpr int TST = L::TST;
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vs = Ks + BN * KST;
  uint16_t* Kt = Vs + BN * KST;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31;
  const int lh = lane >> 5;

  unsigned char* wsp = smem + L::TILE_BYTES + wave * L::WAVE_BYTES;
  float* cs = reinterpret_cast<float*>(wsp);
  uint16_t* Gs = reinterpret_cast<uint16_t*>(wsp + L::CS_BYTES);
  uint16_t* GTs = reinterpret_cast<uint16_t*>(wsp + L::CS_BYTES + L::G_BYTES);
  float* tabs = reinterpret_cast<float*>(smem + L::FIXED);                 // table mode
  uint16_t* et = reinterpret_cast<uint16_t*>(smem + L::FIXED);             // r.E, ESTAGE
  uint16_t* ef = et + et_bytes(a.bias_range, a.R) / 2;

  const int per_q = a.Hq * a.B;
  int qt = blockIdx.x / per_q;
  const int rem = blockIdx.x - qt * per_q;
  const int h = rem % a.Hq;
  const int b = rem / a.Hq;
  if (longest_first) qt = n_qtiles - 1 - qt;

  const int S = a.S;
  const int W = a.window;
  const int Rb = a.bias_range;
  const int wg_i0 = qt * (32 * DQ_WAVES);
  const int i0 = wg_i0 + 32 * wave;
  const bool wave_live = i0 < S;
  const int hkv = h / a.G;
  const int row = i0 + ln;
  const bool row_ok = row < S;
  const int nfc = (a.R + 7) / 8;

  const int wg_last = min(S, wg_i0 + 32 * DQ_WAVES) - 1;
  const int kmin = W ? max(0, wg_i0 - W + 1) : 0;
  const int t_begin = kmin / BN;
  const int t_end = wg_last / BN;

  const size_t q_row = static_cast<size_t>(a.Hq) * D;
  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const uint16_t* kbase = a.k + static_cast<size_t>(b) * S * kv_row + static_cast<size_t>(hkv) * D;
  const uint16_t* vbase = a.v + static_cast<size_t>(b) * S * kv_row + static_cast<size_t>(hkv) * D;
  const size_t qoff = (static_cast<size_t>(b) * S + (row_ok ? row : 0)) * q_row + static_cast<size_t>(h) * D;
  const float* Eh = (MODE == 2) ? a.E + static_cast<size_t>(h) * a.e_hs : nullptr;

  // bias parameters of the head in LDS (made visible by the first barrier of the tile loop)
  if (MODE == 1) {
    const float* tp = a.table + static_cast<size_t>(h) * Rb;
    for (int x = tid; x < Rb + 2 * PADT; x += 256) {
      const int d = x - PADT;
      tabs[x] = (d >= 0 && d < Rb) ? tp[d] * kLog2e : 0.f;
    }
  }
  if (MODE == 2 && ESTAGE) {
    stage_et(a, Eh, et, nfc, tid, 256);
    const int efs = ef_stride(Rb);
    for (int x = tid; x < a.R * efs; x += 256) {
      const int f = x / efs;
      const int d = x - f * efs - PADE;
      ef[x] = (d >= 0 && d < Rb) ? f32_to_bf16(Eh[static_cast<size_t>(f) * Rb + d]) : static_cast<uint16_t>(0);
    }
  }

  // Q^T and dO^T fragments (B operands): lane (n = ln, lh) holds x[row][16c + 8lh .. +7]
  bf16x8 qf[NC], dof[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (row_ok) {
      x = ld16(a.q + qoff + 16 * c + 8 * lh);
      y = ld16(a.dout + qoff + 16 * c + 8 * lh);
    }
    qf[c] = as_bf16x8(x);
    dof[c] = as_bf16x8(y);
  }
  // per-row scalars: lse (log2 units; +inf past the end makes P = 0), rowsum, temperature
  const size_t lrow = (static_cast<size_t>(b) * a.Hq + h) * S + (row_ok ? row : 0);
  const float lse2 = row_ok ? a.lse[lrow] * kLog2e : INFINITY;
  const float dsum = row_ok ? a.dsum[lrow] : 0.f;
  const float tq = temp_factor(visible_keys(row, W), a.temp_len, a.temp_inv_log2);
  const float cq = a.c_qk * tq;

  bf16x8 rf[2];        // r of this row (curve MFMA, B operand)
  bf16x8 rA[2];        // r^T of the wave's rows (dE MFMA, A operand): row f = ln, rows 16kk + 8lh + e
  if (MODE == 2) load_rf(a, b, row, h, rf);
  if (MODE != 0) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint32_t pr[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int rr = i0 + 16 * kk + 8 * lh + 2 * jj + u;
          uint32_t x = 0u;
          if (rr < S) {
            if (MODE == 1) x = (ln == 0) ? 0x3f80u : 0u;   // bf16 1.0
            else if (ln < a.R) x = a.r[((static_cast<size_t>(b) * S + rr) * a.Hq + h) * a.R + ln];
          }
          pr[u] = x;
        }
        w[jj] = pr[0] | (pr[1] << 16);
      }
      rA[kk] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
    }
    // zero the skewed buffers once: every in-band block writes the same set of positions
    for (int x = lane; x < (L::G_BYTES + L::GT_BYTES) / 16; x += 64)
      st16(reinterpret_cast<unsigned char*>(Gs) + 16 * x, u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = zero16();
  f32x16 dracc = zero16();
  float* dEh = (MODE == 2) ? a.dE + static_cast<size_t>(h) * a.e_hs : nullptr;
  float* dtab = (MODE == 1) ? a.dtable + static_cast<size_t>(h) * Rb : nullptr;

  // K / V tiles: the next tile's rows are loaded into registers while the current one is used
  constexpr int KIT = (row_items<D>() + 255) / 256;
  constexpr int NCH = BN * (D / 8);
  constexpr int VIT = (NCH + 255) / 256;
  u32x4 kpre[KIT][4], vpre[VIT];
  auto load_kv = [&](int tk0) {
    load_rows<D, KIT>(kbase, kv_row, tk0, S, kpre, tid, 256);
#pragma unroll
    for (int q = 0; q < VIT; ++q) {
      const int x = tid + 256 * q;
      const int rr = x / (D / 8);
      const int ch = x % (D / 8);
      vpre[q] = u32x4{0u, 0u, 0u, 0u};
      if (x < NCH && tk0 + rr < S) vpre[q] = ld16(vbase + static_cast<size_t>(tk0 + rr) * kv_row + 8 * ch);
    }
  };
  auto store_kv = [&]() {
    store_rows<D, KIT>(kpre, Ks, Kt, tid, 256);
#pragma unroll
    for (int q = 0; q < VIT; ++q) {
      const int x = tid + 256 * q;
      if (x < NCH) st16(Vs + (x / (D / 8)) * KST + 8 * (x % (D / 8)), vpre[q]);
    }
  };
  if (t_begin <= t_end) load_kv(t_begin * BN);

  for (int t = t_begin; t <= t_end; ++t) {
    const int tk0 = t * BN;
    __syncthreads();   // the previous tile's LDS reads are complete
    store_kv();
    __syncthreads();
    if (t < t_end) load_kv(tk0 + BN);
    if (!wave_live) continue;

#pragma unroll 1
    for (int kb = 0; kb < 2; ++kb) {
      const int kb0 = tk0 + 32 * kb;
      const int c = i0 - kb0;                    // delta = c + n - m
      bool on = (c + 31 >= 0) && (kb0 < S);
      if (W) on = on && (c - 31 < W);
      if (!on) continue;

      // operands read one step ahead of the MFMAs that use them
      f32x16 sacc = zero16(), pacc = zero16();
      const uint16_t* kr = Ks + (32 * kb + ln) * KST + 8 * lh;
      const uint16_t* vr = Vs + (32 * kb + ln) * KST + 8 * lh;
      bf16x8 kf = as_bf16x8(ld16(kr)), vf = as_bf16x8(ld16(vr));
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        bf16x8 kn = kf, vn = vf;
        if (cc + 1 < NC) {
          kn = as_bf16x8(ld16(kr + 16 * (cc + 1)));
          vn = as_bf16x8(ld16(vr + 16 * (cc + 1)));
        }
        sacc = mfma32(kf, qf[cc], sacc);
        pacc = mfma32(vf, dof[cc], pacc);
        kf = kn;
        vf = vn;
      }
      // log2-domain logits tau * (scale log2(e) q.k + log2(e) beta)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] *= cq;
      const bool inband = (MODE != 0) && (c - 31 < Rb);
      if (MODE == 1 && inband) {
        // distances c + ln - m lie in [-31, Rb + 62]: inside the zero-padded row
        const float* tb = tabs + PADT + c + ln;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = fmaf(tb[-out_row(i, lh)], tq, sacc[i]);
      }
      if (MODE == 2 && inband) {
        if (ESTAGE) curve_block_lds(et, nfc, rf, c - 31, cs, ln, lh);
        else curve_block<D>(a, Eh, rf, c - 31, cs, ln, lh);
        wave_sync_lds();
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = fmaf(cs[ln * CST + (ln - out_row(i, lh) + 31)], tq, sacc[i]);
        wave_sync_lds();
      }
      // P and dS = P * (dP - rowsum); the temperature factor of dZ = tau dS is applied to the
      // accumulated dq and to the bias-gradient inputs
      float dz[16];
      const bool edge = (c - 31 < 0) || (W && c + 31 >= W);
      if (edge) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = c + ln - out_row(i, lh);
          const bool vis = (d >= 0) & ((W == 0) | (d < W));
          const float p = fast_exp2(sacc[i] - lse2);
          dz[i] = (vis ? p : 0.f) * (pacc[i] - dsum);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) dz[i] = fast_exp2(sacc[i] - lse2) * (pacc[i] - dsum);
      }
      bf16x8 dzf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t w[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) w[jj] = pack_bf16x2(dz[8 * kk + 2 * jj], dz[8 * kk + 2 * jj + 1]);
        dzf[kk] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
      }
      // dQ^T += K^T dS^T
      {
        const uint16_t* ktr = Kt + ln * TST + 32 * kb + 8 * lh;
        bf16x8 kt = as_bf16x8(ld16(ktr));
#pragma unroll
        for (int x = 0; x < 2 * NDB; ++x) {
          bf16x8 kn = kt;
          if (x + 1 < 2 * NDB) kn = as_bf16x8(ld16(ktr + 32 * ((x + 1) >> 1) * TST + 16 * ((x + 1) & 1)));
          dqacc[x >> 1] = mfma32(kt, dzf[x & 1], dqacc[x >> 1]);
          kt = kn;
        }
      }

      if (MODE != 0 && inband) {
        // skewed dZ: G^T[dist][query] (and G[query][dist]) with dist = n - m + 32 over the
        // window c - 32 .. c + 31
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int dp = ln - out_row(i, lh) + 32;
          const uint16_t v16 = f32_to_bf16(dz[i] * tq);
          GTs[dp * GTS + ln] = v16;
          if (MODE == 2) Gs[ln * GST + dp] = v16;
        }
        wave_sync_lds();
        // dE (dtable): D[f][dist] = sum_i r^T[f][i] G[i][dist], 32 distances per MFMA pair
#pragma unroll
        for (int dbp = 0; dbp < 2; ++dbp) {
          f32x16 acc = zero16();
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 gt = as_bf16x8(ld16(GTs + (32 * dbp + ln) * GTS + 16 * kk + 8 * lh));
            acc = mfma32(rA[kk], gt, acc);
          }
          const int dist = c - 32 + 32 * dbp + ln;
          if (dist >= 0 && dist < Rb) {
            if (MODE == 1) {
              if (lh == 0) atomicAdd(dtab + dist, acc[0]);
            } else {
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                const int f = out_row(i, lh);
                if (f < a.R) atomicAdd(dEh + static_cast<size_t>(f) * Rb + dist, acc[i]);
              }
            }
          }
        }
        if (MODE == 2) {
          // dr^T[f][query] += sum_dist E[f][dist] G^T[dist][query], 16 distances per MFMA
          const int efs = ef_stride(Rb);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int d0 = c - 32 + 16 * kk + 8 * lh;
            bf16x8 ea;
            if (ESTAGE) {
              u32x4 x = {0u, 0u, 0u, 0u};
              if (ln < a.R) x = ld16(ef + ln * efs + PADE + d0);
              ea = as_bf16x8(x);
            } else {
              uint32_t w[4];
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                float e2[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                  const int dd = d0 + 2 * jj + u;
                  e2[u] = (ln < a.R && dd >= 0 && dd < Rb) ? Eh[static_cast<size_t>(ln) * Rb + dd] : 0.f;
                }
                w[jj] = pack_bf16x2(e2[0], e2[1]);
              }
              ea = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
            }
            const bf16x8 gf = as_bf16x8(ld16(Gs + ln * GST + 16 * kk + 8 * lh));
            dracc = mfma32(ea, gf, dracc);
          }
        }
        wave_sync_lds();
      }
    }
  }

  if (!wave_live || !row_ok) return;
  uint16_t* dqp = a.dq + qoff;
  const float sq = a.scale * tq;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * db + 8 * g4 + 4 * lh;
      const f32x16& acc = dqacc[db];
      st8(dqp + d, u32x2{pack_bf16x2(acc[4 * g4] * sq, acc[4 * g4 + 1] * sq),
                         pack_bf16x2(acc[4 * g4 + 2] * sq, acc[4 * g4 + 3] * sq)});
    }
  if (MODE == 2) {
    uint16_t* drp = a.dr + ((static_cast<size_t>(b) * S + row) * a.Hq + h) * a.R;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int f = out_row(i, lh);
      if (f < a.R) drp[f] = f32_to_bf16(dracc[i]);
    }
  }
}

// ---- dk, dv: key-parallel ------------------------------------------------------------------------
template <int D>
struct DkvLayout {
  static constexpr int TILES = (2 * BN * (D + 8) + 2 * D * (BN + 8)) * 2 + 4 * BN * 4 + BN * 16 * 2;
  static constexpr int CS_BYTES = DKV_WAVES * 32 * CST * 4;
  // bias parameters after the tiles: table row, or curve scratch (+ staged E)
  static int bytes(int mode, int Rb, int R, bool estage) {
    int n = TILES;
    if (mode == 1) n += (Rb + 2 * PADT) * 4;
    if (mode == 2) n += CS_BYTES + (estage ? et_bytes(Rb, R) : 0);
    return n;
  }
};

template <int D, int MODE, bool ESTAGE>
__global__ __launch_bounds__(64 * DKV_WAVES, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using L = DkvLayout<D>;
  constexpr int QST = D + 8;
  constexpr int TST = BN + 8;
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NT = 64 * DKV_WAVES;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Qs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* dOs = Qs + BN * QST;
  uint16_t* Qt = dOs + BN * QST;
  uint16_t* dOt = Qt + D * TST;
  float* rowp = reinterpret_cast<float*>(dOt + D * TST);   // [4][BN]: lse2, rowsum, c_qk*tau, tau
  uint16_t* rrow = reinterpret_cast<uint16_t*>(rowp + 4 * BN);   // [BN][16]: r of the tile's rows
  float* tabs = reinterpret_cast<float*>(smem + L::TILES);  // table mode: [PADT + Rb + PADT]
  float* cs_all = reinterpret_cast<float*>(smem + L::TILES);
  uint16_t* et = reinterpret_cast<uint16_t*>(smem + L::TILES + L::CS_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31;
  const int lh = lane >> 5;
  float* cs = cs_all + wave * 32 * CST;

  const int per_k = a.Hkv * a.B;
  const int kt = blockIdx.x / per_k;
  const int rem = blockIdx.x - kt * per_k;
  const int hkv = rem % a.Hkv;
  const int b = rem / a.Hkv;

  const int S = a.S;
  const int W = a.window;
  const int Rb = a.bias_range;
  const int j_lo = kt * (32 * DKV_WAVES);
  const int j0w = j_lo + 32 * wave;
  const bool wave_live = j0w < S;
  const int key = j0w + ln;
  const bool key_ok = key < S;
  const int nfc = (a.R + 7) / 8;

  const size_t q_row = static_cast<size_t>(a.Hq) * D;
  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const size_t koff = (static_cast<size_t>(b) * S + (key_ok ? key : 0)) * kv_row + static_cast<size_t>(hkv) * D;

  // K^T and V^T fragments (B operands): lane (n = ln, lh) holds x[key][16c + 8lh .. +7]
  bf16x8 kf[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (key_ok) {
      x = ld16(a.k + koff + 16 * c + 8 * lh);
      y = ld16(a.v + koff + 16 * c + 8 * lh);
    }
    kf[c] = as_bf16x8(x);
    vf[c] = as_bf16x8(y);
  }
  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkacc[db] = zero16();
    dvacc[db] = zero16();
  }

  const int last_key = min(S, j_lo + 32 * DKV_WAVES) - 1;
  const int i_last = W ? min(S - 1, last_key + W - 1) : S - 1;
  const int t_begin = j_lo / BN;
  const int t_end = i_last / BN;

  // (head, query tile) steps in one sequence, so the next step's Q / dO rows and per-row
  // values are loaded into registers while the current step is used
  const int ntiles = t_end - t_begin + 1;
  const int nsteps = ntiles > 0 ? a.G * ntiles : 0;
  constexpr int QIT = (row_items<D>() + NT - 1) / NT;
  u32x4 qpre[QIT][4], dpre[QIT][4];
  float lpre = 0.f, spre = 0.f, tpre = 1.f;
  u32x4 rpre[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
  auto load_step = [&](int st) {
    const int h = hkv * a.G + st / ntiles;
    const int qt0 = (t_begin + st % ntiles) * BN;
    load_rows<D, QIT>(a.q + static_cast<size_t>(b) * S * q_row + static_cast<size_t>(h) * D, q_row, qt0, S,
                      qpre, tid, NT);
    load_rows<D, QIT>(a.dout + static_cast<size_t>(b) * S * q_row + static_cast<size_t>(h) * D, q_row, qt0, S,
                      dpre, tid, NT);
    if (tid < BN) {
      const int rr = qt0 + tid;
      const bool ok = rr < S;
      const size_t lrow = (static_cast<size_t>(b) * a.Hq + h) * S + (ok ? rr : 0);
      lpre = ok ? a.lse[lrow] * kLog2e : INFINITY;
      spre = ok ? a.dsum[lrow] : 0.f;
      tpre = temp_factor(visible_keys(rr, W), a.temp_len, a.temp_inv_log2);
      if (MODE == 2) {   // r of the row, zero past R (16 curves at most)
        const uint16_t* rp = a.r + ((static_cast<size_t>(b) * S + (ok ? rr : 0)) * a.Hq + h) * a.R;
        uint32_t w[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const uint32_t lo = (ok && 2 * jj < a.R) ? rp[2 * jj] : 0u;
          const uint32_t hi = (ok && 2 * jj + 1 < a.R) ? rp[2 * jj + 1] : 0u;
          w[jj] = lo | (hi << 16);
        }
        rpre[0] = u32x4{w[0], w[1], w[2], w[3]};
        rpre[1] = u32x4{w[4], w[5], w[6], w[7]};
      }
    }
  };
  if (nsteps > 0) load_step(0);

  for (int st = 0; st < nsteps; ++st) {
    const int hh = st / ntiles;
    const int h = hkv * a.G + hh;
    const int qt0 = (t_begin + st % ntiles) * BN;
    const float* Eh = (MODE == 2) ? a.E + static_cast<size_t>(h) * a.e_hs : nullptr;
    __syncthreads();   // the previous step's LDS reads are complete
    store_rows<D, QIT>(qpre, Qs, Qt, tid, NT);
    store_rows<D, QIT>(dpre, dOs, dOt, tid, NT);
    if (tid < BN) {
      rowp[tid] = lpre;
      rowp[BN + tid] = spre;
      rowp[2 * BN + tid] = a.c_qk * tpre;
      rowp[3 * BN + tid] = tpre;
      if (MODE == 2) {
        st16(rrow + 16 * tid, rpre[0]);
        st16(rrow + 16 * tid + 8, rpre[1]);
      }
    }
    if (st % ntiles == 0) {   // a new head: its bias parameters
      if (MODE == 1) {
        const float* tp = a.table + static_cast<size_t>(h) * Rb;
        for (int x = tid; x < Rb + 2 * PADT; x += NT) {
          const int d = x - PADT;
          tabs[x] = (d >= 0 && d < Rb) ? tp[d] * kLog2e : 0.f;
        }
      }
      if (MODE == 2 && ESTAGE && (hh == 0 || a.e_hs != 0)) stage_et(a, Eh, et, nfc, tid, NT);
    }
    __syncthreads();
    if (st + 1 < nsteps) load_step(st + 1);
    if (!wave_live) continue;

#pragma unroll 1
    for (int qb = 0; qb < 2; ++qb) {
      const int i0b = qt0 + 32 * qb;
      const int c = i0b - j0w;                  // delta = c + m - n
      bool on = (c + 31 >= 0) && (i0b < S);
      if (W) on = on && (c - 31 < W);
      if (!on) continue;

      // operands read one step ahead of the MFMAs that use them
      f32x16 sacc = zero16(), pacc = zero16();
      const uint16_t* qr = Qs + (32 * qb + ln) * QST + 8 * lh;
      const uint16_t* dr_ = dOs + (32 * qb + ln) * QST + 8 * lh;
      bf16x8 qa = as_bf16x8(ld16(qr)), da = as_bf16x8(ld16(dr_));
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        bf16x8 qn = qa, dn = da;
        if (cc + 1 < NC) {
          qn = as_bf16x8(ld16(qr + 16 * (cc + 1)));
          dn = as_bf16x8(ld16(dr_ + 16 * (cc + 1)));
        }
        sacc = mfma32(qa, kf[cc], sacc);
        pacc = mfma32(da, vf[cc], pacc);
        qa = qn;
        da = dn;
      }
      // bias (log2 units) per element, before the temperature
      const bool inband = (MODE != 0) && (c - 31 < Rb);
      float bias[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) bias[i] = 0.f;
      if (MODE == 1 && inband) {
        // distances c + m - ln lie in [-31, Rb + 62]: inside the zero-padded row
        const float* tb = tabs + PADT + c - ln;
#pragma unroll
        for (int i = 0; i < 16; ++i) bias[i] = tb[out_row(i, lh)];
      }
      if (MODE == 2 && inband) {
        const bf16x8 rf[2] = {as_bf16x8(ld16(rrow + 16 * (32 * qb + ln))),
                              as_bf16x8(ld16(rrow + 16 * (32 * qb + ln) + 8))};
        if (ESTAGE) curve_block_lds(et, nfc, rf, c - 31, cs, ln, lh);
        else curve_block<D>(a, Eh, rf, c - 31, cs, ln, lh);
        wave_sync_lds();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = out_row(i, lh);
          bias[i] = cs[m * CST + (m - ln + 31)];
        }
        wave_sync_lds();
      }
      // P into sacc, dZ = tau * P * (dP - rowsum) into pacc (in place); per row: lse (log2
      // units), rowsum, c_qk * tau and tau (tau = 1 without a temperature).  Interior and
      // edge blocks get separate loops so that no branch sits inside the element loop.
      const bool edge = (c - 31 < 0) || (W && c + 31 >= W);
      const int wlim = W ? W : 0x7fffffff;
      if (edge) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int m0 = 32 * qb + 8 * g4 + 4 * lh;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(rowp + m0);
          const f32x4 s4 = *reinterpret_cast<const f32x4*>(rowp + BN + m0);
          const f32x4 c4 = *reinterpret_cast<const f32x4*>(rowp + 2 * BN + m0);
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(rowp + 3 * BN + m0);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 4 * g4 + u;
            const int d = c + out_row(i, lh) - ln;
            const float p = fast_exp2(fmaf(bias[i], t4[u], fmaf(sacc[i], c4[u], -l4[u])));
            const float pm = ((d >= 0) & (d < wlim)) ? p : 0.f;
            pacc[i] = pm * (pacc[i] - s4[u]) * t4[u];
            sacc[i] = pm;
          }
        }
      } else {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int m0 = 32 * qb + 8 * g4 + 4 * lh;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(rowp + m0);
          const f32x4 s4 = *reinterpret_cast<const f32x4*>(rowp + BN + m0);
          const f32x4 c4 = *reinterpret_cast<const f32x4*>(rowp + 2 * BN + m0);
          const f32x4 t4 = *reinterpret_cast<const f32x4*>(rowp + 3 * BN + m0);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 4 * g4 + u;
            const float p = fast_exp2(fmaf(bias[i], t4[u], fmaf(sacc[i], c4[u], -l4[u])));
            pacc[i] = p * (pacc[i] - s4[u]) * t4[u];
            sacc[i] = p;
          }
        }
      }
      bf16x8 pf[2], dzf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t w[4], x[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          w[jj] = pack_bf16x2(sacc[8 * kk + 2 * jj], sacc[8 * kk + 2 * jj + 1]);
          x[jj] = pack_bf16x2(pacc[8 * kk + 2 * jj], pacc[8 * kk + 2 * jj + 1]);
        }
        pf[kk] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
        dzf[kk] = as_bf16x8(u32x4{x[0], x[1], x[2], x[3]});
      }
      // dV^T += dO^T P,  dK^T += Q^T dZ
      {
        const int off0 = ln * TST + 32 * qb + 8 * lh;
        bf16x8 oa = as_bf16x8(ld16(dOt + off0)), qt = as_bf16x8(ld16(Qt + off0));
#pragma unroll
        for (int x = 0; x < 2 * NDB; ++x) {
          bf16x8 on = oa, qn = qt;
          if (x + 1 < 2 * NDB) {
            const int off = off0 + 32 * ((x + 1) >> 1) * TST + 16 * ((x + 1) & 1);
            on = as_bf16x8(ld16(dOt + off));
            qn = as_bf16x8(ld16(Qt + off));
          }
          dvacc[x >> 1] = mfma32(oa, pf[x & 1], dvacc[x >> 1]);
          dkacc[x >> 1] = mfma32(qt, dzf[x & 1], dkacc[x >> 1]);
          oa = on;
          qt = qn;
        }
      }
    }
  }

  if (!wave_live || !key_ok) return;
  uint16_t* dkp = a.dk + koff;
  uint16_t* dvp = a.dv + koff;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = 32 * db + 8 * g4 + 4 * lh;
      const f32x16& ka = dkacc[db];
      const f32x16& va = dvacc[db];
      st8(dkp + d, u32x2{pack_bf16x2(ka[4 * g4] * a.scale, ka[4 * g4 + 1] * a.scale),
                         pack_bf16x2(ka[4 * g4 + 2] * a.scale, ka[4 * g4 + 3] * a.scale)});
      st8(dvp + d, u32x2{pack_bf16x2(va[4 * g4], va[4 * g4 + 1]),
                         pack_bf16x2(va[4 * g4 + 2], va[4 * g4 + 3])});
    }
}

constexpr int kMaxLds = 160 * 1024;

template <typename K>
hipError_t allow_lds(K* kernel, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int D, int MODE, bool ESTAGE>
hipError_t launch_dq(const BwdArgs& a, hipStream_t s) {
  const int n_qtiles = (a.S + 32 * DQ_WAVES - 1) / (32 * DQ_WAVES);
  const int longest_first = (a.window == 0 || a.window > 32 * DQ_WAVES) ? 1 : 0;
  const int lds = DqLayout<D, MODE>::bytes(a.bias_range, a.R, ESTAGE);
  hipError_t e = allow_lds(&bwd_dq_kernel<D, MODE, ESTAGE>, lds);
  if (e != hipSuccess) return e;
  const long long nq = static_cast<long long>(n_qtiles) * a.Hq * a.B;
  hipLaunchKernelGGL((bwd_dq_kernel<D, MODE, ESTAGE>), dim3(static_cast<unsigned>(nq)), dim3(64 * DQ_WAVES), lds, s,
                     a, n_qtiles, longest_first);
  return hipGetLastError();
}

template <int D, int MODE, bool ESTAGE>
hipError_t launch_dkdv(const BwdArgs& a, hipStream_t s) {
  const int lds = DkvLayout<D>::bytes(MODE, a.bias_range, a.R, ESTAGE);
  hipError_t e = allow_lds(&bwd_dkdv_kernel<D, MODE, ESTAGE>, lds);
  if (e != hipSuccess) return e;
  const int n_ktiles = (a.S + 32 * DKV_WAVES - 1) / (32 * DKV_WAVES);
  const long long nk = static_cast<long long>(n_ktiles) * a.Hkv * a.B;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, MODE, ESTAGE>), dim3(static_cast<unsigned>(nk)), dim3(64 * DKV_WAVES), lds, s,
                     a);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  // pre pass
  float* zero_ptr = nullptr;
  long long n_zero = 0;
  if (MODE == 1) {
    zero_ptr = a.dtable;
    n_zero = static_cast<long long>(a.Hq) * a.bias_range;
  } else if (MODE == 2) {
    zero_ptr = a.dE;
    n_zero = static_cast<long long>(a.e_hs ? a.Hq : 1) * a.R * a.bias_range;
  }
  const long long nrows = static_cast<long long>(a.B) * a.S * a.Hq;
  const long long want = (std::max(nrows, n_zero) + 255) / 256;
  const unsigned pre_grid = static_cast<unsigned>(std::min<long long>(std::max<long long>(want, 1), 8192));
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(pre_grid), dim3(256), 0, s, a, zero_ptr, n_zero);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // r.E: E staged in LDS where it fits beside the tiles
  const bool dq_stage = MODE == 2 && DqLayout<D, MODE>::bytes(a.bias_range, a.R, true) <= kMaxLds;
  const bool kv_stage = MODE == 2 && DkvLayout<D>::bytes(MODE, a.bias_range, a.R, true) <= kMaxLds;
  e = dq_stage ? launch_dq<D, MODE, true>(a, s) : launch_dq<D, MODE, false>(a, s);
  if (e != hipSuccess) return e;
  return kv_stage ? launch_dkdv<D, MODE, true>(a, s) : launch_dkdv<D, MODE, false>(a, s);
}

template <int D>
hipError_t launch_bwd_mode(const BwdArgs& a, int mode, hipStream_t s) {
  switch (mode) {
    case 0: return launch_bwd<D, 0>(a, s);
    case 1: return launch_bwd<D, 1>(a, s);
    default: return launch_bwd<D, 2>(a, s);
  }
}

}  // namespace

// LDS the backward kernels need for this shape (the larger of the two, E read from global
// memory), or -1 past 160 KB.
int bwd_lds_bytes(int D, int mode, int bias_range) {
  int dq = 0, kv = 0;
  if (D == 128) {
    dq = mode == 0 ? DqLayout<128, 0>::bytes(bias_range, 1, false)
                   : (mode == 1 ? DqLayout<128, 1>::bytes(bias_range, 1, false) : DqLayout<128, 2>::bytes(bias_range, 1, false));
    kv = DkvLayout<128>::bytes(mode, bias_range, 1, false);
  } else {
    dq = mode == 0 ? DqLayout<64, 0>::bytes(bias_range, 1, false)
                   : (mode == 1 ? DqLayout<64, 1>::bytes(bias_range, 1, false) : DqLayout<64, 2>::bytes(bias_range, 1, false));
    kv = DkvLayout<64>::bytes(mode, bias_range, 1, false);
  }
  const int m = std::max(dq, kv);
  return m > kMaxLds ? -1 : m;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int D, int mode, hipStream_t s) {
  if (a.B == 0 || a.S == 0) return hipSuccess;
  if (D == 128) return launch_bwd_mode<128>(a, mode, s);
  return launch_bwd_mode<64>(a, mode, s);
}

}  // namespace rba
