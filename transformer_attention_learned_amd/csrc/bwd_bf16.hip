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
// Kernels on one stream:
//   * bwd_pre: rowsum(dO * O) per (batch, head, row) into the workspace, and zero dE / dtable.
//   * bwd_curves (input-dependent bias only): the curve table C[b, h, i, d] = r_i . E[h, :, d]
//     for every row and distance d < bias_range, bf16, with zero distances on both sides of a
//     row, in the workspace.  The two main kernels read the bias from it instead of forming
//     the curves again block by block (the forward forms them once, the backward would form
//     them twice); for the local layer it is 2 * 32 * 4096 rows of 608 bf16, about 320 MB.
//   * bwd_dq: one workgroup = 4 waves x 32 query rows of one head (the forward's transposed
//     layout: S^T = K Q^T, so each lane owns one query row and its lse, rowsum and temperature
//     are scalars).  Per 32 x 32 block it recomputes S^T and dP^T = V dO^T, forms dZ^T and
//     accumulates dQ^T += K^T dZ^T (K^T in LDS with the key permutation of the forward's V^T).
//     A lane's 16 bias values sit at 4 runs of 4 consecutive distances of its own curve row:
//     four 8-byte loads.  In-band blocks also write dZ into two wave-private skewed buffers,
//     G[query][distance] and its transpose, over the block's 64-distance window; then
//       dr^T += E G^T            (one MFMA per 16 distances; E staged in LDS, curve-major)
//       dE   += r^T G  per 32 distances (A = r^T, held in registers for the wave's rows),
//     and the dE / dtable block goes to global memory with fp32 atomics: each instruction
//     adds 32 consecutive distances of one curve, two cache lines.  dtable uses the same MFMA
//     with r replaced by a ones row.
//   * bwd_dkdv: one workgroup = 4 waves x 32 keys of one kv head, looping over the group's
//     query heads and the query tiles that see its keys.  Untransposed layout S = Q K^T (each
//     lane owns one key), K and V held in registers as B operands; Q, dO and their transposes
//     in LDS; per-row lse, rowsum and temperature from LDS.  dV^T += dO^T P and dK^T += Q^T dZ
//     take P and dZ straight from the registers the score MFMAs left them in.  The bias comes
//     from the table row staged in LDS, or from the curve table (one 2-byte load per element,
//     issued before the score MFMAs).

#include <algorithm>

#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

constexpr int BN = 64;        // keys per tile (dq kernel), query rows per tile (dk/dv kernel)
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

// Row of the curve table: CPAD_L zero distances, the bias_range curve values, CPAD_R zeros.
constexpr int CPAD_L = 32;
constexpr int CPAD_R = 64;

// ---- curve table: C[b, h, i, d] = sum_f r[b, i, h, f] E[h, f, d] ---------------------------------
// One workgroup per (batch, head, 64 rows): E[h] staged in LDS (fp32) in the table's own column
// layout (zero outside [0, bias_range)), and the rows' r; a thread holds the E values of 8
// consecutive columns (RM curves, RM >= R) in registers and writes those columns for every
// (256 / chunks)-th row: one 16-byte store per row, the row's r read from LDS.
template <int RM>
__global__ __launch_bounds__(256) void bwd_curves_kernel(BwdArgs a, int pitch) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* es = reinterpret_cast<float*>(smem);                  // [R][pitch]
  float* rsh = es + a.R * pitch;                               // [64][R]
  const int Rb = a.bias_range;
  const int ntile = (a.S + 63) / 64;
  const int tile = blockIdx.x % ntile;
  const int bh = blockIdx.x / ntile;                           // b * Hq + h
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int i0 = tile * 64;
  const float* Eh = a.E + static_cast<size_t>(h) * a.e_hs;
  for (int x = threadIdx.x; x < a.R * pitch; x += 256) {
    const int f = x / pitch;
    const int d = x - f * pitch - CPAD_L;
    es[x] = (d >= 0 && d < Rb) ? Eh[static_cast<size_t>(f) * Rb + d] : 0.f;
  }
  for (int x = threadIdx.x; x < 64 * a.R; x += 256) {
    const int rr = x / a.R;
    const int f = x - rr * a.R;
    const int i = i0 + rr;
    rsh[x] = i < a.S ? bf16_to_f32(a.r[((static_cast<size_t>(b) * a.S + i) * a.Hq + h) * a.R + f]) : 0.f;
  }
  __syncthreads();
  // thread -> (column chunk, row phase): the chunk's E values (R x 8) stay in registers and the
  // rows are walked with a stride of the phase count, so each 16-byte store costs two LDS reads
  // (the row's r) instead of two per curve
  const int chunks = pitch / 8;
  const int rows = min(64, a.S - i0);
  const int cpt = min(chunks, 256);         // chunks side by side
  const int phases = 256 / cpt;             // rows side by side
  const int ph = threadIdx.x / cpt;
  if (ph >= phases) return;
  uint16_t* out = a.ctab + (static_cast<size_t>(bh) * a.S + i0) * pitch;
  for (int ch = threadIdx.x % cpt; ch < chunks; ch += cpt) {
    const int t0 = 8 * ch;
    f32x4 e0[RM], e1[RM];
#pragma unroll
    for (int f = 0; f < RM; ++f) {
      const bool fl = f < a.R;
      e0[f] = fl ? *reinterpret_cast<const f32x4*>(es + f * pitch + t0) : f32x4{0.f, 0.f, 0.f, 0.f};
      e1[f] = fl ? *reinterpret_cast<const f32x4*>(es + f * pitch + t0 + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int rr = ph; rr < rows; rr += phases) {
      f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < RM; ++f) {
        const float rv = f < a.R ? rsh[rr * a.R + f] : 0.f;
        v0 += rv * e0[f];
        v1 += rv * e1[f];
      }
      st16(out + static_cast<size_t>(rr) * pitch + t0,
           u32x4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v1[0], v1[1]),
                 pack_bf16x2(v1[2], v1[3])});
    }
  }
}

// ---- pre pass: rowsum(dO * O) and zeroed parameter gradients ----------------------------------
// 16 lanes per row (each lane 16 bytes of O and of dO for D = 128, 8 bytes for D = 64), so a
// wave reads 4 whole rows per load: coalesced 256-byte runs; a 16-lane sum finishes the row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, float* zero_ptr, long long n_zero) {
  constexpr int LPR = 16;          // lanes per row
  constexpr int EPL = D / LPR;     // elements per lane: 8 (D = 128) or 4 (D = 64)
  const long long nrows = static_cast<long long>(a.B) * a.S * a.Hq;
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  const int sub = threadIdx.x % LPR;
  const long long rstride = stride / LPR;
  // every lane of a 16-lane group walks the same rows, so the group's shuffles see live lanes
  for (long long idx = (static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x) / LPR; idx < nrows;
       idx += rstride) {
    // idx = (b * Hq + h) * S + i, the layout of the row sums: consecutive groups write
    // consecutive floats (and read rows Hq * D apart)
    const long long i = idx % a.S;
    const long long bh = idx / a.S;
    const long long h = bh % a.Hq;
    const long long b = bh / a.Hq;
    const long long row = (b * a.S + i) * a.Hq + h;
    const uint16_t* op = a.o + row * D + EPL * sub;
    const uint16_t* dp = a.dout + row * D + EPL * sub;
    float acc = 0.f;
    uint32_t x[EPL / 2], y[EPL / 2];
    if constexpr (EPL == 8) {
      const u32x4 xv = ld16(op), yv = ld16(dp);
#pragma unroll
      for (int w = 0; w < 4; ++w) { x[w] = xv[w]; y[w] = yv[w]; }
    } else {
      const u32x2 xv = ld8(op), yv = ld8(dp);
#pragma unroll
      for (int w = 0; w < 2; ++w) { x[w] = xv[w]; y[w] = yv[w]; }
    }
#pragma unroll
    for (int w = 0; w < EPL / 2; ++w) {
      acc = fmaf(__uint_as_float(x[w] << 16), __uint_as_float(y[w] << 16), acc);
      acc = fmaf(__uint_as_float(x[w] & 0xffff0000u), __uint_as_float(y[w] & 0xffff0000u), acc);
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, LPR);
    if (sub == 0) a.dsum[idx] = acc;
  }
  for (long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; idx < n_zero; idx += stride)
    zero_ptr[idx] = 0.f;
}

// ---- dq (+ dr, dE, dtable): query-parallel -----------------------------------------------------
// LDS: K, V, K^T tiles; per wave the skewed dZ buffers; the table row (table mode) or E staged
// curve-major for the dr MFMA (r.E).
template <int D, int MODE>
struct DqLayout {
  static constexpr int KST = D + 8;
  static constexpr int TST = BN + 8;
  static constexpr int TILE_BYTES = (2 * BN * KST + D * TST) * 2;
  static constexpr int G_BYTES = (MODE == 2) ? 32 * GST * 2 : 0;
  static constexpr int GT_BYTES = (MODE != 0) ? 64 * GTS * 2 : 0;
  static constexpr int WAVE_BYTES = G_BYTES + GT_BYTES;
  static constexpr int FIXED = TILE_BYTES + DQ_WAVES * WAVE_BYTES;
  static int bytes(int Rb, int R) {
    int n = FIXED;
    if (MODE == 1) n += (Rb + 2 * PADT) * 4;
    if (MODE == 2) n += R * ef_stride(Rb) * 2;
    return n;
  }
  // Row stride (bf16) of E staged curve-major for the dr MFMA.
  __host__ __device__ static int ef_stride(int Rb) { return (Rb + 2 * PADE + 7) & ~7; }
};

template <int D, int MODE>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a, int n_qtiles, int longest_first, int pitch) {
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
  uint16_t* Gs = reinterpret_cast<uint16_t*>(wsp);
  uint16_t* GTs = reinterpret_cast<uint16_t*>(wsp + L::G_BYTES);
  float* tabs = reinterpret_cast<float*>(smem + L::FIXED);                 // table mode
  uint16_t* ef = reinterpret_cast<uint16_t*>(smem + L::FIXED);             // r.E

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
  // this lane's curve row (rows past the end read the last row; their P is zero)
  const uint16_t* crow = (MODE == 2)
      ? a.ctab + ((static_cast<size_t>(b) * a.Hq + h) * S + (row_ok ? row : S - 1)) * pitch + CPAD_L
      : nullptr;

  // bias parameters of the head in LDS (made visible by the first barrier of the tile loop)
  if (MODE == 1) {
    const float* tp = a.table + static_cast<size_t>(h) * Rb;
    for (int x = tid; x < Rb + 2 * PADT; x += 256) {
      const int d = x - PADT;
      tabs[x] = (d >= 0 && d < Rb) ? tp[d] * kLog2e : 0.f;
    }
  }
  const int efs = L::ef_stride(Rb);
  if (MODE == 2) {
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
  const float cb = kLog2e * tq;

  bf16x8 rA[2];        // r^T of the wave's rows (dE MFMA, A operand): row f = ln, rows 16kk + 8lh + e
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
      const bool inband = (MODE != 0) && (c - 31 < Rb);

      // r.E bias: distances c + ln - (8 g + 4 lh + u) of the lane's curve row, four runs of 4
      // (8-byte loads; the distances lie in [-31, Rb + 61], inside the padded row)
      u32x2 braw[4];
      if (MODE == 2 && inband) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 x;
          __builtin_memcpy(&x, crow + c + ln - 8 * g4 - 4 * lh - 3, 8);
          braw[g4] = x;
        }
      }

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
      if (MODE == 1 && inband) {
        // distances c + ln - m lie in [-31, Rb + 62]: inside the zero-padded row
        const float* tb = tabs + PADT + c + ln;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = fmaf(tb[-out_row(i, lh)], tq, sacc[i]);
      }
      if (MODE == 2 && inband) {
        // element u of run g4 is distance (start + 3 - u): the high half of word 1 for u = 0
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t w = braw[g4][(3 - u) >> 1];
            const float beta = __uint_as_float(((3 - u) & 1) ? (w & 0xffff0000u) : (w << 16));
            sacc[4 * g4 + u] = fmaf(beta, cb, sacc[4 * g4 + u]);
          }
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
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int d0 = c - 32 + 16 * kk + 8 * lh;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (ln < a.R) x = ld16(ef + ln * efs + PADE + d0);
            const bf16x8 gf = as_bf16x8(ld16(Gs + ln * GST + 16 * kk + 8 * lh));
            dracc = mfma32(as_bf16x8(x), gf, dracc);
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
  static constexpr int TILES = (2 * BN * (D + 8) + 2 * D * (BN + 8)) * 2 + 4 * BN * 4;
  static int bytes(int mode, int Rb) { return TILES + (mode == 1 ? (Rb + 2 * PADT) * 4 : 0); }
};

template <int D, int MODE>
__global__ __launch_bounds__(64 * DKV_WAVES, 1) void bwd_dkdv_kernel(BwdArgs a, int pitch) {
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
  float* tabs = reinterpret_cast<float*>(smem + L::TILES);  // table mode: [PADT + Rb + PADT]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31;
  const int lh = lane >> 5;

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
    }
  };
  if (nsteps > 0) load_step(0);

  for (int st = 0; st < nsteps; ++st) {
    const int hh = st / ntiles;
    const int h = hkv * a.G + hh;
    const int qt0 = (t_begin + st % ntiles) * BN;
    __syncthreads();   // the previous step's LDS reads are complete
    store_rows<D, QIT>(qpre, Qs, Qt, tid, NT);
    store_rows<D, QIT>(dpre, dOs, dOt, tid, NT);
    if (tid < BN) {
      rowp[tid] = lpre;
      rowp[BN + tid] = spre;
      rowp[2 * BN + tid] = a.c_qk * tpre;
      rowp[3 * BN + tid] = tpre;
    }
    if (MODE == 1 && st % ntiles == 0) {   // a new head: its table row, zero-padded
      const float* tp = a.table + static_cast<size_t>(h) * Rb;
      for (int x = tid; x < Rb + 2 * PADT; x += NT) {
        const int d = x - PADT;
        tabs[x] = (d >= 0 && d < Rb) ? tp[d] * kLog2e : 0.f;
      }
    }
    __syncthreads();
    if (st + 1 < nsteps) load_step(st + 1);
    if (!wave_live) continue;
    // curve rows of this step's queries (rows past the end read the last row; P is zero there)
    const uint16_t* cplane = (MODE == 2) ? a.ctab + (static_cast<size_t>(b) * a.Hq + h) * S * pitch + CPAD_L : nullptr;

#pragma unroll 1
    for (int qb = 0; qb < 2; ++qb) {
      const int i0b = qt0 + 32 * qb;
      const int c = i0b - j0w;                  // delta = c + m - n
      bool on = (c + 31 >= 0) && (i0b < S);
      if (W) on = on && (c - 31 < W);
      if (!on) continue;
      const bool inband = (MODE != 0) && (c - 31 < Rb);

      // r.E bias of element (query m, key ln): curve row i0b + m at distance c + m - ln, in
      // [-31, Rb + 61]; issued before the score MFMAs
      uint16_t braw[16];
      if (MODE == 2 && inband) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = out_row(i, lh);
          const int rr = min(i0b + m, S - 1);
          braw[i] = cplane[static_cast<size_t>(rr) * pitch + c + m - ln];
        }
      }

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
#pragma unroll
        for (int i = 0; i < 16; ++i) bias[i] = bf16_to_f32(braw[i]) * kLog2e;
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
  const long long want = (std::max(16 * nrows, n_zero) + 255) / 256;   // 16 lanes per row
  const unsigned pre_grid = static_cast<unsigned>(std::min<long long>(std::max<long long>(want, 1), 8192));
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(pre_grid), dim3(256), 0, s, a, zero_ptr, n_zero);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int pitch = bwd_curve_pitch(a.bias_range);
  if (MODE == 2) {
    const int lds = (a.R * pitch + 64 * a.R) * 4;
    const long long ng = static_cast<long long>(a.B) * a.Hq * ((a.S + 63) / 64);
    if (a.R > 8) {
      e = allow_lds(&bwd_curves_kernel<16>, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(bwd_curves_kernel<16>, dim3(static_cast<unsigned>(ng)), dim3(256), lds, s, a, pitch);
    } else {
      e = allow_lds(&bwd_curves_kernel<8>, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(bwd_curves_kernel<8>, dim3(static_cast<unsigned>(ng)), dim3(256), lds, s, a, pitch);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dq (+ bias-parameter gradients)
  const int n_qtiles = (a.S + 32 * DQ_WAVES - 1) / (32 * DQ_WAVES);
  const int longest_first = (a.window == 0 || a.window > 32 * DQ_WAVES) ? 1 : 0;
  const long long nq = static_cast<long long>(n_qtiles) * a.Hq * a.B;
  const int dq_lds = DqLayout<D, MODE>::bytes(a.bias_range, a.R);
  e = allow_lds(&bwd_dq_kernel<D, MODE>, dq_lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, MODE>), dim3(static_cast<unsigned>(nq)), dim3(64 * DQ_WAVES), dq_lds, s,
                     a, n_qtiles, longest_first, pitch);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dk, dv
  const int kv_lds = DkvLayout<D>::bytes(MODE, a.bias_range);
  e = allow_lds(&bwd_dkdv_kernel<D, MODE>, kv_lds);
  if (e != hipSuccess) return e;
  const int n_ktiles = (a.S + 32 * DKV_WAVES - 1) / (32 * DKV_WAVES);
  const long long nk = static_cast<long long>(n_ktiles) * a.Hkv * a.B;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, MODE>), dim3(static_cast<unsigned>(nk)), dim3(64 * DKV_WAVES), kv_lds, s,
                     a, pitch);
  return hipGetLastError();
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

int bwd_curve_pitch(int bias_range) { return (CPAD_L + bias_range + CPAD_R + 7) & ~7; }

// LDS the backward kernels need for this shape (the largest of the three), or -1 past 160 KB.
int bwd_lds_bytes(int D, int mode, int bias_range, int R) {
  int dq = 0, kv = 0;
  if (D == 128) {
    dq = mode == 0 ? DqLayout<128, 0>::bytes(bias_range, R)
                   : (mode == 1 ? DqLayout<128, 1>::bytes(bias_range, R) : DqLayout<128, 2>::bytes(bias_range, R));
    kv = DkvLayout<128>::bytes(mode, bias_range);
  } else {
    dq = mode == 0 ? DqLayout<64, 0>::bytes(bias_range, R)
                   : (mode == 1 ? DqLayout<64, 1>::bytes(bias_range, R) : DqLayout<64, 2>::bytes(bias_range, R));
    kv = DkvLayout<64>::bytes(mode, bias_range);
  }
  const int cv = mode == 2 ? (R * bwd_curve_pitch(bias_range) + 64 * R) * 4 : 0;
  const int m = std::max(std::max(dq, kv), cv);
  return m > kMaxLds ? -1 : m;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int D, int mode, hipStream_t s) {
  if (a.B == 0 || a.S == 0) return hipSuccess;
  if (D == 128) return launch_bwd_mode<128>(a, mode, s);
  return launch_bwd_mode<64>(a, mode, s);
}

}  // namespace rba
