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
//   * the input-dependent bias r_i . E[h, :, d] is formed inside both main kernels, block by
//     block, the way the forward forms it: E is converted once per call into the workspace as a
//     bf16 high and low part (the forward's conversion, at scale 1: about 16 mantissa bits,
//     heads x (bias_range + 129) rows, independent of the sequence length), and an in-band
//     32 x 32 block forms the curves of its 32 query rows over its 64 distances with MFMAs over
//     the features (fp32 results), writes them to a wave-private LDS buffer and reads its
//     diagonal back, so the bias reaches the recomputed logits with fp32 accuracy.
//   * both main kernels stream their 32-row tiles (K and V, or q and dout) through a 3-slot LDS
//     ring filled by direct-to-LDS loads two steps ahead, one barrier per step; the gradient
//     products read the tiles transposed (ds_read_b64_tr_b16), so no transposed copy is stored.
//   * bwd_dq: one workgroup = 4 waves x 32 query rows of one head (the forward's transposed
//     layout: S^T = K Q^T, so each lane owns one query row and its lse, rowsum and temperature
//     are scalars).  Per 32-key step it recomputes S^T and dP^T = V dO^T, forms dZ^T and
//     accumulates dQ^T += K^T dZ^T.
//     A lane's 16 bias values lie on its own query row's curve (the forward's skewed curve
//     buffer layout).  In-band blocks also write dZ into two wave-private skewed buffers,
//     G[query][distance] and its transpose, over the block's 64-distance window; then
//       dr^T += E G^T            (one MFMA per 16 distances; E staged in LDS, curve-major)
//       dE   += r^T G  per 32 distances (A = r^T, held in registers for the wave's rows),
//     and the dE / dtable block goes to global memory with fp32 atomics: each instruction
//     adds 32 consecutive distances of one curve, two cache lines.  dtable uses the same MFMA
//     with r replaced by a ones row.
//   * bwd_dkdv: one workgroup = 4 waves x 32 keys of one kv head, looping over the group's
//     query heads and the query tiles that see its keys.  Untransposed layout S = Q K^T (each
//     lane owns one key), K and V held in registers as B operands; per-row lse, rowsum and
//     temperature from LDS, beside the step's tiles.  dV^T += dO^T P and dK^T += Q^T dZ
//     take P and dZ straight from the registers the score MFMAs left them in.  The bias comes
//     from the table row staged in LDS, or from the block's curves (the B operand of their MFMA
//     is r of the block's 32 query rows; a lane reads its key's value from each of the 16 rows
//     it holds, 32 consecutive dwords per row and half-wave).

#include <algorithm>

#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

constexpr int PADT = 64;      // zero distances staged on each side of a table row
constexpr int PADE = 64;      // zero distances staged on each side of E
constexpr int GST = 64 + 8;   // G row stride (bf16): row = query, 64 distances
constexpr int GTS = 32 + 8;   // G^T row stride (bf16): row = distance, 32 queries
constexpr int DQ_WAVES = 4;
constexpr int DKV_WAVES = 4;

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

// ---- input-dependent bias, formed per 32 x 32 block (shared by the dq and dk/dv kernels) -------
// The E rows of a block come from the converted copy (kE2Pad zero distances on each side, EW =
// e2_width(R) entries per row: the high part of the features, then the low part).  A curve MFMA
// pairs lane half lh's 8 K-elements of A (E) with the same lane half of B (r), so with EW = 16
// lane half 0 carries hi * r and lane half 1 lo * r (B holds r[0..7] in both halves); with
// EW = 32 a first MFMA takes hi and a second lo, lane half lh carrying features 8 lh .. 8 lh + 7.
constexpr int CURVE_ROWS_DQ = 36;    // floats per query row, dq kernel (the forward's packed layout)
constexpr int CURVE_ROWS_KV = 40;    // floats per query row, dk/dv kernel
constexpr int CURVE_BYTES_DQ = 32 * CURVE_ROWS_DQ * 4;
constexpr int CURVE_BYTES_KV = 32 * CURVE_ROWS_KV * 4;

typedef __attribute__((address_space(3))) float lds_float;

// r fragment (B operand) of query row `row`: EW = 16: features 0..7 in both lane halves;
// EW = 32: features 8 lh .. 8 lh + 7; zero past R and for rows at or past S.
// Split into the loads and the packing, which masks the features past R and rows at or past S.
// With R = EW / 2 and r 16-byte aligned (rvec) a lane's 8 features are one 16-byte load, kept
// packed in pairs in x[0..3]; otherwise 8 two-byte loads, unconditional and inside the row (the
// feature index is clamped, so that no load sits in a branch of its own and is waited for
// before the next one is issued).
template <int EW>
__device__ __forceinline__ bool r_vec(const BwdArgs& a) {
  return a.R == EW / 2 && (reinterpret_cast<uintptr_t>(a.r) & 15) == 0;
}
// The two load forms keep separate storage: with one array written in either form the compiler
// placed it in scratch memory, and the store there waited for every load in flight.
struct RRaw {
  u32x4 v;          // the 16-byte form: features in pairs
  uint32_t s[8];    // the two-byte form: one feature each
};
template <int EW>
__device__ __forceinline__ void r_load(const BwdArgs& a, bool rvec, int b, int h, int row, int lh, RRaw& x) {
  const int f0 = (EW == 32) ? 8 * lh : 0;
  const uint16_t* rp = a.r + ((static_cast<size_t>(b) * a.S + (row < a.S ? row : 0)) * a.Hq + h) * a.R;
  if (rvec) {
    x.v = ld16(rp + f0);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x.s[e] = rp[min(f0 + e, a.R - 1)];
  }
}
template <int EW>
__device__ __forceinline__ bf16x8 r_pack(const BwdArgs& a, bool rvec, int row, int lh, const RRaw& x) {
  const int f0 = (EW == 32) ? 8 * lh : 0;
  uint32_t w[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    if (rvec) {
      w[jj] = row < a.S ? x.v[jj] : 0u;
    } else {
      const int f = f0 + 2 * jj;
      const uint32_t lo = (row < a.S && f < a.R) ? x.s[2 * jj] : 0u;
      const uint32_t hi = (row < a.S && f + 1 < a.R) ? x.s[2 * jj + 1] : 0u;
      w[jj] = lo | (hi << 16);
    }
  }
  return as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
}
template <int EW>
__device__ __forceinline__ bf16x8 r_frag(const BwdArgs& a, int b, int h, int row, int lh) {
  RRaw x;
  const bool rvec = r_vec<EW>(a);
  r_load<EW>(a, rvec, b, h, row, lh, x);
  return r_pack<EW>(a, rvec, row, lh, x);
}

// E rows of a block whose distances are c - 31 + l (block 0) and c + 1 + l (block 1) for the
// 32 lanes l; c lies in [-31, bias_range + 30] for every in-band block, so the rows read lie
// inside the padded rows.  e2h: the head's converted rows at distance 0.
template <int EW>
__device__ __forceinline__ void e_rows(const uint16_t* e2h, int c, int ln, int lh, u32x4 (&e)[2][EW / 16]) {
  const uint16_t* ep = e2h + (c - 31 + ln) * EW + 8 * lh;
#pragma unroll
  for (int u = 0; u < EW / 16; ++u) {
    e[0][u] = ld16(ep + 16 * u);
    e[1][u] = ld16(ep + 32 * EW + 16 * u);
  }
}

// The curves of the block's 32 query rows over its 64 distances, fp32: lane (n, lh) gets row n
// (the B operand's column) at t = 8 g + 4 lh + k (lo) and 32 + the same (hi), t = distance -
// (c - 31).
template <int EW>
__device__ __forceinline__ void curve_mfma(const u32x4 (&e)[2][EW / 16], const bf16x8& rf, f32x16& lo, f32x16& hi) {
  lo = mfma32(as_bf16x8(e[0][0]), rf, zero16());
  hi = mfma32(as_bf16x8(e[1][0]), rf, zero16());
#pragma unroll
  for (int u = 1; u < EW / 16; ++u) {
    lo = mfma32(as_bf16x8(e[0][u]), rf, lo);
    hi = mfma32(as_bf16x8(e[1][u]), rf, hi);
  }
}

// Writes of the curve chunks row n reads back (t = n .. n + 31): chunk u (t from 32 (u / 4) +
// 8 (u % 4) + 4 lh) is written iff it overlaps that range; row n's entry t goes to
// row_base + t - 4 (n / 4).  Per-lane constant predicates (exec masks, no branches).
__device__ __forceinline__ void curve_write(float* row_base, int n, int lh, const f32x16& lo, const f32x16& hi) {
  float* wp = row_base - 4 * (n >> 2) + 4 * lh;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int t0 = 8 * g + 4 * lh;
    if (__builtin_expect(t0 + 3 >= n, 1))
      st16(wp + 8 * g, __builtin_bit_cast(u32x4, f32x4{lo[4 * g], lo[4 * g + 1], lo[4 * g + 2], lo[4 * g + 3]}));
    if (__builtin_expect(t0 + 32 <= n + 31, 1))
      st16(wp + 32 + 8 * g, __builtin_bit_cast(u32x4, f32x4{hi[4 * g], hi[4 * g + 1], hi[4 * g + 2], hi[4 * g + 3]}));
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

// ---- tile ring shared by the dq and dk/dv kernels --------------------------------------------------
// Each step streams 32 rows of two bf16 tensors (K and V in the dq kernel, q and dout in the dk/dv
// kernel) straight from global memory into a 3-slot LDS ring: rows of 2 D bytes in 16-byte chunks,
// chunk index XOR-swizzled per row (tile_sw), each wave issuing its share of the 1 KB direct-load
// instructions.  The score products read tile rows (A operand, 16 bytes per lane), the gradient
// products read the tile transposed (ds_read_b64_tr_b16).
constexpr int TROWS = 32;   // rows per step
constexpr int NBUF = 3;     // ring slots

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

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

// XOR applied to the 16-byte chunk index of tile row r.  Row reads (16 lanes, rows r .. r + 15
// at one logical chunk) need distinct values over any 16 consecutive rows; a transposing read
// (16 lanes, 4 rows x 32 bytes: rows 4 k .. 4 k + 3, logical chunks 2 m, 2 m + 1) needs the four
// rows' values to differ above bit 0.  D = 128 (256-byte rows, one row spans the 64 banks): row
// bits 0-1 to chunk bits 2-3, bits 2-3 to bits 0-1.  D = 64 (128-byte rows, two rows per bank
// line, row bit 0 selecting the half): row bit 1 to chunk bit 2, bits 2-3 to bits 0-1.
template <int D>
__device__ __forceinline__ int tile_sw(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Per-lane addresses within a tile.  Direct loads: instruction k of wave w fills rows
// RPI (NIT w + k) .. + RPI - 1 (RPI = 1024 / (2 D) rows per instruction); voff is the lane's byte
// offset in global memory (row stride row_b).  Row reads: lane ln reads row ln, logical chunk
// 2 c + lh.  Transposing reads of 16 rows x 32 columns (the A operand of a gradient product over
// 16 rows): lane (ln = column within 32, lh) gets rows 4 lh .. 4 lh + 3 from its "lo" read and 8 +
// the same from its "hi" read (16 more rows at + 16 rows), the row order in which a 32x32 MFMA
// output lane half holds its rows, so the product's B operand is the output packed as it is.
template <int D, int NIT>
struct TileAddr {
  static constexpr int ROW_B = 2 * D;
  static constexpr int CPR = ROW_B / 16;
  static constexpr int RPI = 64 / CPR;
  int voff[NIT];
  int raddr[D / 16];
  int taddr[2][D / 32];
  __device__ __forceinline__ TileAddr(int lane, int wave, int row_b) {
    const int ln = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      const int r = RPI * (NIT * wave + k) + lane / CPR;
      voff[k] = r * row_b + 16 * ((lane % CPR) ^ tile_sw<D>(r));
    }
#pragma unroll
    for (int c = 0; c < D / 16; ++c) raddr[c] = ln * ROW_B + 16 * ((2 * c + lh) ^ tile_sw<D>(ln));
    const int t16 = lane & 15, j = t16 >> 2, q = t16 & 3, gq = (lane >> 4) & 1;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int r = 4 * lh + j + 8 * x;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        taddr[x][db] = r * ROW_B + 16 * ((4 * db + 2 * gq + (q >> 1)) ^ tile_sw<D>(r)) + 8 * (q & 1);
    }
  }
  // A operand of a gradient product: head-dim rows 32 db + ln, tile rows 16 kk + the above
  __device__ __forceinline__ bf16x8 tfrag(const unsigned char* tile, int db, int kk) const {
    const u32x2 lo = tr_read(tile + taddr[0][db] + 16 * ROW_B * kk);
    const u32x2 hi = tr_read(tile + taddr[1][db] + 16 * ROW_B * kk);
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  }
};

// ---- dq (+ dr, dE, dtable): query-parallel -----------------------------------------------------
// One workgroup = 4 waves x 32 query rows of one head, walking the kv head's 32-key tiles (K and
// V through the ring).  The forward's transposed layout: S^T = K Q^T, so each lane owns one query
// row and its lse, rowsum and temperature are scalars; Q^T and dO^T stay in registers as B
// operands.  Per step a wave turns the P^T and dP^T it formed at the end of the previous step
// into dZ^T, accumulates dQ^T += K^T dZ^T (K^T from transposing reads of the K tile) and the
// bias-parameter gradients of in-band steps, and forms the next step's S^T, dP^T and P^T; one
// barrier per step.  LDS besides the ring: per wave the skewed dZ buffers and the curves (r.E); the table row
// (table mode) or E staged curve-major for the dr MFMA (r.E).
template <int D, int MODE>
struct DqLayout {
  static constexpr int ROW_B = 2 * D;
  static constexpr int TILE_B = TROWS * ROW_B;   // K or V tile
  static constexpr int SLOT_B = 2 * TILE_B;
  static constexpr int RING_B = NBUF * SLOT_B;
  static constexpr int G_BYTES = (MODE == 2) ? 32 * GST * 2 : 0;
  static constexpr int GT_BYTES = (MODE != 0) ? 64 * GTS * 2 : 0;
  static constexpr int C_BYTES = (MODE == 2) ? CURVE_BYTES_DQ : 0;   // the step's curves (fp32)
  static constexpr int WAVE_BYTES = G_BYTES + GT_BYTES + C_BYTES;
  static constexpr int FIXED = RING_B + DQ_WAVES * WAVE_BYTES;
  static int bytes(int Rb, int R) {
    int n = FIXED;
    if (MODE == 1) n += (Rb + 2 * PADT) * 4;
    if (MODE == 2) n += R * ef_stride(Rb) * 2;
    return n;
  }
  // Row stride (bf16) of E staged curve-major for the dr MFMA.
  __host__ __device__ static int ef_stride(int Rb) { return (Rb + 2 * PADE + 7) & ~7; }
};

template <int D, int MODE, int EW>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a, int n_qtiles, int longest_first) {
  using L = DqLayout<D, MODE>;
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TILE_B = L::TILE_B;
  constexpr int SLOT_B = L::SLOT_B;
  constexpr int NIT = TROWS / (64 / (L::ROW_B / 16)) / DQ_WAVES;   // direct loads per wave and tile
  static_assert(NIT >= 1 && NIT * (64 / (L::ROW_B / 16)) * DQ_WAVES == TROWS, "tile rows split evenly");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31;
  const int lh = lane >> 5;

  unsigned char* wsp = smem + L::RING_B + wave * L::WAVE_BYTES;
  uint16_t* Gs = reinterpret_cast<uint16_t*>(wsp);
  uint16_t* GTs = reinterpret_cast<uint16_t*>(wsp + L::G_BYTES);
  float* cbuf = reinterpret_cast<float*>(wsp + L::G_BYTES + L::GT_BYTES);   // r.E: the step's curves
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

  // steps: the kv head's 32-key tiles t_begin + js, js < nsteps, that the workgroup's rows see;
  // the wave's own tiles are w_lo .. w_hi
  const int wg_last = min(S, wg_i0 + 32 * DQ_WAVES) - 1;
  const int kmin = W ? max(0, wg_i0 - W + 1) : 0;
  const int t_begin = kmin / TROWS;
  const int nsteps = wg_last / TROWS - t_begin + 1;
  const int w_lo = (W ? max(0, i0 - W + 1) : 0) / TROWS - t_begin;
  const int w_hi = min(S - 1, i0 + 31) / TROWS - t_begin;

  const size_t q_row = static_cast<size_t>(a.Hq) * D;
  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const int kv_row_b = a.Hkv * D * 2;
  const size_t qoff = (static_cast<size_t>(b) * S + (row_ok ? row : 0)) * q_row + static_cast<size_t>(h) * D;
  const float* Eh = (MODE == 2) ? a.E + static_cast<size_t>(h) * a.e_hs : nullptr;
  // r.E: the head's converted E rows at distance 0, the lane's r fragment (its own query row),
  // and the curve buffer geometry (the forward's packed rows: row n in slot
  // ((3 (n / 4) + sigma(n % 4)) % 8) + 8 (n % 4), 36 entries, entry t - 4 (n / 4))
  const uint16_t* e2h = (MODE == 2)
      ? a.e2 + (static_cast<size_t>(a.e_hs ? h : 0) * (Rb + 2 * kE2Pad + 1) + kE2Pad) * EW
      : nullptr;
  bf16x8 rf = {};
  const lds_float* crd = nullptr;
  float* crow_w = nullptr;
  if (MODE == 2) {
    rf = r_frag<EW>(a, b, h, row, lh);
    const int cj = ln >> 2, ce = ln & 3;
    const int cslot = ((3 * cj + (ce & 1) + 4 * (ce >> 1)) & 7) + 8 * ce;
    crow_w = cbuf + CURVE_ROWS_DQ * cslot;
    crd = (const lds_float*)(crow_w - 4 * cj + 4 + ln - 4 * lh);
    asm volatile("" : "+v"(crd));   // one base register, immediate offsets for the reads
  }

  // bias parameters of the head in LDS (made visible by the first barrier)
  if (MODE == 1) {
    const float* tp = a.table + static_cast<size_t>(h) * Rb;
    stage_batched(tid, 256, Rb + 2 * PADT,
        [&](int x) { return __float_as_uint(tp[min(max(x - PADT, 0), Rb - 1)]); },
        [&](int x, uint32_t w) {
          const int d = x - PADT;
          const uint32_t keep = (d >= 0 && d < Rb) ? ~0u : 0u;
          tabs[x] = __uint_as_float(__float_as_uint(__uint_as_float(w) * kLog2e) & keep);
        });
  }
  const int efs = L::ef_stride(Rb);
  if (MODE == 2) {
    stage_batched(tid, 256, a.R * efs,
        [&](int x) {
          const int f = x / efs;
          const int d = x - f * efs - PADE;
          return __float_as_uint(Eh[static_cast<size_t>(f) * Rb + min(max(d, 0), Rb - 1)]);
        },
        [&](int x, uint32_t w) {
          const int f = x / efs;
          const int d = x - f * efs - PADE;
          const uint32_t keep = (d >= 0 && d < Rb) ? 0xFFFFu : 0u;
          ef[x] = static_cast<uint16_t>(f32_to_bf16(__uint_as_float(w)) & keep);
        });
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
      // all 8 loads issued before any is used (clamped inside the rows, masked afterwards as
      // integers, so that none sits behind its own branch)
      uint32_t xr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int rr = i0 + 16 * kk + 8 * lh + e;
        if (MODE == 1) {
          xr[e] = (rr < S && ln == 0) ? 0x3f80u : 0u;   // bf16 1.0
        } else {
          const uint32_t raw = a.r[((static_cast<size_t>(b) * S + min(rr, S - 1)) * a.Hq + h) * a.R + min(ln, a.R - 1)];
          xr[e] = raw & ((rr < S && ln < a.R) ? 0xFFFFu : 0u);
        }
      }
      rA[kk] = as_bf16x8(u32x4{xr[0] | (xr[1] << 16), xr[2] | (xr[3] << 16), xr[4] | (xr[5] << 16), xr[6] | (xr[7] << 16)});
    }
    // zero the skewed buffers once: every in-band step writes the same set of positions
    for (int x = lane; x < (L::G_BYTES + L::GT_BYTES) / 16; x += 64)
      st16(reinterpret_cast<unsigned char*>(Gs) + 16 * x, u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = zero16();
  f32x16 dracc = zero16();
  float* dEh = (MODE == 2) ? a.dE + static_cast<size_t>(h) * a.e_hs : nullptr;
  float* dtab = (MODE == 1) ? a.dtable + static_cast<size_t>(h) * Rb : nullptr;

  const TileAddr<D, NIT> ta(lane, wave, kv_row_b);
  const uint16_t* kbase = a.k + static_cast<size_t>(b) * S * kv_row + static_cast<size_t>(hkv) * D;
  const uint16_t* vbase = a.v + static_cast<size_t>(b) * S * kv_row + static_cast<size_t>(hkv) * D;
  auto dma_tile = [&](int js, unsigned char* slot) __attribute__((always_inline)) {
    const int k0 = (t_begin + js) * TROWS;
    const int rows = min(S - k0, TROWS);
    const int nrec = (rows - 1) * kv_row_b + L::ROW_B;   // keys past S read as zeros
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + static_cast<size_t>(k0) * kv_row, nrec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + static_cast<size_t>(k0) * kv_row, nrec);
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      dma16(rk, slot + (NIT * wave + k) * 1024, ta.voff[k]);
      dma16(rv, slot + TILE_B + (NIT * wave + k) * 1024, ta.voff[k]);
    }
  };
  // element (key m, query n) of a step lies at distance c + n - m, c = i0 - its first key
  auto step_c = [&](int js) { return i0 - (t_begin + js) * TROWS; };
  auto step_on = [&](int js) { return wave_live && js < nsteps && js >= w_lo && js <= w_hi; };
  auto step_inband = [&](int js) { return MODE != 0 && step_c(js) - 31 < Rb; };

  // S^T (log2 units, with the bias) and dP^T of a step
  // S^T and dP^T of a step, and P (in place of S).  The S chain is issued first and the dP chain
  // second, with the vector work on S (scale, bias, exp) in groups between the dP products: a wave
  // runs alone on its SIMD, so its vector work overlaps MFMAs only when interleaved with its own.
  // The r.E curves' MFMAs go ahead of the S chain, so that their results are ready when the
  // curve buffer is written.  Fragments in groups of two head-dim chunks (four 16-byte reads),
  // the next group's reads issued before the current group's MFMAs (scheduling barriers pin the
  // order; left to itself the compiler keeps one fragment in flight and each MFMA waits out its
  // read).
  auto scores = [&](int js, const unsigned char* slot, f32x16& sacc, f32x16& pacc,
                    const u32x4 (&eb)[2][EW / 16]) __attribute__((always_inline)) {
    const int c = step_c(js);
    const bool ib = step_inband(js);
    sacc = zero16();
    pacc = zero16();
    f32x16 clo, chi;
    if (MODE == 2 && ib) curve_mfma<EW>(eb, rf, clo, chi);
    constexpr int NG = NC / 2;   // fragment groups per chain
    bf16x8 fr[2][2];
    // group q < NG: K chunks 2q, 2q + 1; group NG + q: the same V chunks
    auto rd = [&](int q) __attribute__((always_inline)) {
      const unsigned char* t = slot + (q >= NG ? TILE_B : 0);
#pragma unroll
      for (int u = 0; u < 2; ++u) fr[q & 1][u] = as_bf16x8(ld16(t + ta.raddr[2 * (q % NG) + u]));
    };
    rd(0);
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      rd(q + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u) sacc = mfma32(fr[q & 1][u], qf[2 * q + u], sacc);
    }
    // bias of the step in units of the log2-domain logit, fetched while the S chain runs
    float bv[16];
    float bm = 0.f;
    if (MODE == 1 && ib) {
      // distances c + ln - m lie in [-31, Rb + 62]: inside the zero-padded row
      const float* tb = tabs + PADT + c + ln;
#pragma unroll
      for (int i = 0; i < 16; ++i) bv[i] = tb[-out_row(i, lh)];
      bm = tq;
    }
    if (MODE == 2 && ib) {
      // curves of the wave's 32 rows over the step's distances c - 31 .. c + 32, fp32; key
      // m = 8 g + 4 lh + k of row n at distance c + n - m, entry t = 31 + n - m of row n
      curve_write(crow_w, ln, lh, clo, chi);
      wave_sync_lds();
#pragma unroll
      for (int i = 0; i < 16; ++i) bv[i] = crd[27 - 8 * (i >> 2) - (i & 3)];
      wave_sync_lds();   // the next step's writes follow these reads
      bm = cb;
    }
    // dP chain; P = exp2(tau (scale log2(e) q.k + log2(e) beta) - lse2), EPG elements per group
    constexpr int EPG = 16 / NG;
    auto chain = [&](auto bias_c) __attribute__((always_inline)) {
      constexpr bool BIAS = decltype(bias_c)::value;
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        if (q + 1 < NG) rd(NG + q + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 2; ++u) pacc = mfma32(fr[(NG + q) & 1][u], dof[2 * q + u], pacc);
#pragma unroll
        for (int e = 0; e < EPG; ++e) {
          const int i = EPG * q + e;
          float x = sacc[i] * cq;
          if constexpr (BIAS) x = fmaf(bv[i], bm, x);
          sacc[i] = fast_exp2(x - lse2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (MODE != 0 && ib) chain(std::true_type{});
    else chain(std::false_type{});
    if ((c - 31 < 0) || (W && c + 31 >= W)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = c + ln - out_row(i, lh);
        const bool vis = (d >= 0) & ((W == 0) | (d < W));
        sacc[i] = vis ? sacc[i] : 0.f;
      }
    }
  };
  // dZ^T = P (dP - rowsum) and dQ^T += K^T dZ^T.  The first key chunk's dZ (output groups 0
  // and 1) is formed first; its products then run beside the second chunk's dZ.
  auto grads = [&](int js, const unsigned char* slot, const f32x16& pf32,
                   const f32x16& pacc) __attribute__((always_inline)) {
    const int c = step_c(js);
    float dz[16];
    bf16x8 dzf[2];
    auto pack = [&](int kk) __attribute__((always_inline)) {
      uint32_t w[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) w[jj] = pack_bf16x2(dz[8 * kk + 2 * jj], dz[8 * kk + 2 * jj + 1]);
      dzf[kk] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
    };
#pragma unroll
    for (int i = 0; i < 8; ++i) dz[i] = pf32[i] * (pacc[i] - dsum);
    pack(0);
    constexpr int EPX = 8 / NDB;   // second-chunk elements per first-chunk product
    bf16x8 kt[2];
    kt[0] = ta.tfrag(slot, 0, 0);
#pragma unroll
    for (int x = 0; x < 2 * NDB; ++x) {
      // the next product's transposing reads are issued before this product (as in the
      // scores: otherwise each MFMA waits out its own reads)
      if (x + 1 < 2 * NDB) kt[(x + 1) & 1] = ta.tfrag(slot, (x + 1) % NDB, (x + 1) / NDB);
      __builtin_amdgcn_sched_barrier(0);
      dqacc[x % NDB] = mfma32(kt[x & 1], dzf[x / NDB], dqacc[x % NDB]);
      if (x < NDB) {
#pragma unroll
        for (int e = 0; e < EPX; ++e) {
          const int i = 8 + EPX * x + e;
          dz[i] = pf32[i] * (pacc[i] - dsum);
        }
        if (x == NDB - 1) pack(1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    if (MODE != 0 && step_inband(js)) {
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
  };

  // prologue: the first two steps' tiles, the first step's scores
  dma_tile(0, smem);
  if (nsteps > 1) dma_tile(1, smem + SLOT_B);
  u32x4 eb[2][EW / 16];
  if (MODE == 2 && step_on(0) && step_inband(0)) e_rows<EW>(e2h, step_c(0), ln, lh, eb);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's direct loads have landed
  __syncthreads();
  f32x16 sa, pa;
  if (step_on(0)) scores(0, smem, sa, pa, eb);

  // step js: the gradients of js (tiles in slot js % 3), then the scores of js + 1 (slot
  // (js + 1) % 3) into the same registers; the tiles of js + 2 go to the slot js - 1 used.  The
  // slots are passed as restrict pointers: the compiler then knows that the direct loads into ds
  // do not alias the reads of cs and ns and adds no wait for them.
  auto iteration_body = [&](int js, const unsigned char* __restrict__ cs, const unsigned char* __restrict__ ns,
                            unsigned char* __restrict__ ds, auto inner_c) __attribute__((always_inline)) {
    constexpr bool INNER = decltype(inner_c)::value;   // js + 2 < nsteps is known
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    u32x4 e[2][EW / 16];
    if (MODE == 2 && step_on(js + 1) && step_inband(js + 1)) e_rows<EW>(e2h, step_c(js + 1), ln, lh, e);
    // the E rows are requested before the tiles of js + 2, so that the wait for them
    // (vector-memory counts retire in order) does not wait for the tiles
    __builtin_amdgcn_sched_barrier(0);
    if (INNER || js + 2 < nsteps) dma_tile(js + 2, ds);
    if (step_on(js)) grads(js, cs, sa, pa);
    if (step_on(js + 1)) scores(js + 1, ns, sa, pa, e);
  };
  using true_t = std::integral_constant<bool, true>;
  using false_t = std::integral_constant<bool, false>;
  auto iteration = [&](int js, int sl, auto inner_c) __attribute__((always_inline)) {
    iteration_body(js, smem + sl * SLOT_B, smem + ((sl + 1) % NBUF) * SLOT_B, smem + ((sl + 2) % NBUF) * SLOT_B,
                   inner_c);
  };
  int js = 0;
  for (; js + 4 < nsteps; js += 3) {
    iteration(js, 0, true_t{});
    iteration(js + 1, 1, true_t{});
    iteration(js + 2, 2, true_t{});
  }
  for (; js + 1 < nsteps; ++js) iteration(js, js % NBUF, false_t{});
  if (step_on(js)) grads(js, smem + (js % NBUF) * SLOT_B, sa, pa);

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
// One workgroup = 4 waves x 32 keys of one kv head, walking (query head of the group, 32-row query
// tile) steps, head-major.  The forward's structure with the roles of queries and keys swapped:
// K and V stay in registers as B operands, and each step's q and dout rows go straight from
// global memory into a 3-slot LDS ring (16-byte chunks, swizzled so that both the row reads of
// the score products and the transposing reads of the gradient products are free of bank
// conflicts), with the step's per-row values (lse, rowsum, temperature) beside them, two steps
// ahead.  Per step a wave turns the P and dP = dO V^T it formed at the end of the previous step
// into dZ, accumulates dV^T += dO^T P and dK^T += Q^T dZ, and forms the next step's
// S = Q K^T, dP and P; one barrier per step.
template <int D>
struct DkvLayout {
  static constexpr int ROW_B = 2 * D;                  // bytes per tile row
  static constexpr int TILE_B = TROWS * ROW_B;       // q or dout tile
  static constexpr int REC_B = 4 * TROWS * 4;        // per-row lse2, rowsum, c_qk tau, tau
  static constexpr int SLOT_B = 2 * TILE_B + REC_B;
  static constexpr int RING_B = NBUF * SLOT_B;
  // table mode: two head slots of the zero-padded table row; r.E: a curve buffer per wave
  static int bytes(int mode, int Rb) {
    return RING_B + (mode == 1 ? 2 * (Rb + 2 * PADT) * 4 : 0) + (mode == 2 ? DKV_WAVES * CURVE_BYTES_KV : 0);
  }
};

template <int D, int MODE, int EW>
__global__ __launch_bounds__(64 * DKV_WAVES, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using L = DkvLayout<D>;
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NT = 64 * DKV_WAVES;
  constexpr int ROW_B = L::ROW_B;
  constexpr int TILE_B = L::TILE_B;
  constexpr int SLOT_B = L::SLOT_B;
  constexpr int CPR = ROW_B / 16;                     // chunks per row
  constexpr int RPI = 64 / CPR;                       // rows per direct-load instruction
  constexpr int NIT = TROWS / RPI / DKV_WAVES;      // instructions per wave and tile
  static_assert(NIT >= 1 && NIT * RPI * DKV_WAVES == TROWS, "tile rows split evenly over the waves");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int Rb = a.bias_range;
  const int TROW = Rb + 2 * PADT;
  float* tabs = reinterpret_cast<float*>(smem + L::RING_B);   // table mode: 2 x [PADT + Rb + PADT]

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
  const int G = a.G;
  const int j_lo = kt * (32 * DKV_WAVES);
  const int j0w = j_lo + 32 * wave;
  const bool wave_live = j0w < S;
  const int key = j0w + ln;
  const bool key_ok = key < S;
  const float inv_scale = 1.f / a.scale;   // bias in units of the raw score q.k

  const size_t q_row = static_cast<size_t>(a.Hq) * D;
  const int q_row_b = a.Hq * D * 2;
  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const size_t koff = (static_cast<size_t>(b) * S + (key_ok ? key : 0)) * kv_row + static_cast<size_t>(hkv) * D;

  // r.E: the wave's curve buffer, query row m at 40 m + t - 4 (m / 4) (entries t = m .. m + 31
  // of the row are written); key n reads row m at t = 31 + m - n, which for element i (query
  // m = 8 g + 4 lh + k) is 320 g + 41 k + 160 lh + 31 - n: one base register per lane and
  // immediate offsets, and each half-wave reads 32 consecutive dwords of one row
  float* cbuf = (MODE == 2) ? reinterpret_cast<float*>(smem + L::RING_B) + wave * (CURVE_BYTES_KV / 4) : nullptr;
  const lds_float* crd = nullptr;
  if (MODE == 2) {
    crd = (const lds_float*)(cbuf + 160 * lh + 31 - ln);
    asm volatile("" : "+v"(crd));
  }

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

  // steps: (query head hh of the group, query tile t_begin + t), t < ntiles
  const int last_key = min(S, j_lo + 32 * DKV_WAVES) - 1;
  const int i_last = W ? min(S - 1, last_key + W - 1) : S - 1;
  const int t_begin = j_lo / TROWS;
  const int ntiles = i_last / TROWS - t_begin + 1;
  const int nsteps = G * ntiles;
  // the wave's tiles within a head: from the tile of its first key to that of its keys' last
  // visible query row
  const int w_lo = wave;
  const int w_hi = (W ? min(S - 1, j0w + 31 + W - 1) : S - 1) / TROWS - t_begin;

  // a step's position (head hh, tile t), advanced one step at a time (no divisions per step);
  // hh == G past the last step
  struct Pos {
    int hh, t;
  };
  auto pos_next = [&](Pos p) {
    if (++p.t == ntiles) {
      p.t = 0;
      ++p.hh;
    }
    return p;
  };
  auto step_head = [&](Pos p) { return p.hh; };
  auto step_row0 = [&](Pos p) { return (t_begin + p.t) * TROWS; };
  auto step_on = [&](Pos p) { return wave_live && p.hh < G && p.t >= w_lo && p.t <= w_hi; };
  // element (query m, key n) of a step lies at distance c + m - n, c = its first row - j0w
  auto step_inband = [&](Pos js) { return MODE != 0 && step_row0(js) - j0w - 31 < a.bias_range; };
  auto step_edge = [&](Pos js) {
    const int i0 = step_row0(js);
    const int c = i0 - j0w;
    return (c - 31 < 0) || (W && c + 31 >= W) || (i0 + TROWS > S);
  };

  const TileAddr<D, NIT> ta(lane, wave, q_row_b);
  auto dma_tile = [&](Pos js, unsigned char* slot) __attribute__((always_inline)) {
    const int h = hkv * G + step_head(js);
    const int i0 = step_row0(js);
    const int rows = min(S - i0, TROWS);
    const int nrec = (rows - 1) * q_row_b + ROW_B;   // rows past S read as zeros
    const size_t off = (static_cast<size_t>(b) * S + i0) * q_row + static_cast<size_t>(h) * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + off, nrec);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dout + off, nrec);
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
      dma16(rq, slot + (NIT * wave + k) * 1024, ta.voff[k]);
      dma16(rd, slot + TILE_B + (NIT * wave + k) * 1024, ta.voff[k]);
    }
  };
  // per-row values of a step, through lanes 0..31 of wave 0: requested with the step's tiles (two
  // steps ahead) and stored beside them at the end of that iteration, ahead of the barrier that
  // publishes both; rows past S get lse = +inf (P = 0)
  float rec_l = INFINITY, rec_s = 0.f;
  int rec_row = 0;
  auto rec_load = [&](Pos js) __attribute__((always_inline)) {
    if (wave == 0 && lh == 0) {
      const int h = hkv * G + step_head(js);
      rec_row = step_row0(js) + ln;
      rec_l = INFINITY;
      rec_s = 0.f;
      if (rec_row < S) {
        const size_t lrow = (static_cast<size_t>(b) * a.Hq + h) * S + rec_row;
        rec_l = a.lse[lrow];
        rec_s = a.dsum[lrow];
      }
    }
  };
  auto rec_store = [&](unsigned char* slot) __attribute__((always_inline)) {
    if (wave == 0 && lh == 0) {
      float* rp = reinterpret_cast<float*>(slot + 2 * TILE_B);
      const float tq = temp_factor(visible_keys(rec_row, W), a.temp_len, a.temp_inv_log2);
      rp[ln] = rec_l * kLog2e;
      rp[TROWS + ln] = rec_s;
      rp[2 * TROWS + ln] = a.c_qk * tq;
      rp[3 * TROWS + ln] = tq;
    }
  };
  // table mode: head hh's row (in units of the raw score), zero-padded, into slot hh % 2
  auto stage_table = [&](int hh) __attribute__((always_inline)) {
    float* tab = tabs + (hh & 1) * TROW;
    const float* tp = a.table + static_cast<size_t>(hkv * G + hh) * Rb;
    stage_batched(tid, NT, TROW,
        [&](int x) { return __float_as_uint(tp[min(max(x - PADT, 0), Rb - 1)]); },
        [&](int x, uint32_t w) {
          const int d = x - PADT;
          const uint32_t keep = (d >= 0 && d < Rb) ? ~0u : 0u;
          tab[x] = __uint_as_float(__float_as_uint(__uint_as_float(w) * inv_scale) & keep);
        });
  };

  const uint16_t* e2b = (MODE == 2) ? a.e2 + kE2Pad * EW : nullptr;
  const bool rvec = r_vec<EW>(a);
  auto e_load = [&](Pos js, u32x4 (&eb)[2][EW / 16], RRaw& rx) __attribute__((always_inline)) {
    const int h = hkv * G + step_head(js);
    const int i0 = step_row0(js);
    e_rows<EW>(e2b + static_cast<size_t>(a.e_hs ? h : 0) * (Rb + 2 * kE2Pad + 1) * EW, i0 - j0w, ln, lh, eb);
    r_load<EW>(a, rvec, b, h, i0 + ln, lh, rx);
  };

  // S (plus the bias, in units of q.k), dP and P of a step (P in place of S).  The S chain is
  // issued first and the dP chain second, with the vector work on S (bias, exp) in groups between
  // the dP products: a wave runs alone on its SIMD, so its vector work overlaps MFMAs only when
  // interleaved with its own.  The r.E curves' MFMAs go ahead of the S chain.  Per row: lse
  // (log2 units) and c_qk * tau from the step's row values.  Fragments in groups of two head-dim
  // chunks (four 16-byte reads), the next group's reads issued before the current group's MFMAs
  // (scheduling barriers pin the order; left to itself the compiler keeps one fragment in flight
  // and each MFMA waits out its read).
  auto scores = [&](Pos js, const unsigned char* slot, f32x16& sacc, f32x16& pacc, const u32x4 (&eb)[2][EW / 16],
                    const RRaw& rx) __attribute__((always_inline)) {
    const int i0 = step_row0(js);
    const int c = i0 - j0w;
    const bool ib = step_inband(js);
    const float* rp = reinterpret_cast<const float*>(slot + 2 * TILE_B);
    sacc = zero16();
    pacc = zero16();
    if (MODE == 1 && ib) {
      // distances c + m - ln lie in [-31, Rb + 62]: inside the zero-padded row
      const float* tb = tabs + (step_head(js) & 1) * TROW + PADT + c - ln;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = tb[out_row(i, lh)];
    }
    f32x16 clo, chi;
    if (MODE == 2 && ib) curve_mfma<EW>(eb, r_pack<EW>(a, rvec, i0 + ln, lh, rx), clo, chi);
    constexpr int NG = NC / 2;   // fragment groups per chain
    bf16x8 fr[2][2];
    // group q < NG: q chunks 2q, 2q + 1; group NG + q: the same dout chunks
    auto rd = [&](int q) __attribute__((always_inline)) {
      const unsigned char* t = slot + (q >= NG ? TILE_B : 0);
#pragma unroll
      for (int u = 0; u < 2; ++u) fr[q & 1][u] = as_bf16x8(ld16(t + ta.raddr[2 * (q % NG) + u]));
    };
    rd(0);
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      rd(q + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u) sacc = mfma32(fr[q & 1][u], kf[2 * q + u], sacc);
      // the curves are written halfway through the S chain, once their MFMAs have finished
      if (MODE == 2 && q == NG / 2 - 1 && ib) curve_write(cbuf + CURVE_ROWS_KV * ln, ln, lh, clo, chi);
    }
    // rows 8 g + 4 lh .. + 3 of element group g
    f32x4 l4[4], c4[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      l4[g4] = *reinterpret_cast<const f32x4*>(rp + 8 * g4 + 4 * lh);
      c4[g4] = *reinterpret_cast<const f32x4*>(rp + 2 * TROWS + 8 * g4 + 4 * lh);
    }
    float bv[16];
    if (MODE == 2 && ib) {
      wave_sync_lds();
#pragma unroll
      for (int i = 0; i < 16; ++i) bv[i] = crd[320 * (i >> 2) + 41 * (i & 3)];
      wave_sync_lds();   // the next step's writes follow these reads
    }
    constexpr int EPG = 16 / NG;   // elements per dP group
    auto chain = [&](auto bias_c) __attribute__((always_inline)) {
      constexpr bool BIAS = decltype(bias_c)::value;
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        if (q + 1 < NG) rd(NG + q + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 2; ++u) pacc = mfma32(fr[(NG + q) & 1][u], vf[2 * q + u], pacc);
#pragma unroll
        for (int e = 0; e < EPG; ++e) {
          const int i = EPG * q + e;
          float x = sacc[i];
          if constexpr (BIAS) x = fmaf(bv[i], inv_scale, x);
          sacc[i] = fast_exp2(fmaf(x, c4[i >> 2][i & 3], -l4[i >> 2][i & 3]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (MODE == 2 && ib) chain(std::true_type{});
    else chain(std::false_type{});
    if (step_edge(js)) {
      const int wlim = W ? W : 0x7fffffff;
      const int mlim = S - i0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = out_row(i, lh);
        const int d = c + m - ln;
        sacc[i] = ((d >= 0) & (d < wlim) & (m < mlim)) ? sacc[i] : 0.f;
      }
    }
  };
  // dZ = tau * P * (dP - rowsum) and the gradient products dV^T += dO^T P, dK^T += Q^T dZ, with
  // P and dZ rounded to bf16 as their B operands: the dV products (P alone) run beside the dZ
  // work, then the dK products.  The next product's transposing reads are issued before this
  // product (as in the scores).
  auto grads = [&](const unsigned char* slot, const f32x16& pr, f32x16& pacc) __attribute__((always_inline)) {
    const float* rp = reinterpret_cast<const float*>(slot + 2 * TILE_B);
    bf16x8 pf[2], dzf[2];
    auto pack = [&](const f32x16& v, bf16x8 (&f)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t w[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) w[jj] = pack_bf16x2(v[8 * kk + 2 * jj], v[8 * kk + 2 * jj + 1]);
        f[kk] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
      }
    };
    pack(pr, pf);
    f32x4 s4[4], t4[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      s4[g4] = *reinterpret_cast<const f32x4*>(rp + TROWS + 8 * g4 + 4 * lh);
      t4[g4] = *reinterpret_cast<const f32x4*>(rp + 3 * TROWS + 8 * g4 + 4 * lh);
    }
    constexpr int NX = 2 * NDB;    // products per gradient
    constexpr int EPX = 16 / NX;   // dZ elements per dV product
    // product y < NX: dV, head-dim block y / 2 over query rows 16 (y % 2) ..; then dK
    auto tr = [&](int y) __attribute__((always_inline)) {
      return y < NX ? ta.tfrag(slot + TILE_B, y >> 1, y & 1) : ta.tfrag(slot, (y - NX) >> 1, y & 1);
    };
    bf16x8 fa[2];
    fa[0] = tr(0);
#pragma unroll
    for (int y = 0; y < 2 * NX; ++y) {
      if (y + 1 < 2 * NX) fa[(y + 1) & 1] = tr(y + 1);
      __builtin_amdgcn_sched_barrier(0);
      if (y < NX) {
        dvacc[y >> 1] = mfma32(fa[y & 1], pf[y & 1], dvacc[y >> 1]);
#pragma unroll
        for (int e = 0; e < EPX; ++e) {
          const int i = EPX * y + e;
          pacc[i] = pr[i] * (pacc[i] - s4[i >> 2][i & 3]) * t4[i >> 2][i & 3];
        }
        if (y == NX - 1) pack(pacc, dzf);
      } else {
        const int x = y - NX;
        dkacc[x >> 1] = mfma32(fa[y & 1], dzf[x & 1], dkacc[x >> 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: the first two steps' tiles and row values, the first step's scores
  if (MODE == 1) {
    stage_table(0);
    if (ntiles == 1 && G > 1) stage_table(1);
  }
  Pos p0 = {0, 0};
  Pos p1 = pos_next(p0);
  Pos p2 = pos_next(p1);
  rec_load(p0);
  dma_tile(p0, smem);
  if (nsteps > 1) dma_tile(p1, smem + SLOT_B);
  rec_store(smem);
  if (nsteps > 1) {
    rec_load(p1);
    rec_store(smem + SLOT_B);
  }
  u32x4 eb[2][EW / 16];
  RRaw rx;
  if (MODE == 2 && step_on(p0) && step_inband(p0)) e_load(p0, eb, rx);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's direct loads have landed
  __syncthreads();
  f32x16 sa, pa;
  if (step_on(p0)) scores(p0, smem, sa, pa, eb, rx);

  // step js: dZ and the gradient products of js (its row values and tiles in slot js % 3, P and
  // dP in registers), then the scores and P of js + 1 (slot (js + 1) % 3) into the same
  // registers; the tiles and row values of js + 2 go to the slot js - 1 used.  The slots are
  // passed as restrict pointers: the compiler then knows that the direct loads into ds do not
  // alias the reads of cs and ns and adds no wait for them.
  auto iteration_body = [&](const unsigned char* __restrict__ cs, const unsigned char* __restrict__ ns,
                            unsigned char* __restrict__ ds, auto inner_c) __attribute__((always_inline)) {
    constexpr bool INNER = decltype(inner_c)::value;   // step js + 2 exists
    const bool more = INNER || p2.hh < G;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    u32x4 e[2][EW / 16];
    RRaw x;
    if (MODE == 2 && step_on(p1) && step_inband(p1)) e_load(p1, e, x);
    if (MODE == 1 && more && p2.t == 0) stage_table(p2.hh);
    if (more) rec_load(p2);
    // the bias operands and row values are requested before the tiles of js + 2, so that the
    // waits for them (vector-memory counts retire in order) do not wait for the tiles
    __builtin_amdgcn_sched_barrier(0);
    if (more) dma_tile(p2, ds);
    if (step_on(p0)) grads(cs, sa, pa);
    if (step_on(p1)) scores(p1, ns, sa, pa, e, x);
    if (more) rec_store(ds);
    p0 = p1;
    p1 = p2;
    p2 = pos_next(p2);
  };
  using true_t = std::integral_constant<bool, true>;
  using false_t = std::integral_constant<bool, false>;
  auto iteration = [&](int sl, auto inner_c) __attribute__((always_inline)) {
    iteration_body(smem + sl * SLOT_B, smem + ((sl + 1) % NBUF) * SLOT_B, smem + ((sl + 2) % NBUF) * SLOT_B,
                   inner_c);
  };
  int js = 0;
  for (; js + 4 < nsteps; js += 3) {
    iteration(0, true_t{});
    iteration(1, true_t{});
    iteration(2, true_t{});
  }
  for (; js + 1 < nsteps; ++js) iteration(js % NBUF, false_t{});
  if (step_on(p0)) grads(smem + (js % NBUF) * SLOT_B, sa, pa);

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
hipError_t allow_lds(K* kernel, int bytes, hipStream_t s) {
  return set_max_lds(reinterpret_cast<const void*>(kernel), bytes, s);
}

template <int D, int MODE, int EW>
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
  if (MODE == 2) {   // E as bf16 high and low parts (scale 1: the kernels add the bias in its own units)
    e = launch_e2_convert(a.E, a.e_hs, a.R, a.bias_range, 1.f, a.e_hs ? a.Hq : 1, a.e2, s);
    if (e != hipSuccess) return e;
  }
  // dq (+ bias-parameter gradients)
  const int n_qtiles = (a.S + 32 * DQ_WAVES - 1) / (32 * DQ_WAVES);
  const int longest_first = (a.window == 0 || a.window > 32 * DQ_WAVES) ? 1 : 0;
  const long long nq = static_cast<long long>(n_qtiles) * a.Hq * a.B;
  const int dq_lds = DqLayout<D, MODE>::bytes(a.bias_range, a.R);
  e = allow_lds(&bwd_dq_kernel<D, MODE, EW>, dq_lds, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, MODE, EW>), dim3(static_cast<unsigned>(nq)), dim3(64 * DQ_WAVES), dq_lds, s,
                     a, n_qtiles, longest_first);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dk, dv
  const int kv_lds = DkvLayout<D>::bytes(MODE, a.bias_range);
  e = allow_lds(&bwd_dkdv_kernel<D, MODE, EW>, kv_lds, s);
  if (e != hipSuccess) return e;
  const int n_ktiles = (a.S + 32 * DKV_WAVES - 1) / (32 * DKV_WAVES);
  const long long nk = static_cast<long long>(n_ktiles) * a.Hkv * a.B;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, MODE, EW>), dim3(static_cast<unsigned>(nk)), dim3(64 * DKV_WAVES), kv_lds, s,
                     a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_mode(const BwdArgs& a, int mode, hipStream_t s) {
  switch (mode) {
    case 0: return launch_bwd<D, 0, 16>(a, s);
    case 1: return launch_bwd<D, 1, 16>(a, s);
    default: return e2_width(a.R) == 32 ? launch_bwd<D, 2, 32>(a, s) : launch_bwd<D, 2, 16>(a, s);
  }
}

}  // namespace

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
  const int m = std::max(dq, kv);
  return m > kMaxLds ? -1 : m;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int D, int mode, hipStream_t s) {
  if (a.B == 0 || a.S == 0) return hipSuccess;
  if (D == 128) return launch_bwd_mode<128>(a, mode, s);
  return launch_bwd_mode<64>(a, mode, s);
}

}  // namespace rba
