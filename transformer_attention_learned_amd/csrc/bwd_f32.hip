// fp32 backward of the relative-position-bias attention on the vector ALUs (no bf16
// anywhere), the gradient counterpart of attn_f32.hip.
//
// The bias is a learned part of the layer ("Thinking Machines dropped RoPE": the bank of distance
// curves and the coefficient projection are trained with the model; "Learned Relative-Position
// Bias", section "Standard Relative Bias (T5-style)": the table is a learned parameter), so the
// pass returns the gradients of q, k, v and of the bias parameters.  With the forward's logits
// z = tau (scale q.k + beta), P = exp(z - lse) and rowsum = sum_d dout * o:
//   dP = dout . v,  dZ = tau P (dP - rowsum),  dq = scale sum_j dZ k,  dk = scale sum_i dZ q,
//   dv = sum_i P dout,  and at in-band pairs dtable[h, delta] += dZ (table), or
//   dr[i, f] += dZ E[h, f, delta] and dE[h, f, delta] += dZ r[i, f] (r.E).
//
// Three kernels: the row sums (and zeroed bias gradients); a query-parallel pass (dq, dr and the
// bias-parameter gradients: diagonal sums of each 32 x 32 block, one atomic add per distance);
// a key-parallel pass (dk, dv), which recomputes the block's P and dZ.  Every block is 32 query
// rows x 32 keys staged in LDS; the 256 threads of a workgroup each take 4 pairs of the block
// for the dot products and a run of (row, dim) accumulators for the products with the block.

#include <algorithm>

#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

constexpr int T = 32;      // query rows and keys per block
constexpr int NTH = 256;   // threads per workgroup
constexpr int RS = 17;     // LDS row stride of the r coefficients (R <= 16)

template <int D>
constexpr int tile_floats() { return T * (D + 1); }

// LDS floats of both main kernels: four row tiles (q, dout, k, v), the P and dZ blocks, the
// query tile's r coefficients and its per-row lse, rowsum and temperature.
constexpr int NBD = 2 * T;  // distances a block's pairs span (63), padded
constexpr int RB_MAX = 16;   // bias parameters per distance (E rows; 1 for the table)

template <int D>
constexpr int bwd_f32_lds_floats() { return 4 * tile_floats<D>() + 2 * T * (T + 1) + T * RS + 3 * T + RB_MAX * NBD; }

// One wave per (batch, row, head): rowsum(dout * o) into dsum [B, Hq, S]; the first workgroups
// also clear dtable / dE, which the query-parallel kernel accumulates into.
__global__ __launch_bounds__(NTH) void bwd_f32_pre(BwdF32Args a, long long n_zero, float* zero_dst) {
  const long long rows = static_cast<long long>(a.B) * a.S * a.Hq;
  const long long row = static_cast<long long>(blockIdx.x) * (NTH / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row < rows) {
    const float* dp = a.dout + row * a.D;
    const float* op = a.o + row * a.D;
    float s = 0.f;
    for (int d = lane; d < a.D; d += 64) s = fmaf(dp[d], op[d], s);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) {
      // row = (b * S + i) * Hq + h
      const long long h = row % a.Hq;
      const long long bi = row / a.Hq;
      const long long i = bi % a.S;
      const long long b = bi / a.S;
      a.dsum[(b * a.Hq + h) * a.S + i] = s;
    }
  }
  for (long long z = static_cast<long long>(blockIdx.x) * NTH + threadIdx.x; z < n_zero;
       z += static_cast<long long>(gridDim.x) * NTH)
    zero_dst[z] = 0.f;
}

// Shared block machinery of the two main kernels.
template <int D, int MODE>
struct Block {
  float* Qs;    // [T][D + 1] query rows (zero past S)
  float* dOs;   // [T][D + 1] their output gradients
  float* Ks;    // [T][D + 1] keys
  float* Vs;    // [T][D + 1] values
  float* Ps;    // [T][T + 1] P of the block
  float* Zs;    // [T][T + 1] dZ of the block
  float* rS;    // [T][RS]    r of the query rows (MODE 2)
  float* lse_s; // [T]
  float* dsum_s;
  float* tau_s;
  float* Bs;    // [R][NBD] E rows (MODE 2) or [NBD] table entries (MODE 1) over the block's
                // distances i0 - j0 - 31 ..

  __device__ explicit Block(float* sm) {
    Qs = sm;
    dOs = Qs + tile_floats<D>();
    Ks = dOs + tile_floats<D>();
    Vs = Ks + tile_floats<D>();
    Ps = Vs + tile_floats<D>();
    Zs = Ps + T * (T + 1);
    rS = Zs + T * (T + 1);
    lse_s = rS + T * RS;
    dsum_s = lse_s + T;
    tau_s = dsum_s + T;
    Bs = tau_s + T;
  }

  // rows r0 .. r0 + 31 of a [B, S, H, D] tensor (head h of batch b) into dst, zero past S
  // (8 loads in flight per thread: rows past S read row S - 1 and are stored as zero)
  __device__ static void load_rows(float* dst, const float* src, const BwdF32Args& a, int b, int h, int H, int r0) {
    stage_batched(threadIdx.x, NTH, T * D,
        [&](int idx) {
          const int rr = idx / D;
          return __float_as_uint(src[((static_cast<size_t>(b) * a.S + min(r0 + rr, a.S - 1)) * H + h) * D + idx - rr * D]);
        },
        [&](int idx, uint32_t w) {
          const int rr = idx / D;
          dst[rr * (D + 1) + idx - rr * D] = __uint_as_float(w & ((r0 + rr < a.S) ? ~0u : 0u));
        });
  }

  // the bias parameters over the distances of block (i0.., j0..): dmin = i0 - j0 - 31 ..
  // dmin + 62, table entries (MODE 1) or the R rows of E (MODE 2), with 8 loads in flight per
  // thread; entries outside [0, bias_range) are zero and never read
  __device__ void load_bias(const BwdF32Args& a, int h, int i0, int j0) {
    if (MODE == 0 || a.bias_range <= 0) return;
    const int dmin = i0 - j0 - (T - 1);
    const float* src = MODE == 2 ? a.E + static_cast<size_t>(h) * a.e_hs : a.table + static_cast<size_t>(h) * a.bias_range;
    stage_batched(threadIdx.x, NTH, (MODE == 2 ? a.R : 1) * NBD,
        [&](int x) {
          const int f = x / NBD;
          const int d = min(max(dmin + x - f * NBD, 0), a.bias_range - 1);
          return __float_as_uint(src[static_cast<size_t>(f) * a.bias_range + d]);
        },
        [&](int x, uint32_t w) {
          const int d = dmin + x - (x / NBD) * NBD;
          Bs[x] = __uint_as_float(w & ((d >= 0 && d < a.bias_range) ? ~0u : 0u));
        });
  }

  // the query side of a block: q, dout, lse, rowsum, temperature (and r) of rows i0 .. i0 + 31
  __device__ void load_queries(const BwdF32Args& a, int b, int h, int i0) {
    load_rows(Qs, a.q, a, b, h, a.Hq, i0);
    load_rows(dOs, a.dout, a, b, h, a.Hq, i0);
    const int t = threadIdx.x;
    if (t < T) {
      const int i = i0 + t;
      const bool live = i < a.S;
      lse_s[t] = live ? a.lse[(static_cast<size_t>(b) * a.Hq + h) * a.S + i] : 0.f;
      dsum_s[t] = live ? a.dsum[(static_cast<size_t>(b) * a.Hq + h) * a.S + i] : 0.f;
      tau_s[t] = temp_factor(visible_keys(i, a.window), a.temp_len, a.temp_inv_log2);
    }
    if (MODE == 2) {
      for (int idx = t; idx < T * RS; idx += NTH) {
        const int rr = idx / RS, f = idx - rr * RS;
        const int i = i0 + rr;
        rS[idx] = (i < a.S && f < a.R) ? a.r[((static_cast<size_t>(b) * a.S + i) * a.Hq + h) * a.R + f] : 0.f;
      }
    }
  }

  // the key side: k and v of keys j0 .. j0 + 31 (kv head g)
  __device__ void load_keys(const BwdF32Args& a, int b, int g, int j0) {
    load_rows(Ks, a.k, a, b, g, a.Hkv, j0);
    load_rows(Vs, a.v, a, b, g, a.Hkv, j0);
  }

  // P and dZ of the block (query rows i0.., keys j0.., query head h) into Ps / Zs; thread t takes
  // row t / 8 and keys 4 (t % 8) .. + 3.  Invisible pairs get P = dZ = 0.
  __device__ void probs(const BwdF32Args& a, int h, int i0, int j0) {
    const int t = threadIdx.x;
    const int ii = t >> 3;
    const int i = i0 + ii;
    const float* qr = Qs + ii * (D + 1);
    const float* dr_ = dOs + ii * (D + 1);
    const float* bd0 = Bs - (i0 - j0 - (T - 1));   // bias parameters at distance 0
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int jj = 4 * (t & 7) + p;
      const int j = j0 + jj;
      const int delta = i - j;
      const bool vis = i < a.S && j < a.S && delta >= 0 && (a.window == 0 || delta < a.window);
      float P = 0.f, dZ = 0.f;
      if (vis) {
        const float* kr = Ks + jj * (D + 1);
        const float* vr = Vs + jj * (D + 1);
        float s = 0.f, dp = 0.f;
#pragma unroll 8
        for (int d = 0; d < D; ++d) {
          s = fmaf(qr[d], kr[d], s);
          dp = fmaf(dr_[d], vr[d], dp);
        }
        float beta = 0.f;
        if (MODE == 1 && delta < a.bias_range) beta = bd0[delta];
        if (MODE == 2 && delta < a.bias_range) {
#pragma unroll 1
          for (int f = 0; f < a.R; ++f) beta = fmaf(rS[ii * RS + f], bd0[f * NBD + delta], beta);
        }
        const float tau = tau_s[ii];
        P = expf(tau * fmaf(a.scale, s, beta) - lse_s[ii]);
        dZ = tau * P * (dp - dsum_s[ii]);
      }
      Ps[ii * (T + 1) + jj] = P;
      Zs[ii * (T + 1) + jj] = dZ;
    }
  }
};

// Query-parallel pass: workgroup = (query tile, head, batch); dq, dr and the bias-parameter
// gradients.  Thread t accumulates dq of row t / 8 at dims t % 8 + 8 u.
template <int D, int MODE>
__global__ __launch_bounds__(NTH) void bwd_f32_dq(BwdF32Args a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  Block<D, MODE> blk(sm);
  const int n_qt = (a.S + T - 1) / T;
  const int qt = blockIdx.x % n_qt;
  const int h = (blockIdx.x / n_qt) % a.Hq;
  const int b = blockIdx.x / (n_qt * a.Hq);
  const int g = h / a.G;
  const int i0 = qt * T;
  const int t = threadIdx.x;
  const int ii = t >> 3;
  const int i = i0 + ii;

  blk.load_queries(a, b, h, i0);

  constexpr int NU = D / 8;
  float acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = 0.f;
  float racc[2] = {0.f, 0.f};   // dr of row ii at features t % 8 and t % 8 + 8
  float* dEh = (MODE == 2) ? a.dE + static_cast<size_t>(h) * a.e_hs : nullptr;

  const int row_last = min(a.S, i0 + T) - 1;
  const int kmin = a.window ? max(0, i0 - a.window + 1) : 0;
  for (int j0 = kmin / T * T; j0 <= row_last; j0 += T) {
    __syncthreads();   // the previous block's reads are done
    blk.load_keys(a, b, g, j0);
    blk.load_bias(a, h, i0, j0);
    __syncthreads();
    blk.probs(a, h, i0, j0);
    __syncthreads();
    const float* zr = blk.Zs + ii * (T + 1);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int d = (t & 7) + 8 * u;
      float sacc = 0.f;
#pragma unroll 4
      for (int jj = 0; jj < T; ++jj) sacc = fmaf(zr[jj], blk.Ks[jj * (D + 1) + d], sacc);
      acc[u] += sacc;
    }
    if (MODE == 2) {
      const float* bd0 = blk.Bs - (i0 - j0 - (T - 1));   // E rows at distance 0
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int f = (t & 7) + 8 * w;
        if (f < a.R && i < a.S) {
          float s = 0.f;
#pragma unroll 4
          for (int jj = 0; jj < T; ++jj) {
            const int delta = i - (j0 + jj);
            if (delta >= 0 && delta < a.bias_range) s = fmaf(zr[jj], bd0[f * NBD + delta], s);
          }
          racc[w] += s;
        }
      }
    }
    // bias-parameter gradients: for each distance of the block (delta = i0 - j0 + e, e in
    // -31 .. 31) the sum along its diagonal, times r for dE, one atomic add per distance
    if (MODE == 1) {
      if (t < 2 * T - 1) {
        const int e = t - (T - 1);
        const int delta = i0 - j0 + e;
        if (delta >= 0 && delta < a.bias_range) {
          float s = 0.f;
#pragma unroll 4
          for (int r2 = max(0, e); r2 < min(T, T + e); ++r2) s += blk.Zs[r2 * (T + 1) + (r2 - e)];
          if (s != 0.f) atomicAdd(a.dtable + static_cast<size_t>(h) * a.bias_range + delta, s);
        }
      }
    }
    if (MODE == 2) {
      for (int idx = t; idx < (2 * T - 1) * a.R; idx += NTH) {
        const int f = idx / (2 * T - 1);
        const int e = idx - f * (2 * T - 1) - (T - 1);
        const int delta = i0 - j0 + e;
        if (delta >= 0 && delta < a.bias_range) {
          float s = 0.f;
#pragma unroll 4
          for (int r2 = max(0, e); r2 < min(T, T + e); ++r2)
            s = fmaf(blk.Zs[r2 * (T + 1) + (r2 - e)], blk.rS[r2 * RS + f], s);
          if (s != 0.f) atomicAdd(dEh + static_cast<size_t>(f) * a.bias_range + delta, s);
        }
      }
    }
  }
  if (i < a.S) {
    float* dqp = a.dq + ((static_cast<size_t>(b) * a.S + i) * a.Hq + h) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u) dqp[(t & 7) + 8 * u] = a.scale * acc[u];
    if (MODE == 2) {
      float* drp = a.dr + ((static_cast<size_t>(b) * a.S + i) * a.Hq + h) * a.R;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int f = (t & 7) + 8 * w;
        if (f < a.R) drp[f] = racc[w];
      }
    }
  }
}

// Key-parallel pass: workgroup = (key tile, kv head, batch), looping over the group's query
// heads and the query tiles that see its keys; dk and dv of key t / 8 at dims t % 8 + 8 u.
template <int D, int MODE>
__global__ __launch_bounds__(NTH) void bwd_f32_dkdv(BwdF32Args a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  Block<D, MODE> blk(sm);
  const int n_kt = (a.S + T - 1) / T;
  const int kt = blockIdx.x % n_kt;
  const int g = (blockIdx.x / n_kt) % a.Hkv;
  const int b = blockIdx.x / (n_kt * a.Hkv);
  const int j0 = kt * T;
  const int t = threadIdx.x;
  const int jj = t >> 3;
  const int j = j0 + jj;

  blk.load_keys(a, b, g, j0);

  constexpr int NU = D / 8;
  float dk[NU], dv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) dk[u] = dv[u] = 0.f;

  // query rows that see any of the keys: j0 .. (last key + window - 1), clipped to S
  const int key_last = min(a.S, j0 + T) - 1;
  const int row_end = a.window ? min(a.S - 1, key_last + a.window - 1) : a.S - 1;
  for (int hq = 0; hq < a.G; ++hq) {
    const int h = g * a.G + hq;
    for (int i0 = j0; i0 <= row_end; i0 += T) {
      __syncthreads();   // the previous block's reads are done
      blk.load_queries(a, b, h, i0);
      blk.load_bias(a, h, i0, j0);
      __syncthreads();
      blk.probs(a, h, i0, j0);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int d = (t & 7) + 8 * u;
        float sk = 0.f, sv = 0.f;
#pragma unroll 4
        for (int r2 = 0; r2 < T; ++r2) {
          sk = fmaf(blk.Zs[r2 * (T + 1) + jj], blk.Qs[r2 * (D + 1) + d], sk);
          sv = fmaf(blk.Ps[r2 * (T + 1) + jj], blk.dOs[r2 * (D + 1) + d], sv);
        }
        dk[u] += sk;
        dv[u] += sv;
      }
    }
  }
  if (j < a.S) {
    const size_t base = ((static_cast<size_t>(b) * a.S + j) * a.Hkv + g) * D;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      a.dk[base + (t & 7) + 8 * u] = a.scale * dk[u];
      a.dv[base + (t & 7) + 8 * u] = dv[u];
    }
  }
}

template <int D, int MODE>
hipError_t launch_d(const BwdF32Args& a, hipStream_t s) {
  const int lds = bwd_f32_lds_floats<D>() * 4;
  hipError_t e = set_max_lds(reinterpret_cast<const void*>(&bwd_f32_dq<D, MODE>), lds, s);
  if (e == hipSuccess) e = set_max_lds(reinterpret_cast<const void*>(&bwd_f32_dkdv<D, MODE>), lds, s);
  if (e != hipSuccess) return e;
  // the bias-parameter gradients are accumulated with atomics: cleared by the pre pass
  long long n_zero = 0;
  float* zero_dst = nullptr;
  if (MODE == 1) {
    n_zero = static_cast<long long>(a.Hq) * a.bias_range;
    zero_dst = a.dtable;
  } else if (MODE == 2) {
    n_zero = (a.e_hs ? static_cast<long long>(a.Hq) : 1LL) * a.R * a.bias_range;
    zero_dst = a.dE;
  }
  const long long rows = static_cast<long long>(a.B) * a.S * a.Hq;
  const long long pre_blocks = std::max<long long>((rows + NTH / 64 - 1) / (NTH / 64), 1);
  hipLaunchKernelGGL(bwd_f32_pre, dim3(static_cast<unsigned>(pre_blocks)), dim3(NTH), 0, s, a, n_zero, zero_dst);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_t = (a.S + T - 1) / T;
  hipLaunchKernelGGL((bwd_f32_dq<D, MODE>), dim3(static_cast<unsigned>(static_cast<long long>(n_t) * a.Hq * a.B)),
                     dim3(NTH), lds, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_f32_dkdv<D, MODE>), dim3(static_cast<unsigned>(static_cast<long long>(n_t) * a.Hkv * a.B)),
                     dim3(NTH), lds, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mode(const BwdF32Args& a, hipStream_t s) {
  if (a.mode == 1) return launch_d<D, 1>(a, s);
  if (a.mode == 2) return launch_d<D, 2>(a, s);
  return launch_d<D, 0>(a, s);
}

}  // namespace

hipError_t launch_bwd_f32(const BwdF32Args& a, hipStream_t s) {
  if (a.D == 32) return launch_mode<32>(a, s);
  if (a.D == 64) return launch_mode<64>(a, s);
  if (a.D == 128) return launch_mode<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace rba
