// fp32 attention with a relative-position bias on the vector ALUs (no bf16
// anywhere): used for fp32 prefill and fp32 decode.  A workgroup of 4 waves handles 64
// consecutive query rows of one head (lane = row); key tiles of 64 rows are staged in LDS, and
// wave w runs an online softmax over the keys 4 i + w of each tile that its rows can see, so a
// short problem still spreads its per-row key loop over four waves.  The four partial results
// (running max, sum and accumulator, in the log2 domain) are merged through LDS at the end.
//
// Same operation as the bf16 kernels: logit = scale * q.k + bias(delta), bias
// zero at and beyond the range, causal / sliding-window visibility
// ("Learned Relative-Position Bias", section "Standard Relative Bias
// (T5-style)"; "Thinking Machines dropped RoPE", steps 3-5).

#include <algorithm>

#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

constexpr int TK = 64;
constexpr int NW = 4;   // waves per workgroup, splitting each tile's keys

constexpr int NDS = 2 * TK;   // distances a tile's pairs span (64 rows x TK keys)
constexpr int RMAX_F32 = 16;

template <int D>
constexpr int f32_lds_floats() {
  // K and V tiles and the tile's bias parameters (table entries or E rows over its distance
  // span) during the key loop; the merge buffers after it
  return std::max(2 * TK * (D + 1) + RMAX_F32 * NDS, 2 * NW * 64 + (NW - 1) * 64 * 33);
}

template <int D>
__global__ __launch_bounds__(64 * NW) void attn_f32_kernel(F32Args a) {
  __shared__ float sm[f32_lds_floats<D>()];
  float (*Kt)[D + 1] = reinterpret_cast<float (*)[D + 1]>(sm);
  float (*Vt)[D + 1] = reinterpret_cast<float (*)[D + 1]>(sm + TK * (D + 1));
  float* bs = sm + 2 * TK * (D + 1);   // [R][NDS] E rows, or [NDS] table entries, of the tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qtiles = (a.Sq + 63) / 64;
  const int qt = blockIdx.x % qtiles;
  const int h = (blockIdx.x / qtiles) % a.Hq;
  const int b = blockIdx.x / (qtiles * a.Hq);
  const int g = h / a.G;
  const int qi = qt * 64 + lane;
  const bool live = qi < a.Sq;
  const int pos = a.q_pos0 + qi;

  float qv[D], acc[D];
  const float* qp = a.q + ((static_cast<size_t>(b) * a.Sq + (live ? qi : 0)) * a.Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = live ? qp[d] : 0.f;
    acc[d] = 0.f;
  }
  float rv[16];
  if (a.mode == 2) {
    const float* rp = a.r + ((static_cast<size_t>(b) * a.Sq + (live ? qi : 0)) * a.Hq + h) * a.R;
#pragma unroll
    for (int f = 0; f < 16; ++f) rv[f] = (f < a.R && live) ? rp[f] : 0.f;
  }
  // running max and sum in the log2 domain (logit x log2(e))
  float m = -INFINITY, l = 0.f;
  // context-length temperature of this query (keys 0..pos exist), on q.k and bias alike
  const float tq = temp_factor(visible_keys(pos, a.window), a.temp_len, a.temp_inv_log2);
  const float c2 = tq * kLog2e;

  // keys any row of this tile can see
  const int pos_lo = a.q_pos0 + qt * 64;
  const int pos_hi = a.q_pos0 + min(a.Sq, qt * 64 + 64) - 1;
  const int kbeg = a.window ? max(0, pos_lo - a.window + 1) : 0;
  const int kend = min(a.Lk - 1, pos_hi);
  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const float* kb = a.k + static_cast<size_t>(b) * a.kv_rows * kv_row + static_cast<size_t>(g) * D;
  const float* vb = a.v + static_cast<size_t>(b) * a.kv_rows * kv_row + static_cast<size_t>(g) * D;

  const int nb = a.mode == 2 ? a.R : 1;   // bias parameters per distance
  const float* bsrc = a.mode == 2 ? a.E + static_cast<size_t>(h) * a.e_hs
                                  : (a.mode == 1 ? a.table + static_cast<size_t>(h) * a.bias_range : nullptr);
  for (int t0 = kbeg; t0 <= kend; t0 += TK) {
    __syncthreads();
    // the tile's K and V rows and its bias parameters, each with 8 loads in flight per thread
    // (rows past kend read row kend and are stored as zero)
    auto load_kv = [&](const float* base) {
      return [=](int idx) {
        const int key = min(t0 + idx / D, kend);
        return __float_as_uint(base[static_cast<size_t>(key) * kv_row + idx % D]);
      };
    };
    auto store_kv = [&](float (*tile)[D + 1]) {
      return [=](int idx, uint32_t w) {
        const int row = idx / D;
        tile[row][idx % D] = __uint_as_float(w & ((t0 + row <= kend) ? ~0u : 0u));
      };
    };
    stage_batched(tid, 64 * NW, TK * D, load_kv(kb), store_kv(Kt));
    stage_batched(tid, 64 * NW, TK * D, load_kv(vb), store_kv(Vt));
    // distances dmin .. dmin + NDS - 1 cover every pair of this tile; entries outside
    // [0, bias_range) are zero (and never read)
    const int dmin = pos_lo - (t0 + TK - 1);
    if (a.mode != 0 && a.bias_range > 0)
      stage_batched(tid, 64 * NW, nb * NDS,
          [&](int x) {
            const int f = x / NDS;
            const int d = min(max(dmin + x - f * NDS, 0), a.bias_range - 1);
            return __float_as_uint(bsrc[static_cast<size_t>(f) * a.bias_range + d]);
          },
          [&](int x, uint32_t w) {
            const int d = dmin + x - (x / NDS) * NDS;
            bs[x] = __uint_as_float(w & ((d >= 0 && d < a.bias_range) ? ~0u : 0u));
          });
    __syncthreads();
    if (!live) continue;
    const int n = min(TK, kend - t0 + 1);
    for (int jj = wave; jj < n; jj += NW) {
      const int key = t0 + jj;
      const int delta = pos - key;
      if (delta < 0 || (a.window && delta >= a.window)) continue;
      float sp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < D; ++d) sp[d & 3] = fmaf(qv[d], Kt[jj][d], sp[d & 3]);
      float s = ((sp[0] + sp[1]) + (sp[2] + sp[3])) * a.scale;
      if (a.mode != 0 && delta < a.bias_range) {
        const float* bd = bs + (delta - (pos_lo - (t0 + TK - 1)));
        if (a.mode == 1) {
          s += bd[0];
        } else {
          float bsum = 0.f;
#pragma unroll
          for (int f = 0; f < RMAX_F32; ++f)
            if (f < a.R) bsum = fmaf(rv[f], bd[f * NDS], bsum);
          s += bsum;
        }
      }
      s *= c2;
      const float m_new = fmaxf(m, s);
      const float alpha = fast_exp2(m - m_new);
      const float p = fast_exp2(s - m_new);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Vt[jj][d], acc[d] * alpha);
      m = m_new;
    }
  }

  // ---- merge the four waves' partials of each row: max, then sums rescaled to it ----------
  float* cm = sm;                    // [NW][64] running maxima
  float* cl = sm + NW * 64;          // [NW][64] running sums
  float* cacc = sm + 2 * NW * 64;    // [NW - 1][64][33] accumulator chunks of waves 1..3
  __syncthreads();                   // the tiles are dead
  cm[wave * 64 + lane] = m;
  cl[wave * 64 + lane] = l;
  __syncthreads();
  float M = cm[lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, cm[w * 64 + lane]);
  // every row sees its own key, so M is finite for live rows; a wave that saw none of the
  // row's keys has m = -inf and contributes zero
  float ltot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float mw = cm[w * 64 + lane];
    ltot += (mw == -INFINITY) ? 0.f : cl[w * 64 + lane] * fast_exp2(mw - M);
  }
  const float own = (m == -INFINITY || !live) ? 0.f : fast_exp2(m - M);
#pragma unroll
  for (int dc = 0; dc < D / 32; ++dc) {
    __syncthreads();   // the previous chunk has been read
    if (wave > 0) {
#pragma unroll
      for (int k = 0; k < 32; ++k) cacc[((wave - 1) * 64 + lane) * 33 + k] = acc[32 * dc + k] * own;
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        float x = acc[32 * dc + k] * own;
#pragma unroll
        for (int w = 1; w < NW; ++w) x += cacc[((w - 1) * 64 + lane) * 33 + k];
        acc[32 * dc + k] = x;
      }
    }
  }
  if (wave != 0 || !live) return;
  const float inv = 1.f / ltot;
  float* op = a.o + ((static_cast<size_t>(b) * a.Sq + qi) * a.Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
  if (a.lse) a.lse[(static_cast<size_t>(b) * a.Hq + h) * a.Sq + qi] = (M + fast_log2(ltot)) * kLn2;
}

}  // namespace

hipError_t launch_attn_f32(const F32Args& a, hipStream_t s) {
  const long long nblk = static_cast<long long>((a.Sq + 63) / 64) * a.Hq * a.B;
  if (nblk <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nblk));
  switch (a.D) {
    case 32: hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(64 * NW), 0, s, a); break;
    case 64: hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64 * NW), 0, s, a); break;
    default: hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64 * NW), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace rba
