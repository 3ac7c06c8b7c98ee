// fp32 attention with a relative-position bias on the vector ALUs (no bf16
// anywhere): used for fp32 prefill and fp32 decode.  One wave handles 64
// consecutive query rows of one head; key tiles of 64 rows are staged in LDS
// and each lane runs an online softmax over the keys its row can see.
//
// Same operation as the bf16 kernels: logit = scale * q.k + bias(delta), bias
// zero at and beyond the range, causal / sliding-window visibility
// ("Learned Relative-Position Bias", section "Standard Relative Bias
// (T5-style)"; "Thinking Machines dropped RoPE", steps 3-5).

#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

constexpr int TK = 64;

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(F32Args a) {
  __shared__ float Kt[TK][D + 1];
  __shared__ float Vt[TK][D + 1];

  const int lane = threadIdx.x;
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
  float m = -INFINITY, l = 0.f;
  // context-length temperature of this query (keys 0..pos exist), on q.k and bias alike
  const float tq = temp_factor(visible_keys(pos, a.window), a.temp_len, a.temp_inv_log2);

  // keys any row of this tile can see
  const int pos_lo = a.q_pos0 + qt * 64;
  const int pos_hi = a.q_pos0 + min(a.Sq, qt * 64 + 64) - 1;
  const int kbeg = a.window ? max(0, pos_lo - a.window + 1) : 0;
  const int kend = min(a.Lk - 1, pos_hi);
  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const float* kb = a.k + static_cast<size_t>(b) * a.kv_rows * kv_row + static_cast<size_t>(g) * D;
  const float* vb = a.v + static_cast<size_t>(b) * a.kv_rows * kv_row + static_cast<size_t>(g) * D;

  for (int t0 = kbeg; t0 <= kend; t0 += TK) {
    __syncthreads();
    for (int idx = lane; idx < TK * D; idx += 64) {
      const int row = idx / D, d = idx % D;
      const int key = t0 + row;
      const bool ok = key <= kend;
      Kt[row][d] = ok ? kb[static_cast<size_t>(key) * kv_row + d] : 0.f;
      Vt[row][d] = ok ? vb[static_cast<size_t>(key) * kv_row + d] : 0.f;
    }
    __syncthreads();
    if (!live) continue;
    const int n = min(TK, kend - t0 + 1);
    for (int jj = 0; jj < n; ++jj) {
      const int key = t0 + jj;
      const int delta = pos - key;
      if (delta < 0 || (a.window && delta >= a.window)) continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qv[d], Kt[jj][d], s);
      s *= a.scale;
      if (a.mode != 0 && delta < a.bias_range) {
        if (a.mode == 1) {
          s += a.table[static_cast<size_t>(h) * a.bias_range + delta];
        } else {
          const float* Eh = a.E + static_cast<size_t>(h) * a.e_hs + delta;
          float bsum = 0.f;
#pragma unroll
          for (int f = 0; f < 16; ++f)
            if (f < a.R) bsum = fmaf(rv[f], Eh[static_cast<size_t>(f) * a.bias_range], bsum);
          s += bsum;
        }
      }
      s *= tq;
      const float m_new = fmaxf(m, s);
      const float alpha = expf(m - m_new);
      const float p = expf(s - m_new);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Vt[jj][d], acc[d] * alpha);
      m = m_new;
    }
  }
  if (!live) return;
  const float inv = 1.f / l;
  float* op = a.o + ((static_cast<size_t>(b) * a.Sq + qi) * a.Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
  if (a.lse) a.lse[(static_cast<size_t>(b) * a.Hq + h) * a.Sq + qi] = m + logf(l);
}

}  // namespace

hipError_t launch_attn_f32(const F32Args& a, hipStream_t s) {
  const long long nblk = static_cast<long long>((a.Sq + 63) / 64) * a.Hq * a.B;
  if (nblk <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nblk));
  switch (a.D) {
    case 32: hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(64), 0, s, a); break;
    case 64: hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, s, a); break;
    default: hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace rba
