// Prefill: causal attention with a relative-position bias, bf16 in, fp32 MFMA
// accumulation, for gfx950 (CDNA4).
//
// The method ("Thinking Machines dropped RoPE", steps 1-5 and the kernel-cost
// section): the logit of query i and key j is scale * q_i.k_j plus a bias read
// at the distance i - j, zero at and beyond the bias range, added before the
// softmax next to the causal mask; the bias has to be formed inside the tiled
// key loop, block by block, since the full score matrix is never stored.
//
// Structure (one workgroup = 4 waves; a wave owns 32*QB query rows of one head):
//   * The scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: the key tile (from LDS) is the A operand and
//     the query rows (registers, loaded once) the B operand, so every lane owns
//     one query row.  Row max and row sum stay inside a lane except for one
//     exchange with the lane 32 apart.
//   * O^T = V^T P^T: P^T leaves the first MFMA in exactly the B-operand layout
//     of the second, so P never leaves the registers.  V^T comes from LDS,
//     where V is stored transposed with a key permutation that makes every
//     lane's 8 keys contiguous (one 16-byte LDS read).
//   * The waves of a workgroup are query heads of one GQA group (or query
//     sub-tiles of one head), so the K / V tiles in LDS serve all four.
//   * Bias, table form: read from the head's table row at the distance
//     (global memory, cached), only in key blocks that reach below the range.
//   * Bias, input-dependent form r_i . E[h, :, delta]: the curve block
//     C[delta, n] = sum_f E[h, f, delta] r[n, f] is one more MFMA per 32
//     distances (E split into a bf16 high and low part so that the product
//     keeps ~16 mantissa bits), written to a per-wave LDS scratch and read
//     back along the skewed diagonal delta = c + n - m.
//   * Key blocks wholly outside the window skip all work; blocks wholly beyond
//     the bias range skip the bias (the content-only tail of global layers).
//   * Scores are kept in the log2 domain (scale * log2 e folded into one
//     multiply, the bias pre-multiplied by log2 e) so the softmax uses v_exp_f32.

#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

constexpr int BN = 64;        // keys per LDS tile
constexpr int NWAVE = 4;
constexpr int CST = 65;       // row stride (floats) of the curve scratch

// LDS position of key x inside a 64-key V^T row: bits 2 and 3 swapped, so the
// 8 keys lane (l / 32 = h) feeds to PV MFMA (kb, kk) are contiguous.
__device__ __forceinline__ int vt_pos(int x) {
  return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

template <int D, int QB, int MODE>
__global__ __launch_bounds__(256, QB == 1 ? 2 : 1) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int KST = D + 8;          // K row stride in LDS (bf16)
  constexpr int VST = BN + 8;         // V^T row stride in LDS (bf16)
  constexpr int NC = D / 16;          // K = 16 chunks of the head dim
  constexpr int NDB = D / 32;         // 32-wide head-dim blocks of O^T
  constexpr int CS_FLOATS = (MODE == 2) ? NWAVE * 32 * CST : 1;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VST];
  __shared__ float Cs[CS_FLOATS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31;
  const int lh = lane >> 5;

  // workgroup -> (query tile, head group, batch)
  const int per_q = a.n_hgroups * a.B;
  int qt = blockIdx.x / per_q;
  const int rem = blockIdx.x - qt * per_q;
  const int hg = rem % a.n_hgroups;
  const int b = rem / a.n_hgroups;
  if (a.longest_first) qt = a.n_qtiles - 1 - qt;

  const int S = a.S;
  const int wg_i0 = qt * a.rows_wg;
  const int h = hg * a.hpw + (wave % a.hpw);
  const int hkv = h / a.G;
  const int i0 = wg_i0 + (wave / a.hpw) * (32 * QB);
  const bool wave_live = i0 < S;

  const int wg_last = min(S, wg_i0 + a.rows_wg) - 1;
  const int kmin = a.window ? max(0, wg_i0 - a.window + 1) : 0;
  const int t_begin = kmin / BN;
  const int t_end = wg_last / BN;     // inclusive

  const size_t q_row = static_cast<size_t>(a.Hq) * D;
  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const uint16_t* kbase = a.k + static_cast<size_t>(b) * S * kv_row + static_cast<size_t>(hkv) * D;
  const uint16_t* vbase = a.v + static_cast<size_t>(b) * S * kv_row + static_cast<size_t>(hkv) * D;

  // Q^T fragments (B operand): lane (n = ln, lh) holds q[row][16c + 8lh .. +7].
  bf16x8 qf[QB][NC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = i0 + 32 * qb + ln;
    const uint16_t* qp = a.q + (static_cast<size_t>(b) * S + row) * q_row + static_cast<size_t>(h) * D + 8 * lh;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < S) v = ld16(qp + 16 * c);
      qf[qb][c] = as_bf16x8(v);
    }
  }

  // r fragments (B operand of the curve MFMA): both halves carry r[row][8fc + j].
  constexpr int NFC = 2;  // up to 16 curves
  bf16x8 rf[QB][NFC];
  const int nfc = (a.R + 7) / 8;
  if (MODE == 2) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = i0 + 32 * qb + ln;
      // every load issued (row and feature clamped into range) before any is used, masked
      // afterwards as integers: no load waits behind its own branch
      const uint16_t* rp = a.r + ((static_cast<size_t>(b) * S + min(row, S - 1)) * a.Hq + h) * a.R;
      if ((a.R == 8 || a.R == 16) && (reinterpret_cast<uintptr_t>(a.r) & 15) == 0) {
        // R = 8 or 16, r 16-byte aligned: a lane's features are one or two 16-byte loads
#pragma unroll
        for (int fc = 0; fc < NFC; ++fc) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (8 * fc < a.R) v = ld16(rp + 8 * fc);
          const uint32_t keep = row < S ? ~0u : 0u;
          rf[qb][fc] = as_bf16x8(u32x4{v[0] & keep, v[1] & keep, v[2] & keep, v[3] & keep});
        }
        continue;
      }
      uint32_t raw[8 * NFC];
#pragma unroll
      for (int f = 0; f < 8 * NFC; ++f) raw[f] = rp[min(f, a.R - 1)];
#pragma unroll
      for (int fc = 0; fc < NFC; ++fc) {
        uint32_t w[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int f0 = 8 * fc + 2 * jj;
          const uint32_t lo = raw[f0] & ((row < S && f0 < a.R) ? 0xFFFFu : 0u);
          const uint32_t hi = raw[f0 + 1] & ((row < S && f0 + 1 < a.R) ? 0xFFFFu : 0u);
          w[jj] = lo | (hi << 16);
        }
        rf[qb][fc] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
      }
    }
  }

  float m_run[QB], l_run[QB];
  f32x16 oacc[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.f;
  }

  const float NEG_INF = -INFINITY;
  float* cs = Cs + (MODE == 2 ? wave * 32 * CST : 0);
  const float* tab = (MODE == 1) ? a.table + static_cast<size_t>(h) * a.bias_range : nullptr;
  const float* Eh = (MODE == 2) ? a.E + static_cast<size_t>(h) * a.e_hs : nullptr;

  for (int t = t_begin; t <= t_end; ++t) {
    const int tk0 = t * BN;
    __syncthreads();  // the previous tile's LDS reads are complete
    // K tile: row-major copy, 16 bytes per thread per step (coalesced rows).
#pragma unroll
    for (int it = 0; it < (BN * D / 8) / 256; ++it) {
      const int idx = it * 256 + tid;
      const int row = idx / (D / 8);
      const int ch = idx % (D / 8);
      const int key = tk0 + row;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key < S) v = ld16(kbase + static_cast<size_t>(key) * kv_row + 8 * ch);
      st16(Ks + row * KST + 8 * ch, v);
    }
    // V tile, transposed: a thread takes 4 consecutive keys x 8 head dims.
    if (tid < (BN / 4) * (D / 8)) {
      const int kg = tid & 15;
      const int dg = tid >> 4;
      u32x4 rows[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int key = tk0 + 4 * kg + s;
        rows[s] = u32x4{0u, 0u, 0u, 0u};
        if (key < S) rows[s] = ld16(vbase + static_cast<size_t>(key) * kv_row + 8 * dg);
      }
      const int pos = vt_pos(4 * kg);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const int sh = (e & 1) * 16;
        const uint32_t k0 = (rows[0][w] >> sh) & 0xffffu;
        const uint32_t k1 = (rows[1][w] >> sh) & 0xffffu;
        const uint32_t k2 = (rows[2][w] >> sh) & 0xffffu;
        const uint32_t k3 = (rows[3][w] >> sh) & 0xffffu;
        st8(Vt + (8 * dg + e) * VST + pos, u32x2{k0 | (k1 << 16), k2 | (k3 << 16)});
      }
    }
    __syncthreads();
    if (!wave_live) continue;

    // ---- S^T = K Q^T for every (query block, key block) of this tile -------------
    f32x16 sacc[QB][2];
    bool on[QB][2];
    bool any_on = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int c = (i0 + 32 * qb) - (tk0 + 32 * kb);   // delta = c + n - m
        bool o = (c + 31 >= 0) && (tk0 + 32 * kb < S) && (i0 + 32 * qb < S);
        if (a.window) o = o && (c - 31 < a.window);
        on[qb][kb] = o;
        any_on |= o;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[qb][kb][i] = 0.f;
      }
    if (!any_on) continue;

#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 kf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        kf[kb] = as_bf16x8(ld16(Ks + (32 * kb + ln) * KST + 16 * c + 8 * lh));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (on[qb][kb]) sacc[qb][kb] = mfma32(kf[kb], qf[qb][c], sacc[qb][kb]);
    }

    // ---- log2-domain logits, bias, mask, online softmax, P -------------------------
    bf16x8 pf[QB][2][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (!on[qb][0] && !on[qb][1]) continue;
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!on[qb][kb]) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[qb][kb][i] = NEG_INF;
          continue;
        }
        const int c = (i0 + 32 * qb) - (tk0 + 32 * kb);
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[qb][kb][i] *= a.c_qk;
        const bool inband = (MODE != 0) && (c - 31 < a.bias_range);
        if (MODE == 1 && inband) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + 4 * lh + (i & 3);
            const int d = c + ln - m;
            const int dc = min(max(d, 0), a.bias_range - 1);
            const float tv = tab[dc];
            sacc[qb][kb][i] += (d >= 0 && d < a.bias_range) ? tv * kLog2e : 0.f;
          }
        }
        if (MODE == 2 && inband) {
          // Two 32-distance curve blocks cover delta in [c - 31, c + 32].
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int d0 = c - 31 + 32 * half;
            const int dl = d0 + ln;              // A-operand row: distance d0 + ln
            const bool dok = dl >= 0 && dl < a.bias_range;
            // the block's E values all requested (distance and feature clamped into range)
            // before any is used, masked afterwards as integers
            const float* ep = Eh + min(max(dl, 0), a.bias_range - 1);
            uint32_t raw[8 * NFC];
#pragma unroll
            for (int f = 0; f < 8 * NFC; ++f) raw[f] = __float_as_uint(ep[static_cast<size_t>(min(f, a.R - 1)) * a.bias_range]);
            f32x16 cacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) cacc[i] = 0.f;
#pragma unroll
            for (int fc = 0; fc < NFC; ++fc) {
              if (fc >= nfc) break;
              uint32_t w[4];
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                float e2[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                  const int f = 8 * fc + 2 * jj + u;
                  const uint32_t keep = (f < a.R && dok) ? ~0u : 0u;
                  const float e = __uint_as_float(__float_as_uint(__uint_as_float(raw[f]) * kLog2e) & keep);
                  const float hi = bf16_to_f32(f32_to_bf16(e));
                  e2[u] = lh ? (e - hi) : e;      // lane half 1 feeds the low part
                }
                w[jj] = pack_bf16x2(e2[0], e2[1]);
              }
              cacc = mfma32(as_bf16x8(u32x4{w[0], w[1], w[2], w[3]}), rf[qb][fc], cacc);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int sidx = 8 * (i >> 2) + 4 * lh + (i & 3);
              cs[ln * CST + 32 * half + sidx] = cacc[i];
            }
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + 4 * lh + (i & 3);
            sacc[qb][kb][i] += cs[ln * CST + (ln - m + 31)];
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        if (a.temp_len) {   // context-length temperature of the lane's query row, on q.k and bias
          const float tq = temp_factor(visible_keys(i0 + 32 * qb + ln, a.window), a.temp_len, a.temp_inv_log2);
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[qb][kb][i] *= tq;
        }
        const bool edge = (c - 31 < 0) || (a.window && c + 31 >= a.window);
        if (edge) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + 4 * lh + (i & 3);
            const int d = c + ln - m;
            if (d < 0 || (a.window && d >= a.window)) sacc[qb][kb][i] = NEG_INF;
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[qb][kb][i]);
      }
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run[qb], mx);
      const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[qb] - m_use);
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          uint32_t w[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float p0 = fast_exp2(sacc[qb][kb][8 * kk + 2 * jj] - m_use);
            const float p1 = fast_exp2(sacc[qb][kb][8 * kk + 2 * jj + 1] - m_use);
            psum += p0 + p1;
            w[jj] = pack_bf16x2(p0, p1);
          }
          pf[qb][kb][kk] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
        }
      }
      l_run[qb] = l_run[qb] * alpha + psum;
      m_run[qb] = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[qb][db][i] *= alpha;
    }

    // ---- O^T += V^T P^T ---------------------------------------------------------------
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 vf = as_bf16x8(ld16(Vt + (32 * db + ln) * VST + 32 * kb + 16 * kk + 8 * lh));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if (on[qb][kb]) oacc[qb][db] = mfma32(vf, pf[qb][kb][kk], oacc[qb][db]);
        }
  }

  if (!wave_live) return;
  // ---- epilogue: normalise, store O (bf16) and the log-sum-exp ---------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = i0 + 32 * qb + ln;
    const float lt = l_run[qb] + xor32(l_run[qb]);
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

template <int D, int QB, int MODE>
hipError_t launch_one(const FwdArgs& a0, hipStream_t s) {
  FwdArgs a = a0;
  a.rows_wg = 32 * QB * (NWAVE / a.hpw);
  a.n_qtiles = (a.S + a.rows_wg - 1) / a.rows_wg;
  a.n_hgroups = a.Hq / a.hpw;
  a.longest_first = (a.window == 0 || a.window > a.rows_wg) ? 1 : 0;
  const long long nblk = static_cast<long long>(a.n_qtiles) * a.n_hgroups * a.B;
  if (nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, MODE>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, int QB>
hipError_t launch_mode(const FwdArgs& a, int mode, hipStream_t s) {
  switch (mode) {
    case 0: return launch_one<D, QB, 0>(a, s);
    case 1: return launch_one<D, QB, 1>(a, s);
    default: return launch_one<D, QB, 2>(a, s);
  }
}

}  // namespace

namespace {
// The MFMA kernels address K and V through 32-bit buffer offsets within one sequence.
bool kv_off32(const FwdArgs& a, int D) { return static_cast<long long>(a.S) * a.Hkv * D * 2 < (1LL << 31); }
// Every layer the split kernel's domain covers takes it (head_dim 128, GQA groups of 4k heads,
// positive scale, LDS within half a CU: its 32-row workgroups pair up on a CU and it reads E rows
// converted once per call).  The kernel above takes the other shapes: head_dim 64, other group
// sizes, ranges off the 4-distance grid, a table range too long for the split kernel's LDS.
bool use_split(const FwdArgs& a, int D, int mode) {
  return kv_off32(a, D) &&
         fwd_split_workspace(D, a.G, mode, a.bias_range, a.R, a.e_hs == 0, a.Hq, a.c_qk) >= 0;
}
}  // namespace

long long fwd_bf16_workspace(const FwdArgs& a, int D, int mode) {
  if (!use_split(a, D, mode)) return 0;
  const long long n = fwd_split_workspace(D, a.G, mode, a.bias_range, a.R, a.e_hs == 0, a.Hq, a.c_qk);
  return (n + 255) / 256 * 256;
}

hipError_t launch_fwd_bf16(const FwdArgs& a0, int D, int mode, void* workspace, hipStream_t s) {
  if (use_split(a0, D, mode)) return launch_fwd_bf16_split(a0, mode, workspace, s);
  FwdArgs a = a0;
  a.hpw = (a.G % 4 == 0) ? 4 : (a.G % 2 == 0 ? 2 : 1);
  if (D == 128) return launch_mode<128, 1>(a, mode, s);
  return launch_mode<64, 1>(a, mode, s);
}

}  // namespace rba
