// Single-token decode with a relative-position bias, bf16 KV cache, gfx950.
//
// One new query per sequence at position kv_len - 1 attends to cache rows
// [max(0, kv_len - window), kv_len).  Only the last bias_range rows carry a
// bias; every older row is content-only (the NoPE tail of global layers,
// "Learned Relative-Position Bias", section "Inkling's Input-Dependent Version
// (Conceptual)"), so only the chunk holding those rows evaluates it.
//
// The step is bound by streaming K and V from HBM.  Grid = (split, kv head,
// batch); each of the 4 waves of a workgroup streams its own contiguous run of
// cache rows, 32 at a time, with the next tile's loads in flight during the current one:
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16, the K rows loaded straight from
//     global memory into the A operand (16 bytes per lane, no LDS), the G query
//     heads of the kv head as B-operand columns;
//   * V is staged in a wave-private LDS tile, transposed, and O^T = V^T P^T
//     runs on the same MFMA with P kept in registers;
//   * the bias curve of a tile's 32 distances (table row or r.E) is evaluated by its wave
//     during the previous tile, into a wave-private LDS buffer read once per logit;
//   * the 4 waves merge (max / sum-exp) through LDS; with several splits the
//     workgroup writes an unnormalised partial that a second kernel combines.

#include <mutex>
#include <type_traits>

#include "relbias_attn.h"
#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

constexpr int TK = 32;          // cache rows per tile (one 32x32 MFMA block)

#ifndef RBA_DECODE_TARGET_WG
#define RBA_DECODE_TARGET_WG 2048   // workgroups the split aims for
#endif
#ifndef RBA_DECODE_MIN_ROWS
#define RBA_DECODE_MIN_ROWS 128     // fewest cache rows per wave
#endif

__device__ __forceinline__ int vt_pos(int x) {
  return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// 8 MXFP4 codes (element 2j in the low nibble of byte j) times the block scale -> 8 bf16,
// with the hardware FP4 conversion (v_cvt_scalef32_pk_bf16_fp4, one byte per instruction).
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t codes, float sc) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3))};
}
// E8M0 scale byte -> 2^(byte - 127) as fp32 (byte 0, an all-zero block, reads as 0).
__device__ __forceinline__ float e8m0(uint32_t byte) { return __uint_as_float(byte << 23); }

// V items of a tile: 4 cache rows (keys 4 kg .. + 3, kg = lane % 8) x 8 head dims (8 dg .. + 7).
// Item it of lane l covers dims group dg: (l + 64 it) / 8 in general; with MXFP4 caches and two
// items per lane, 2 (l / 8) + it, so that the lane's two items are adjacent dims of the same rows
// (one 8-byte code load and one scale byte per row instead of two of each).
template <bool FP4, int NVI>
__device__ __forceinline__ int v_item_dg(int lane, int it) {
  return (FP4 && NVI == 2) ? 2 * (lane >> 3) + it : (lane + 64 * it) >> 3;
}

// RMAX: r.E features held per curve item (8 or 16; 1 for the table).  FP4: MXFP4 caches (codes
// and scales as in the 16x16 kernel below); a lane half's K fragments then cover head dims
// (D / 2) lh + 8 c .. + 7, one or two 16-byte code loads and D / 64 scale bytes per row, and the
// query fragments use the same dims; V rows arrive as 8-dim pieces of 4 code bytes and a scale.
template <int D, int MODE, int RMAX, bool FP4 = false>
__global__ __launch_bounds__(256, 2) void decode_bf16_kernel(DecodeArgs a, int curve_off) {
  constexpr int VST = TK + 8;          // V^T row stride (bf16): 80-byte rows, 16-byte aligned
  constexpr int NC = D / 16;           // K = 16 chunks of the head dim
  constexpr int NDB = D / 32;          // 32-wide head-dim blocks of O^T
  constexpr int NVI = (TK / 4) * (D / 8) / 64;   // V items (4 rows x 8 dims) per lane
  constexpr int VT_BYTES = D * VST * 2;          // per wave
  // dynamic LDS: [4 x V^T tile | merge buffer, when larger] then the bias curve [G][n_curve]
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 31;
  const int lh = lane >> 5;
  const int split = blockIdx.x;
  const int hkv = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.G;
  const int h = hkv * G + ln;            // query head of this lane's column (valid if ln < G)
  const bool col_live = ln < G;

  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const bool paged = a.block_table != nullptr;
  // this sequence's cache length (paged: per sequence, clamped to the bound the launch was
  // sized for) and first visible row
  const int kv_len = paged ? min(max(a.kv_lens[b], 0), a.kv_len) : a.kv_len;
  const int key_begin = paged ? (a.window ? max(0, kv_len - a.window) : 0) : a.key_begin;
  // context-length temperature of this sequence's query, on q.k and bias alike
  const float tq = temp_factor(visible_keys(kv_len - 1, a.window), a.temp_len, a.temp_inv_log2);
  const float c_qk = a.c_qk * tq;
  const float c_bias = kLog2e * tq;
  const uint16_t* kbase = a.k + static_cast<size_t>(hkv) * D + (paged ? 0 : static_cast<size_t>(b) * a.L_max * kv_row);
  const uint16_t* vbase = a.v + static_cast<size_t>(hkv) * D + (paged ? 0 : static_cast<size_t>(b) * a.L_max * kv_row);
  const int* bt = paged ? a.block_table + static_cast<size_t>(b) * a.max_pages : nullptr;
  // pool row of cache row `key` of this sequence (paged), page index clamped into the pool
  auto pool_row = [&](int key) -> int {
    const int pg = min(max(bt[key / a.page_size], 0), a.num_pages - 1);
    return pg * a.page_size + key % a.page_size;
  };
  const int qpos = kv_len - 1;

  // This wave's rows.
  const int w_beg = key_begin + (split * 4 + wave) * a.keys_per_wave;
  const int w_end = min(kv_len, w_beg + a.keys_per_wave);
  const int ntiles = w_end > w_beg ? (w_end - w_beg + TK - 1) / TK : 0;

  // ---- registers of the tile in flight: K as MFMA A-operand fragments, V as row pieces ---
  u32x4 kreg[FP4 ? 1 : NC], vreg[NVI][FP4 ? 1 : 4];
  // FP4: a lane half's D / 4 code bytes and D / 64 scale bytes per K row, 4 code bytes and a
  // scale byte per V piece
  constexpr int NKB = FP4 ? D / 64 : 1;   // 16-byte code loads (and scale blocks) per K row
  u32x4 kc[NKB];
  uint32_t ksb[NKB], vc[NVI][4], vsb[NVI][4];
  constexpr int CB = D / 2, SB = D / 32;
  const size_t crow = static_cast<size_t>(a.Hkv) * CB, srow = static_cast<size_t>(a.Hkv) * SB;
  const size_t cbatch = paged ? 0 : static_cast<size_t>(b) * a.L_max;
  const uint8_t* kcb = reinterpret_cast<const uint8_t*>(a.k) + (cbatch * a.Hkv + hkv) * CB;
  const uint8_t* vcb = reinterpret_cast<const uint8_t*>(a.v) + (cbatch * a.Hkv + hkv) * CB;
  const uint8_t* ksp = FP4 ? a.k_scale + (cbatch * a.Hkv + hkv) * SB : nullptr;
  const uint8_t* vsp = FP4 ? a.v_scale + (cbatch * a.Hkv + hkv) * SB : nullptr;
  auto load_tile = [&](int tk0) {
    const int key = tk0 + ln;
    // paged: one table read per lane (its K row); the V rows take theirs from the K lanes
    const int prow = paged ? (key < w_end ? pool_row(key) : 0) : key;
    if constexpr (FP4) {
      const uint8_t* kp = kcb + static_cast<size_t>(prow) * crow + (D / 4) * lh;
#pragma unroll
      for (int u = 0; u < NKB; ++u) {
        kc[u] = u32x4{0u, 0u, 0u, 0u};
        ksb[u] = 0u;
        if (key < w_end) {
          kc[u] = ld16(kp + 16 * u);
          ksb[u] = ksp[static_cast<size_t>(prow) * srow + NKB * lh + u];
        }
      }
    } else {
      const uint16_t* kp = kbase + static_cast<size_t>(prow) * kv_row + 8 * lh;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        kreg[c] = u32x4{0u, 0u, 0u, 0u};
        if (key < w_end) kreg[c] = ld16(kp + 16 * c);
      }
    }
    if constexpr (FP4 && NVI == 2) {
      // the lane's two V items are dims 16 (l / 8) .. + 15 of the same 4 rows: one 8-byte code
      // load and one scale byte per row (both halves lie in one 32-dim scale block)
      const int kg = lane & 7;
      const int dg0 = v_item_dg<FP4, NVI>(lane, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kk = tk0 + 4 * kg + s;
        const int vrow = paged ? __shfl(prow, 4 * kg + s, 64) : kk;
        vc[0][s] = vc[1][s] = 0u;
        vsb[0][s] = vsb[1][s] = 0u;
        if (kk < w_end) {
          const u32x2 w2 = ld8(vcb + static_cast<size_t>(vrow) * crow + 4 * dg0);
          vc[0][s] = w2[0];
          vc[1][s] = w2[1];
          vsb[0][s] = vsb[1][s] = vsp[static_cast<size_t>(vrow) * srow + (dg0 >> 2)];
        }
      }
    } else {
#pragma unroll
    for (int it = 0; it < NVI; ++it) {
      const int item = lane + 64 * it;
      const int kg = item & 7;
      const int dg = item >> 3;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kk = tk0 + 4 * kg + s;
        const int vrow = paged ? __shfl(prow, 4 * kg + s, 64) : kk;
        if constexpr (FP4) {
          vc[it][s] = 0u;
          vsb[it][s] = 0u;
          if (kk < w_end) {
            vc[it][s] = *reinterpret_cast<const uint32_t*>(vcb + static_cast<size_t>(vrow) * crow + 4 * dg);
            vsb[it][s] = vsp[static_cast<size_t>(vrow) * srow + (dg >> 2)];
          }
        } else {
          vreg[it][s] = u32x4{0u, 0u, 0u, 0u};
          if (kk < w_end) vreg[it][s] = ld16(vbase + static_cast<size_t>(vrow) * kv_row + 8 * dg);
        }
      }
    }
    }
  };

  bf16x8 qf[NC];
  {
    const uint16_t* qp = a.q + (static_cast<size_t>(b) * a.Hq + (col_live ? h : 0)) * D + (FP4 ? (D / 2) * lh : 8 * lh);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (col_live) v = ld16(qp + (FP4 ? 8 * c : 16 * c));
      qf[c] = as_bf16x8(v);
    }
  }
  if (ntiles > 0) load_tile(w_beg);

  // ---- bias: each wave evaluates the curve of the next tile's 32 distances while the current
  // tile is processed, into a wave-private pair of buffers [G][TK] (log2 units).  The curve of
  // query head n at distance delta is table[h, delta] or sum_f r[b, h, f] E[h, f, delta]; it is
  // zero at and beyond bias_range.  r is staged once per workgroup.
  float* rs = reinterpret_cast<float*>(smem + curve_off);                  // [G][R] (r.E)
  float* cbuf = rs + (MODE == 2 ? G * a.R : 0) + wave * 2 * G * TK;         // [2][G][TK]
  if (MODE == 2) {
    for (int i = tid; i < G * a.R; i += 256)
      rs[i] = bf16_to_f32(a.r[(static_cast<size_t>(b) * a.Hq + hkv * G) * a.R + i]);
    __syncthreads();
  }
  // items (n, j) of a tile curve: head n < G, row j < TK; lane l takes items l, l + 64, ...
  const int n_items = G * TK;
  auto tile_in_band = [&](int tk0) { return MODE != 0 && qpos - (tk0 + TK - 1) < a.bias_range; };
  // The first 128 items of a tile curve are fetched early (next to the tile's K/V loads) into
  // registers and finished after the current tile; larger groups do the rest in place.
  float epre[2][RMAX];
  auto item_geo = [&](int tk0, int item, int& n, int& d, bool& live) {
    n = item / TK;
    const int j = item - n * TK;
    d = qpos - (tk0 + j);
    live = item < n_items && d >= 0 && d < a.bias_range && tk0 + j < w_end;
    if (item >= n_items) n = 0;
  };
  auto fetch_items = [&](int tk0, int base, float (&e)[2][RMAX]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int n, d;
      bool live;
      item_geo(tk0, base + lane + 64 * u, n, d, live);
      const int hh = hkv * G + n;
      if (MODE == 1) {
        e[u][0] = live ? a.table[static_cast<size_t>(hh) * a.bias_range + d] : 0.f;
      } else {
        const float* ep = a.E + static_cast<size_t>(hh) * a.e_hs + (live ? d : 0);
#pragma unroll
        for (int f = 0; f < RMAX; ++f) e[u][f] = (live && f < a.R) ? ep[static_cast<size_t>(f) * a.bias_range] : 0.f;
      }
    }
  };
  auto finish_items = [&](int tk0, int base, const float (&e)[2][RMAX], float* dst) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int item = base + lane + 64 * u;
      int n, d;
      bool live;
      item_geo(tk0, item, n, d, live);
      float acc = 0.f;
      if (MODE == 1) {
        acc = e[u][0];
      } else {
#pragma unroll
        for (int f = 0; f < RMAX; ++f)
          if (f < a.R) acc = fmaf(rs[n * a.R + f], e[u][f], acc);
      }
      if (item < n_items) dst[item] = acc * c_bias;
    }
  };
  auto curve_finish = [&](int tk0, float* dst) {
    finish_items(tk0, 0, epre, dst);
    for (int base = 128; base < n_items; base += 128) {
      float e[2][RMAX];
      fetch_items(tk0, base, e);
      finish_items(tk0, base, e, dst);
    }
  };
  if (ntiles > 0 && tile_in_band(w_beg)) {
    fetch_items(w_beg, 0, epre);
    curve_finish(w_beg, cbuf);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  uint16_t* vt = reinterpret_cast<uint16_t*>(smem) + wave * (VT_BYTES / 2);
  const float NEG_INF = -INFINITY;

  for (int t = 0; t < ntiles; ++t) {
    const int tk0 = w_beg + t * TK;
    // S^T = K Q^T from the registers of this tile
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    if constexpr (FP4) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        sacc = mfma32(as_bf16x8(fp4x8_to_bf16(kc[c / 4][c % 4], e8m0(ksb[c / 4]))), qf[c], sacc);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) sacc = mfma32(as_bf16x8(kreg[c]), qf[c], sacc);
    }
    // V of this tile -> LDS, transposed (the previous tile's reads of this buffer are done)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < NVI; ++it) {
      const int kg = lane & 7;
      const int dg = v_item_dg<FP4, NVI>(lane, it);
      const int pos = vt_pos(4 * kg);
      u32x4 rows[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        if constexpr (FP4) rows[s4] = fp4x8_to_bf16(vc[it][s4], e8m0(vsb[it][s4]));
        else rows[s4] = vreg[it][s4];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t p01 = __builtin_amdgcn_perm(rows[1][w], rows[0][w], sel);
        const uint32_t p23 = __builtin_amdgcn_perm(rows[3][w], rows[2][w], sel);
        st8(vt + (8 * dg + e) * VST + pos, u32x2{p01, p23});
      }
    }
    // registers are free: the next tile's loads are now in flight during this tile's work
    if (t + 1 < ntiles) load_tile(tk0 + TK);
    const bool next_band = t + 1 < ntiles && tile_in_band(tk0 + TK);
    if (next_band) fetch_items(tk0 + TK, 0, epre);

    // logits (log2 units), bias of in-band rows, mask beyond this wave's rows
    const bool in_band = tile_in_band(tk0);
    const float* cv = cbuf + (t & 1) * G * TK + (col_live ? ln : 0) * TK + 4 * lh;
    float mx = NEG_INF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = tk0 + 8 * (i >> 2) + 4 * lh + (i & 3);
      float sv = sacc[i] * c_qk;
      if (in_band) sv += cv[8 * (i >> 2) + (i & 3)];   // zero past the range and past the rows
      if (key >= w_end) sv = NEG_INF;
      sacc[i] = sv;
      mx = fmaxf(mx, sv);
    }
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = l_run * alpha;
    bf16x8 pf[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float p0 = fast_exp2(sacc[8 * kk + 2 * jj] - m_use);
        const float p1 = fast_exp2(sacc[8 * kk + 2 * jj + 1] - m_use);
        w[jj] = pack_bf16x2(p0, p1);
        psum = sum_bf16x2(w[jj], psum);
      }
      pf[kk] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
    }
    l_run = psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 vf = as_bf16x8(ld16(vt + (32 * db + ln) * VST + 16 * kk + 8 * lh));
        oacc[db] = mfma32(vf, pf[kk], oacc[db]);
      }
    // curve of the next tile into the other buffer (this tile's logits are done with theirs)
    if (next_band) curve_finish(tk0 + TK, cbuf + ((t + 1) & 1) * G * TK);
  }

  // ---- merge the 4 waves through LDS (reusing the V^T area) ---------------------------
  const float l_tot = pair_sum(l_run);
  __syncthreads();
  float* mb = reinterpret_cast<float*>(smem);           // [4][G][D] partial acc
  float* ml = mb + 4 * G * D;                           // [4][G][2] (m, l)
  if (col_live) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 32 * db + 8 * (i >> 2) + 4 * lh + (i & 3);
        mb[(wave * G + ln) * D + d] = oacc[db][i];
      }
    if (lh == 0) {
      ml[(wave * G + ln) * 2 + 0] = m_run;
      ml[(wave * G + ln) * 2 + 1] = l_tot;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int n = idx / D;
    const int d = idx % D;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[(w * G + n) * 2]);
    const float Mu = (M == NEG_INF) ? 0.f : M;
    float acc = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = fast_exp2(ml[(w * G + n) * 2] - Mu);
      acc += sc * mb[(w * G + n) * D + d];
      l += sc * ml[(w * G + n) * 2 + 1];
    }
    const int hh = hkv * G + n;
    if (a.n_split == 1) {
      a.o[(static_cast<size_t>(b) * a.Hq + hh) * D + d] = f32_to_bf16(acc / l);
      if (d == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.Hq + hh] = (M + fast_log2(l)) * kLn2;
    } else {
      float* wp = a.ws + ((static_cast<size_t>(b) * a.Hq + hh) * a.n_split + split) * (D + 2);
      wp[d] = acc;
      if (d == 0) {
        wp[D] = M;
        wp[D + 1] = l;
      }
    }
  }
}

// Decode for groups of at most 16 query heads on v_mfma_f32_16x16x32_bf16: the heads are the
// 16 MFMA columns, which halves the O accumulators and the query fragments against the 32x32
// form and leaves registers for two cache tiles in flight per wave (the step is bound by how
// many bytes each wave keeps in flight).  Same work split, bias, merge and partials as above.
//   * S^T (16 rows x 16 heads) per 16-row block: A = K rows straight from global memory,
//     B = q; a lane holds rows 16 kb + 4 (l / 16) + i of head l % 16.
//   * O^T += V^T P^T with the 32 rows of a tile as K: the rows are paired with the MFMA's K
//     elements in the order the scores already sit in (element j of lane group g is row
//     16 (j / 4) + 4 g + j % 4), so P is packed in place; V^T is stored in LDS with the rows
//     permuted to that order, one 16-byte read per lane.

// FP4: the caches hold MXFP4 codes (a.k / a.v: D / 2 bytes per row and kv head) and E8M0
// block scales (a.k_scale / a.v_scale: D / 32 bytes); the tiles in flight are the packed bytes
// (a quarter of the registers of bf16 rows) and are widened to bf16 where the MFMAs use them.
// A lane's K fragment then covers head dims (D / 4) g + 8 c .. + 7 (one 16-byte load per row at
// D = 128, 8 bytes at D = 64, and a single scale), so the query fragments use the same dims.
// PIPE: the pipelined tile loop, for contiguous caches or (PAGED) page pools, bf16 or MXFP4.
// Loads complete in issue order, so a wait for any load also waits for every tile requested
// before it; here the tile loop keeps the next tile in flight during each wait: every K / V
// load is issued unconditionally (contiguous: buffer resources that read zeros past the wave's
// last row; paged: rows clamped into the sequence, masked in the logits), so the compiler
// counts the loads in flight exactly; page entries are requested a tile ahead of the tile that
// uses them, before the tile two ahead; and the bias curves of the wave's first four tiles
// (every tile of a 512-row window) are formed up front from inputs requested ahead of the first
// tiles, so that no curve load follows a tile.
template <int D, int MODE, int RMAX, bool FP4, bool PIPE = false, bool PAGED = false>
__global__ __launch_bounds__(256, 2) void decode16_kernel(DecodeArgs a, int curve_off) {
  constexpr int VST = TK + 8;          // V^T row stride (bf16)
  constexpr int NC = D / 32;           // K = 32 chunks of the head dim
  constexpr int NDB = D / 16;          // 16-wide head-dim blocks of O^T
  constexpr int NVI = (TK / 4) * (D / 8) / 64;   // V items (4 rows x 8 dims) per lane
  constexpr int VT_BYTES = D * VST * 2;          // per wave
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: tile bases stay scalar
  const int n16 = lane & 15;           // head column
  const int g = lane >> 4;             // row group
  const int split = blockIdx.x;
  const int hkv = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.G;
  const bool col_live = n16 < G;

  const size_t kv_row = static_cast<size_t>(a.Hkv) * D;
  const bool paged = PIPE ? PAGED : a.block_table != nullptr;
  const int kv_len = paged ? min(max(a.kv_lens[b], 0), a.kv_len) : a.kv_len;
  const int key_begin = paged ? (a.window ? max(0, kv_len - a.window) : 0) : a.key_begin;
  // context-length temperature of this sequence's query, on q.k and bias alike
  const float tq = temp_factor(visible_keys(kv_len - 1, a.window), a.temp_len, a.temp_inv_log2);
  const float c_qk = a.c_qk * tq;
  const float c_bias = kLog2e * tq;
  const uint16_t* kbase = a.k + static_cast<size_t>(hkv) * D + (paged ? 0 : static_cast<size_t>(b) * a.L_max * kv_row);
  const uint16_t* vbase = a.v + static_cast<size_t>(hkv) * D + (paged ? 0 : static_cast<size_t>(b) * a.L_max * kv_row);
  const int* bt = paged ? a.block_table + static_cast<size_t>(b) * a.max_pages : nullptr;
  auto pool_row = [&](int key) -> int {
    const int pg = min(max(bt[key / a.page_size], 0), a.num_pages - 1);
    return pg * a.page_size + key % a.page_size;
  };
  const int qpos = kv_len - 1;

  const int w_beg = key_begin + (split * 4 + wave) * a.keys_per_wave;
  const int w_end = min(kv_len, w_beg + a.keys_per_wave);
  const int ntiles = w_end > w_beg ? (w_end - w_beg + TK - 1) / TK : 0;

  // ---- two register sets of tiles in flight: K as A-operand fragments, V as row pieces ----
  u32x4 kreg[2][2][FP4 ? 1 : NC], vreg[2][NVI][FP4 ? 1 : 4];
  // FP4: 16 code bytes and the scale byte per K row, 4 code bytes and a scale byte per V row
  u32x4 kc[2][2];
  uint32_t vc[2][NVI][4];
  uint8_t ksb[2][2], vsb[2][NVI][4];   // scale bytes, widened where they are used
  constexpr int CB = D / 2, SB = D / 32;
  constexpr int EPL = D / 4;   // FP4: head-dim elements of a lane's K fragment (D = 64 or 128)
  static_assert(!FP4 || EPL == 16 || EPL == 32, "MXFP4 caches: head_dim 64 or 128");
  const size_t crow = static_cast<size_t>(a.Hkv) * CB, srow = static_cast<size_t>(a.Hkv) * SB;
  const size_t cbatch = paged ? 0 : static_cast<size_t>(b) * a.L_max;
  const uint8_t* kcb = reinterpret_cast<const uint8_t*>(a.k) + (cbatch * a.Hkv + hkv) * CB;
  const uint8_t* vcb = reinterpret_cast<const uint8_t*>(a.v) + (cbatch * a.Hkv + hkv) * CB;
  const uint8_t* ksp = FP4 ? a.k_scale + (cbatch * a.Hkv + hkv) * SB : nullptr;
  const uint8_t* vsp = FP4 ? a.v_scale + (cbatch * a.Hkv + hkv) * SB : nullptr;
  // PIPE && PAGED: page entries of the K rows (rows 16 kb + l % 16) of the tile a register set
  // receives next, requested a tile ahead (keys clamped into the sequence: valid table entries)
  int pgv[2][2] = {{0, 0}, {0, 0}};
  auto key_clamp = [&](int key) { return max(0, min(key, w_end - 1)); };
  auto fetch_pages = [&](int set, int tk0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) pgv[set][kb] = bt[key_clamp(tk0 + 16 * kb + n16) / a.page_size];
  };
  auto load_tile = [&](int set, int tk0) {
    if constexpr (PIPE && PAGED) {
      // pool rows of this lane's K rows, and of its V rows from the lanes holding them (lane
      // l < 32 holds row tk0 + l); rows past the wave's end read its last row (masked later)
      int prow[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int pg = min(max(pgv[set][kb], 0), a.num_pages - 1);
        prow[kb] = pg * a.page_size + key_clamp(tk0 + 16 * kb + n16) % a.page_size;
      }
      const int prow32 = prow[g & 1];
      if constexpr (FP4) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint8_t* kp = kcb + static_cast<size_t>(prow[kb]) * crow + (EPL / 2) * g;
          if constexpr (EPL == 32) {
            kc[set][kb] = ld16(kp);
          } else {
            const u32x2 w2 = ld8(kp);
            kc[set][kb] = u32x4{w2[0], w2[1], 0u, 0u};
          }
          ksb[set][kb] = ksp[static_cast<size_t>(prow[kb]) * srow + (EPL * g) / 32];
        }
        const int kg = lane & 7;
        if constexpr (NVI == 2) {
          const int dg0 = v_item_dg<FP4, NVI>(lane, 0);
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const int vrow = __shfl(prow32, 4 * kg + s4, 64);
            const u32x2 w2 = ld8(vcb + static_cast<size_t>(vrow) * crow + 4 * dg0);
            vc[set][0][s4] = w2[0];
            vc[set][1][s4] = w2[1];
            vsb[set][0][s4] = vsb[set][1][s4] = vsp[static_cast<size_t>(vrow) * srow + (dg0 >> 2)];
          }
        } else {
#pragma unroll
          for (int it = 0; it < NVI; ++it) {
            const int dg = v_item_dg<FP4, NVI>(lane, it);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
              const int vrow = __shfl(prow32, 4 * kg + s4, 64);
              vc[set][it][s4] = *reinterpret_cast<const uint32_t*>(vcb + static_cast<size_t>(vrow) * crow + 4 * dg);
              vsb[set][it][s4] = vsp[static_cast<size_t>(vrow) * srow + (dg >> 2)];
            }
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint16_t* kp = kbase + static_cast<size_t>(prow[kb]) * kv_row + 8 * g;
#pragma unroll
          for (int c = 0; c < NC; ++c) kreg[set][kb][c] = ld16(kp + 32 * c);
        }
#pragma unroll
        for (int it = 0; it < NVI; ++it) {
          const int kg = lane & 7;
          const int dg = v_item_dg<FP4, NVI>(lane, it);
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const int vrow = __shfl(prow32, 4 * kg + s4, 64);
            vreg[set][it][s4] = ld16(vbase + static_cast<size_t>(vrow) * kv_row + 8 * dg);
          }
        }
      }
      return;
    }
    if constexpr (PIPE) {
      // rows tk0 .. tk0 + 31 through buffer resources over the tile's existing rows: the
      // resource ends at the last row's 2 D bytes, so every chunk of a row at or past w_end
      // reads as zeros (a row is row_b >= 2 D bytes from the next), and a tile wholly past
      // w_end has an empty resource (no memory access)
      const int left = w_end - tk0;
      const int nrows = left <= 0 ? 0 : (left < TK ? left : TK);
      if constexpr (FP4) {
        // codes (crow bytes per row, CB of this kv head) and scale bytes (srow, SB) likewise
        const int crow_i = static_cast<int>(crow), srow_i = static_cast<int>(srow);
        const int cbytes = nrows > 0 ? (nrows - 1) * crow_i + CB : 0;
        const int sbytes = nrows > 0 ? (nrows - 1) * srow_i + SB : 0;
        const __amdgpu_buffer_rsrc_t rkc = make_rsrc(kcb + static_cast<size_t>(tk0) * crow, cbytes);
        const __amdgpu_buffer_rsrc_t rks = make_rsrc(ksp + static_cast<size_t>(tk0) * srow, sbytes);
        const __amdgpu_buffer_rsrc_t rvc = make_rsrc(vcb + static_cast<size_t>(tk0) * crow, cbytes);
        const __amdgpu_buffer_rsrc_t rvs = make_rsrc(vsp + static_cast<size_t>(tk0) * srow, sbytes);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int r = 16 * kb + n16;
          if constexpr (EPL == 32) {
            kc[set][kb] = buf_ld16(rkc, r * crow_i + (EPL / 2) * g);
          } else {
            const u32x2 w2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rkc, r * crow_i + (EPL / 2) * g, 0, 0));
            kc[set][kb] = u32x4{w2[0], w2[1], 0u, 0u};
          }
          ksb[set][kb] = __builtin_amdgcn_raw_buffer_load_b8(rks, r * srow_i + (EPL * g) / 32, 0, 0);
        }
        const int kg = lane & 7;
        if constexpr (NVI == 2) {
          const int dg0 = v_item_dg<FP4, NVI>(lane, 0);
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const int r = 4 * kg + s4;
            const u32x2 w2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rvc, r * crow_i + 4 * dg0, 0, 0));
            vc[set][0][s4] = w2[0];
            vc[set][1][s4] = w2[1];
            vsb[set][0][s4] = vsb[set][1][s4] = __builtin_amdgcn_raw_buffer_load_b8(rvs, r * srow_i + (dg0 >> 2), 0, 0);
          }
        } else {
#pragma unroll
          for (int it = 0; it < NVI; ++it) {
            const int dg = v_item_dg<FP4, NVI>(lane, it);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
              const int r = 4 * kg + s4;
              vc[set][it][s4] = __builtin_amdgcn_raw_buffer_load_b32(rvc, r * crow_i + 4 * dg, 0, 0);
              vsb[set][it][s4] = __builtin_amdgcn_raw_buffer_load_b8(rvs, r * srow_i + (dg >> 2), 0, 0);
            }
          }
        }
        return;
      }
      const int row_b = a.Hkv * D * 2;
      const int nbytes = nrows > 0 ? (nrows - 1) * row_b + D * 2 : 0;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + static_cast<size_t>(tk0) * kv_row, nbytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + static_cast<size_t>(tk0) * kv_row, nbytes);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < NC; ++c) kreg[set][kb][c] = buf_ld16(rk, (16 * kb + n16) * row_b + 2 * (8 * g + 32 * c));
#pragma unroll
      for (int it = 0; it < NVI; ++it) {
        const int kg = lane & 7;
        const int dg = v_item_dg<FP4, NVI>(lane, it);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) vreg[set][it][s4] = buf_ld16(rv, (4 * kg + s4) * row_b + 16 * dg);
      }
      return;
    }
    // K rows tk0 + 16 kb + (l % 16); paged: one table read per lane and row block, and lane
    // l < 32 keeps the pool row of cache row tk0 + l for the V loads below
    int prow32 = 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = tk0 + 16 * kb + n16;
      const int prow = paged ? (key < w_end ? pool_row(key) : 0) : key;
      if (kb == (g & 1)) prow32 = prow;
      if constexpr (FP4) {
        kc[set][kb] = u32x4{0u, 0u, 0u, 0u};
        ksb[set][kb] = 0u;
        if (key < w_end) {
          const uint8_t* kp = kcb + static_cast<size_t>(prow) * crow + (EPL / 2) * g;
          if constexpr (EPL == 32) {
            kc[set][kb] = ld16(kp);
          } else {
            const u32x2 w2 = ld8(kp);
            kc[set][kb] = u32x4{w2[0], w2[1], 0u, 0u};
          }
          ksb[set][kb] = ksp[static_cast<size_t>(prow) * srow + (EPL * g) / 32];
        }
      } else {
        const uint16_t* kp = kbase + static_cast<size_t>(prow) * kv_row + 8 * g;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          kreg[set][kb][c] = u32x4{0u, 0u, 0u, 0u};
          if (key < w_end) kreg[set][kb][c] = ld16(kp + 32 * c);
        }
      }
    }
    if constexpr (FP4 && NVI == 2) {
      // the lane's two V items are dims 16 (l / 8) .. + 15 of the same 4 rows: one 8-byte code
      // load and one scale byte per row (both halves lie in one 32-dim scale block)
      const int kg = lane & 7;
      const int dg0 = v_item_dg<FP4, NVI>(lane, 0);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int kk = tk0 + 4 * kg + s4;
        int vrow = kk;
        if (paged) vrow = __shfl(prow32, 4 * kg + s4, 64);
        vc[set][0][s4] = vc[set][1][s4] = 0u;
        vsb[set][0][s4] = vsb[set][1][s4] = 0u;
        if (kk < w_end) {
          const u32x2 w2 = ld8(vcb + static_cast<size_t>(vrow) * crow + 4 * dg0);
          vc[set][0][s4] = w2[0];
          vc[set][1][s4] = w2[1];
          vsb[set][0][s4] = vsb[set][1][s4] = vsp[static_cast<size_t>(vrow) * srow + (dg0 >> 2)];
        }
      }
    } else {
#pragma unroll
    for (int it = 0; it < NVI; ++it) {
      const int item = lane + 64 * it;
      const int kg = item & 7;
      const int dg = item >> 3;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int kk = tk0 + 4 * kg + s4;
        int vrow = kk;
        if (paged) vrow = __shfl(prow32, 4 * kg + s4, 64);
        if constexpr (FP4) {
          vc[set][it][s4] = 0u;
          vsb[set][it][s4] = 0u;
          if (kk < w_end) {
            vc[set][it][s4] = *reinterpret_cast<const uint32_t*>(vcb + static_cast<size_t>(vrow) * crow + 4 * dg);
            vsb[set][it][s4] = vsp[static_cast<size_t>(vrow) * srow + (dg >> 2)];
          }
        } else {
          vreg[set][it][s4] = u32x4{0u, 0u, 0u, 0u};
          if (kk < w_end) vreg[set][it][s4] = ld16(vbase + static_cast<size_t>(vrow) * kv_row + 8 * dg);
        }
      }
    }
    }
  };

  // ---- bias curves per tile, as in the 32x32 kernel -----------------------------------------
  float* rs = reinterpret_cast<float*>(smem + curve_off);                  // [G][R] (r.E)
  // per wave a ring of tile curves [NSLOT][G][TK] (PIPE: the up-front curves of the first
  // NSLOT tiles, then the later in-band tiles in turn)
  constexpr int NSLOT = PIPE ? 4 : 2;
  float* cbuf = rs + (MODE == 2 ? G * a.R : 0) + wave * NSLOT * G * TK;
  auto stage_r = [&]() {
    for (int i = tid; i < G * a.R; i += 256)
      rs[i] = bf16_to_f32(a.r[(static_cast<size_t>(b) * a.Hq + hkv * G) * a.R + i]);
    __syncthreads();
  };
  const int n_items = G * TK;
  auto tile_in_band = [&](int tk0) { return MODE != 0 && qpos - (tk0 + TK - 1) < a.bias_range; };
  auto item_geo = [&](int tk0, int item, int& n, int& d, bool& live) {
    n = item / TK;
    const int j = item - n * TK;
    d = qpos - (tk0 + j);
    live = item < n_items && d >= 0 && d < a.bias_range && tk0 + j < w_end;
    if (item >= n_items) n = 0;
  };
  auto fetch_items = [&](int tk0, int base, float (&e)[2][RMAX]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int n, d;
      bool live;
      item_geo(tk0, base + lane + 64 * u, n, d, live);
      const int hh = hkv * G + n;
      if (MODE == 1) {
        e[u][0] = live ? a.table[static_cast<size_t>(hh) * a.bias_range + d] : 0.f;
      } else {
        const float* ep = a.E + static_cast<size_t>(hh) * a.e_hs + (live ? d : 0);
#pragma unroll
        for (int f = 0; f < RMAX; ++f) e[u][f] = (live && f < a.R) ? ep[static_cast<size_t>(f) * a.bias_range] : 0.f;
      }
    }
  };
  // PIPE: the same values through one buffer resource over the group's table rows or E
  // slabs (heads hkv G .. hkv G + G - 1): a lane's offset is its item's (head, distance), the
  // feature's offset is scalar (clamped to feature R - 1), and an item that is not live reads
  // zeros from an offset past the resource, so no load sits behind a per-lane branch.  The
  // launcher guarantees that the resource's extent fits 31 bits.
  const __amdgpu_buffer_rsrc_t e_rsrc = [&]() {
    if (MODE == 1)
      return make_rsrc(a.table + static_cast<size_t>(hkv) * G * a.bias_range, G * a.bias_range * 4);
    const long long hs = a.e_hs;
    return make_rsrc(a.E + static_cast<size_t>(hkv) * G * hs,
                     static_cast<int>(((G - 1) * hs + static_cast<long long>(a.R) * a.bias_range) * 4));
  }();
  auto fetch_items_buf = [&](int tk0, int base, float (&e)[2][RMAX]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int n, d;
      bool live;
      item_geo(tk0, base + lane + 64 * u, n, d, live);
      const int voff = live ? 4 * static_cast<int>((MODE == 1 ? static_cast<long long>(a.bias_range) : a.e_hs) * n + d)
                            : 0x7FFFFFF0;
      if (MODE == 1) {
        e[u][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(e_rsrc, voff, 0, 0));
      } else {
#pragma unroll
        for (int f = 0; f < RMAX; ++f) {
          const int soff = 4 * (f < a.R ? f : a.R - 1) * a.bias_range;
          e[u][f] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(e_rsrc, voff, soff, 0));
        }
      }
    }
  };
  auto finish_items = [&](int tk0, int base, const float (&e)[2][RMAX], float* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int item = base + lane + 64 * u;
      int n, d;
      bool live;
      item_geo(tk0, item, n, d, live);
      float acc = 0.f;
      if (MODE == 1) {
        acc = e[u][0];
      } else {
#pragma unroll
        for (int f = 0; f < RMAX; ++f)
          if (f < a.R) acc = fmaf(rs[n * a.R + f], e[u][f], acc);
      }
      if (item < n_items) dst[item] = acc * c_bias;
    }
  };
  // (the inputs are fetched where they are used: registers go to the tiles in flight)
  // PIPE: the same with a static trip count (n_items <= 256: G <= 8): a loop of unknown trip
  // count around loads makes the compiler's counts of loads in flight unknown after it, and
  // every later wait for a tile would then wait for all loads
  auto curve_tile_static = [&](int tk0, float* dst, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k >= k0 && 128 * k < n_items) {
        float e[2][RMAX];
        fetch_items_buf(tk0, 128 * k, e);
        finish_items(tk0, 128 * k, e, dst);
      }
    }
  };
  auto curve_tile = [&](int tk0, float* dst, int base0) {
    for (int base = base0; base < n_items; base += 128) {
      float e[2][RMAX];
      fetch_items(tk0, base, e);
      finish_items(tk0, base, e, dst);
    }
  };
  bf16x8 qf[NC];
  if constexpr (PIPE) {
    // r (one entry per thread, G R <= 128) and the curve inputs of the wave's first NPRE tiles
    // (their first 128 items each) are requested first, while no tile registers are live, then
    // the query rows and the first two tiles; the curves are formed while those are in flight,
    // and the tile loop then waits for no curve input of these tiles
    constexpr int NPRE = (MODE == 2 && RMAX > 8) ? 2 : NSLOT;
    // page pools: the page entries of the first two tiles first (their rows' addresses wait
    // for them)
    if constexpr (PAGED) {
      fetch_pages(0, w_beg);
      fetch_pages(1, w_beg + TK);
    }
    uint32_t r_raw = 0;
    if (MODE == 2) {
      const __amdgpu_buffer_rsrc_t r_rsrc =
          make_rsrc(a.r + (static_cast<size_t>(b) * a.Hq + hkv * G) * a.R, G * a.R * 2);
      r_raw = __builtin_amdgcn_raw_buffer_load_b16(r_rsrc, tid < G * a.R ? 2 * tid : 0x7FFFFFF0, 0, 0);
    }
    float ep[NPRE][2][RMAX];
#pragma unroll
    for (int i = 0; i < NPRE; ++i)
      if (i < ntiles && tile_in_band(w_beg + i * TK)) fetch_items_buf(w_beg + i * TK, 0, ep[i]);
    // keeps the compiler from moving those loads below the tile loads (loads may be reordered
    // freely, and it would sink them to their use)
    asm volatile("" ::: "memory");
  {
    const uint16_t* qp = a.q + (static_cast<size_t>(b) * a.Hq + hkv * G + (col_live ? n16 : 0)) * D + (FP4 ? EPL * g : 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (col_live) v = ld16(qp + (FP4 ? 8 * c : 32 * c));
      qf[c] = as_bf16x8(v);
    }
  }
    load_tile(0, w_beg);
    load_tile(1, w_beg + TK);
    if constexpr (PAGED) fetch_pages(0, w_beg + 2 * TK);   // for the first tile loop step
    if (MODE == 2) {
      if (tid < G * a.R) rs[tid] = bf16_to_f32(static_cast<uint16_t>(r_raw));
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < NSLOT; ++i) {
      if (i < ntiles && tile_in_band(w_beg + i * TK)) {
        float* dst = cbuf + i * G * TK;
        if (i < NPRE) {
          finish_items(w_beg + i * TK, 0, ep[i < NPRE ? i : 0], dst);
          curve_tile_static(w_beg + i * TK, dst, 1);
        } else {
          curve_tile_static(w_beg + i * TK, dst, 0);
        }
      }
    }
  } else {
  {
    const uint16_t* qp = a.q + (static_cast<size_t>(b) * a.Hq + hkv * G + (col_live ? n16 : 0)) * D + (FP4 ? EPL * g : 8 * g);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (col_live) v = ld16(qp + (FP4 ? 8 * c : 32 * c));
      qf[c] = as_bf16x8(v);
    }
  }
    if (ntiles > 0) load_tile(0, w_beg);
    if (ntiles > 1) load_tile(1, w_beg + TK);
    if (MODE == 2) stage_r();
    if (ntiles > 0 && tile_in_band(w_beg)) curve_tile(w_beg, cbuf, 0);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint16_t* vt = reinterpret_cast<uint16_t*>(smem) + wave * (VT_BYTES / 2);
  const float NEG_INF = -INFINITY;
  // V^T position of tile row k: 8 (k % 16 / 4) + 4 (k / 16) + k % 4
  auto vt_pos16 = [](int k) { return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3); };

  // LATE: this call may form the next tile's curve (always outside PIPE; in PIPE only in
  // the second phase of the tile loop below)
  auto process = [&](int t, int set, auto late_c) {
    constexpr bool LATE = decltype(late_c)::value;
    const int tk0 = w_beg + t * TK;
    // S^T of the two 16-row blocks
    f32x4 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (FP4) {
        const float ks = e8m0(ksb[set][kb]);
#pragma unroll
        for (int c = 0; c < NC; ++c)
          sacc[kb] = mfma16(as_bf16x8(fp4x8_to_bf16(kc[set][kb][c], ks)), qf[c], sacc[kb]);
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) sacc[kb] = mfma16(as_bf16x8(kreg[set][kb][c]), qf[c], sacc[kb]);
      }
    }
    // V of this tile -> LDS, transposed and row-permuted (the previous tile's reads are done)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < NVI; ++it) {
      const int kg = lane & 7;
      const int dg = v_item_dg<FP4, NVI>(lane, it);
      const int pos = vt_pos16(4 * kg);
      if constexpr (FP4) {
        u32x4 rows[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) rows[s4] = fp4x8_to_bf16(vc[set][it][s4], e8m0(vsb[set][it][s4]));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t p01 = __builtin_amdgcn_perm(rows[1][w], rows[0][w], sel);
          const uint32_t p23 = __builtin_amdgcn_perm(rows[3][w], rows[2][w], sel);
          st8(vt + (8 * dg + e) * VST + pos, u32x2{p01, p23});
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t p01 = __builtin_amdgcn_perm(vreg[set][it][1][w], vreg[set][it][0][w], sel);
          const uint32_t p23 = __builtin_amdgcn_perm(vreg[set][it][3][w], vreg[set][it][2][w], sel);
          st8(vt + (8 * dg + e) * VST + pos, u32x2{p01, p23});
        }
      }
    }
    // this set's registers are free: the tile two ahead goes in flight (PIPE: always issued,
    // empty past the wave's rows)
    if constexpr (PIPE) {
      // page pools: the next tile's page entries first, so that their wait (in the next call)
      // leaves this tile in flight
      if constexpr (PAGED) fetch_pages(1 - set, tk0 + 3 * TK);
      load_tile(set, tk0 + 2 * TK);
    } else if (t + 2 < ntiles) {
      load_tile(set, tk0 + 2 * TK);
    }

    // logits (log2 units), bias of in-band rows, mask beyond this wave's rows
    const bool in_band = tile_in_band(tk0);
    const float* cv = cbuf + (t & (NSLOT - 1)) * G * TK + (col_live ? n16 : 0) * TK + 4 * g;
    float mx = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = tk0 + 16 * kb + 4 * g + i;
        float sv = sacc[kb][i] * c_qk;
        if (in_band) sv += cv[16 * kb + i];
        if (key >= w_end) sv = NEG_INF;
        sacc[kb][i] = sv;
        mx = fmaxf(mx, sv);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = l_run * alpha;
    uint32_t w4[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float p0 = fast_exp2(sacc[kb][i] - m_use);
        const float p1 = fast_exp2(sacc[kb][i + 1] - m_use);
        w4[2 * kb + i / 2] = pack_bf16x2(p0, p1);
        psum = sum_bf16x2(w4[2 * kb + i / 2], psum);
      }
    const bf16x8 pf = as_bf16x8(u32x4{w4[0], w4[1], w4[2], w4[3]});
    l_run = psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16x8 vf = as_bf16x8(ld16(vt + (16 * db + n16) * VST + 8 * g));
      oacc[db] = mfma16(vf, pf, oacc[db]);
    }
    // the curve of the next tile (PIPE: only past the up-front ones; its inputs then wait
    // behind the tile just requested)
    if (LATE && (!PIPE || t + 1 >= NSLOT) && t + 1 < ntiles && tile_in_band(tk0 + TK)) {
      float* dst = cbuf + ((t + 1) & (NSLOT - 1)) * G * TK;
      if constexpr (PIPE)
        curve_tile_static(tk0 + TK, dst, 0);
      else
        curve_tile(tk0 + TK, dst, 0);
    }
  };
  // two register sets: the unroll keeps their indices static
  using late_t = std::integral_constant<bool, true>;
  using early_t = std::integral_constant<bool, false>;
  if constexpr (PIPE) {
    // Phase 1, tiles [0, t1): every curve they need was formed up front (tiles < NSLOT) or
    // none is (out of band), so its loop body has fixed load counts and no curve loads.  In-band
    // tiles are a suffix of the wave's tiles; t1 is the first in-band tile at or past NSLOT,
    // rounded down to even (tile t uses register set t % 2).  Phase 2, the in-band tiles past
    // the up-front ones (only where the bias range covers more than 4 of a wave's tiles), forms
    // each tile's curve during the tile before, as the general kernel does.
    int tb = ntiles;
    if (MODE != 0) {
      const int x = qpos - a.bias_range - w_beg - TK + 2;   // tile t in band iff t TK >= x
      tb = x <= 0 ? 0 : (x + TK - 1) / TK;
    }
    const int t1 = min(ntiles, max(NSLOT, tb)) & ~1;
    int t = 0;
    for (; t < t1; t += 2) {
      process(t, 0, early_t{});
      process(t + 1, 1, early_t{});
    }
    if (t < ntiles) {
      if (t >= NSLOT && tile_in_band(w_beg + t * TK))
        curve_tile_static(w_beg + t * TK, cbuf + (t & (NSLOT - 1)) * G * TK, 0);
      for (; t + 1 < ntiles; t += 2) {
        process(t, 0, late_t{});
        process(t + 1, 1, late_t{});
      }
      if (t < ntiles) process(t, 0, late_t{});
    }
  } else {
    for (int t = 0; t < ntiles; t += 2) {
      process(t, 0, late_t{});
      if (t + 1 < ntiles) process(t + 1, 1, late_t{});
    }
  }

  // ---- merge the 4 waves through LDS (reusing the V^T area) ---------------------------
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  __syncthreads();
  float* mb = reinterpret_cast<float*>(smem);           // [4][G][D] partial acc
  float* ml = mb + 4 * G * D;                           // [4][G][2] (m, l)
  if (col_live) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) mb[(wave * G + n16) * D + 16 * db + 4 * g + i] = oacc[db][i];
    if (g == 0) {
      ml[(wave * G + n16) * 2 + 0] = m_run;
      ml[(wave * G + n16) * 2 + 1] = l_tot;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int n = idx / D;
    const int d = idx % D;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[(w * G + n) * 2]);
    const float Mu = (M == NEG_INF) ? 0.f : M;
    float acc = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = fast_exp2(ml[(w * G + n) * 2] - Mu);
      acc += sc * mb[(w * G + n) * D + d];
      l += sc * ml[(w * G + n) * 2 + 1];
    }
    const int hh = hkv * G + n;
    if (a.n_split == 1) {
      a.o[(static_cast<size_t>(b) * a.Hq + hh) * D + d] = f32_to_bf16(acc / l);
      if (d == 0 && a.lse) a.lse[static_cast<size_t>(b) * a.Hq + hh] = (M + fast_log2(l)) * kLn2;
    } else {
      float* wp = a.ws + ((static_cast<size_t>(b) * a.Hq + hh) * a.n_split + split) * (D + 2);
      wp[d] = acc;
      if (d == 0) {
        wp[D] = M;
        wp[D + 1] = l;
      }
    }
  }
}

// Combine the split partials of one (batch, head): o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  const float* wp = a.ws + static_cast<size_t>(bh) * a.n_split * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, wp[s * (D + 2) + D]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float acc = 0.f, l = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const float sc = fast_exp2(wp[s * (D + 2) + D] - Mu);
    acc += sc * wp[s * (D + 2) + d];
    l += sc * wp[s * (D + 2) + D + 1];
  }
  a.o[static_cast<size_t>(bh) * D + d] = f32_to_bf16(acc / l);
  if (d == 0 && a.lse) a.lse[bh] = (M + fast_log2(l)) * kLn2;
}

template <int D, int MODE, int RMAX, bool FP4 = false>
hipError_t launch_d(DecodeArgs a, hipStream_t s) {
  const dim3 grid(a.n_split, a.Hkv, a.B);
  constexpr int VT_ALL = 4 * D * (TK + 8) * 2;
  const int merge = 4 * a.G * (D + 2) * 4;
  const int curve_off = ((VT_ALL > merge ? VT_ALL : merge) + 15) / 16 * 16;
  // after the V^T tiles / merge buffer: r [G][R] (r.E), then per wave two tile curves [G][TK]
  const bool narrow = a.G <= 16;
  // groups of up to 8 query heads: the 16x16 kernel with the pipelined tile loop (fixed load
  // counts per tile, up-front curves; contiguous caches or page pools), its curve inputs read
  // through one buffer resource, whose extent must fit 31 bits
  const long long e_extent = MODE == 1 ? 4LL * a.G * a.bias_range
                                       : 4LL * ((a.G - 1) * a.e_hs + static_cast<long long>(a.R) * a.bias_range);
  const bool pipe = a.G <= 8 && e_extent < (1LL << 31);
  const bool pool = a.block_table != nullptr;
  const int nslot = pipe ? 4 : 2;   // tile curves per wave
  const int total = curve_off + (MODE == 2 ? a.G * a.R * 4 : 0) + (MODE != 0 ? 4 * nslot * a.G * TK * 4 : 0);
  if (total > 160 * 1024) return hipErrorInvalidValue;
  // groups of up to 16 query heads: the 16x16 MFMA kernel (two tiles in flight per wave)
  const void* fn = pipe ? (pool ? reinterpret_cast<const void*>(&decode16_kernel<D, MODE, RMAX, FP4, true, true>)
                                : reinterpret_cast<const void*>(&decode16_kernel<D, MODE, RMAX, FP4, true, false>))
                   : narrow ? reinterpret_cast<const void*>(&decode16_kernel<D, MODE, RMAX, FP4>)
                            : reinterpret_cast<const void*>(&decode_bf16_kernel<D, MODE, RMAX, FP4>);
  {
    const hipError_t e = set_max_lds(fn, total, s);
    if (e != hipSuccess) return e;
  }
  if (pipe && pool)
    hipLaunchKernelGGL((decode16_kernel<D, MODE, RMAX, FP4, true, true>), grid, dim3(256), total, s, a, curve_off);
  else if (pipe)
    hipLaunchKernelGGL((decode16_kernel<D, MODE, RMAX, FP4, true, false>), grid, dim3(256), total, s, a, curve_off);
  else if (narrow)
    hipLaunchKernelGGL((decode16_kernel<D, MODE, RMAX, FP4>), grid, dim3(256), total, s, a, curve_off);
  else
    hipLaunchKernelGGL((decode_bf16_kernel<D, MODE, RMAX, FP4>), grid, dim3(256), total, s, a, curve_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.Hq), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// ---- fixed scratch of the allocation-free decode entry point ------------------------------------
// The split partials of relbias_attn_decode_noalloc live in this file-scope device array instead
// of a caller workspace: one copy per GPU the library runs on, held until the process ends.  Host
// code never uses the array's name as an address (in host code it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device with that device current, and
// is kept per device.
static __device__ __align__(256) unsigned char scratch[RBA_DECODE_NOALLOC_SCRATCH_BYTES];

hipError_t decode_noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

void decode_split(int B, int Hkv, int kv_len, int window, int* n_split, int* keys_per_wave) {
  // Enough workgroups to keep every CU streaming (2 resident per CU, 4 waves each); a wave
  // takes a contiguous run of cache rows, a multiple of the 32-row tile.
  const int key_begin = window ? (kv_len > window ? kv_len - window : 0) : 0;
  const long long n_vis = static_cast<long long>(kv_len) - key_begin;
  const long long pairs = static_cast<long long>(B) * Hkv;
  const long long target_wg = RBA_DECODE_TARGET_WG;
  long long ns = (target_wg + pairs - 1) / pairs;
  const long long max_ns = (n_vis + 4 * RBA_DECODE_MIN_ROWS - 1) / (4 * RBA_DECODE_MIN_ROWS);   // rows per wave
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  long long kpw = (n_vis + 4 * ns - 1) / (4 * ns);
  kpw = (kpw + TK - 1) / TK * TK;
  if (kpw < TK) kpw = TK;
  ns = (n_vis + 4 * kpw - 1) / (4 * kpw);
  if (ns < 1) ns = 1;
  *n_split = static_cast<int>(ns);
  *keys_per_wave = static_cast<int>(kpw);
}

hipError_t launch_decode_fp4(DecodeArgs a, int D, int mode, hipStream_t s) {
  if (D == 128) {
    switch (mode) {
      case 0: return launch_d<128, 0, 1, true>(a, s);
      case 1: return launch_d<128, 1, 1, true>(a, s);
      default: return a.R > 8 ? launch_d<128, 2, 16, true>(a, s) : launch_d<128, 2, 8, true>(a, s);
    }
  }
  switch (mode) {
    case 0: return launch_d<64, 0, 1, true>(a, s);
    case 1: return launch_d<64, 1, 1, true>(a, s);
    default: return a.R > 8 ? launch_d<64, 2, 16, true>(a, s) : launch_d<64, 2, 8, true>(a, s);
  }
}

hipError_t launch_decode_bf16(DecodeArgs a, int D, int mode, hipStream_t s) {
  if (D == 128) {
    switch (mode) {
      case 0: return launch_d<128, 0, 1>(a, s);
      case 1: return launch_d<128, 1, 1>(a, s);
      default: return a.R > 8 ? launch_d<128, 2, 16>(a, s) : launch_d<128, 2, 8>(a, s);
    }
  }
  switch (mode) {
    case 0: return launch_d<64, 0, 1>(a, s);
    case 1: return launch_d<64, 1, 1>(a, s);
    default: return a.R > 8 ? launch_d<64, 2, 16>(a, s) : launch_d<64, 2, 8>(a, s);
  }
}

}  // namespace rba
