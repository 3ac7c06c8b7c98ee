// Device helpers for the gfx950 kernels: vector types, bf16 packing, MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rba {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> one packed pair of bf16 (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// acc + lo(x) + hi(x) for a packed bf16 pair x (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// Buffer resource over `bytes` bytes from `base` (raw, unswizzled): loads whose 16 bytes
// lie past the end return zeros, so row guards need no branches.  The base must be uniform
// across the wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// D = A * B + C on a 32x32 output tile, K = 16 bf16 (fp32 accumulate).
// Lane l holds A row (l % 32) and B column (l % 32), 8 K-elements each; the
// K-elements of the two operands are paired by (l / 32, element index), so any
// fixed assignment of logical k to (l / 32, element) used on both sides gives
// the same sum.  Output: lane l holds column l % 32, rows
// 8 * (i / 4) + 4 * (l / 32) + (i % 4) for i = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A * B + C on a 16x16 output tile, K = 32 bf16 (fp32 accumulate).  Lane l holds A row
// (l % 16) and B column (l % 16), 8 K-elements each, paired by (l / 16, element index) as in
// the 32x32 form; output: lane l holds column l % 16, rows 4 * (l / 16) + i for i = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of the lane 32 apart (the two halves of a 32x32 MFMA column).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max / sum over the lane pair (l, l ^ 32) with v_permlane32_swap: both results of the
// swap hold {x[l % 32], x[l % 32 + 32]} in every lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Fills entries [0, n) of a staging buffer, thread t taking t, t + nt, t + 2 nt, ...: in
// batches of 8, all of a batch's loads are issued before any is used (a loop of one load and its
// store per entry waits out one memory round trip per entry).  Indices past n are clamped to
// n - 1 (that entry is loaded and stored again with the same value), so that neither the loads
// nor the stores sit behind a branch the compiler could sink a load into.  load(x) returns the
// raw 32-bit word of entry x from an address valid for any x in [0, n); store(x, w) writes
// entry x from that word (masks as integer operations, for the same reason).
template <typename LoadF, typename StoreF>
__device__ __forceinline__ void stage_batched(int tid, int nt, int n, LoadF load, StoreF store) {
  for (int x0 = tid; x0 < n; x0 += 8 * nt) {
    uint32_t w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = load(min(x0 + u * nt, n - 1));
#pragma unroll
    for (int u = 0; u < 8; ++u) store(min(x0 + u * nt, n - 1), w[u]);
  }
}

}  // namespace rba
