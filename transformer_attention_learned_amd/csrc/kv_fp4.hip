// MXFP4 quantisation of bf16 rows (a KV cache) for gfx950.
//
// The FP4 KV cache of the pages ("models/inkling" (archdiff), the component diagram: KV-cache
// compression with FP4 KV; MXFP4 among the FP4 formats of training) in the OCP Microscaling
// form: blocks of 32 elements along a row share one E8M0 scale byte (2^(byte - 127)), each
// element an E2M1 code (sign in bit 3; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  The block
// exponent is floor(log2(max |x|)) - 2, clamped to [-126, 127]; x / 2^exponent is rounded to
// the nearest magnitude, ties to the even code, saturating at 6; an all-zero block gets byte 0.
// Element 2j of a row sits in the low nibble of byte j, element 2j + 1 in the high nibble.
//
// One thread per block: four 16-byte loads, the block maximum, the codes as a count of the
// rounding thresholds passed, one 16-byte store of codes and one scale byte.

#include "rba_device.h"
#include "rba_internal.h"

namespace rba {

namespace {

// Nearest E2M1 magnitude code of a >= 0: one step per threshold passed.  The thresholds are
// the midpoints of consecutive values; at a midpoint the even code wins, hence > for the
// midpoints whose upper neighbour is odd and >= where it is even.
__device__ __forceinline__ uint32_t e2m1_code(float a) {
  return static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
         static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
         static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
         static_cast<uint32_t>(a > 5.0f);
}

__global__ __launch_bounds__(256) void quantize_fp4_kernel(const uint16_t* x, uint8_t* codes, uint8_t* scales,
                                                          long long nblk) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long blk = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; blk < nblk; blk += stride) {
    const uint16_t* src = x + blk * 32;
    u32x4 raw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = ld16(src + 8 * c);
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[8 * c + 2 * w] = __uint_as_float(raw[c][w] << 16);
        v[8 * c + 2 * w + 1] = __uint_as_float(raw[c][w] & 0xffff0000u);
      }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // floor(log2(amax)) from the exponent field (subnormals give -127 and clamp below)
    const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff) - 127;
    const int s = min(max(e - 2, -126), 127);
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - s) << 23);   // 2^-s, exact
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float xv = v[8 * q + j];
        const uint32_t code = e2m1_code(fabsf(xv * inv)) | (xv < 0.f ? 8u : 0u);
        word |= code << (4 * j);
      }
      w[q] = word;
    }
    const bool zero = !(amax > 0.f);
    if (zero) w[0] = w[1] = w[2] = w[3] = 0u;
    st16(codes + blk * 16, u32x4{w[0], w[1], w[2], w[3]});
    scales[blk] = zero ? static_cast<uint8_t>(0) : static_cast<uint8_t>(s + 127);
  }
}

}  // namespace

hipError_t launch_quantize_fp4(const uint16_t* x, uint8_t* codes, uint8_t* scales, long long nblk, hipStream_t s) {
  if (nblk <= 0) return hipSuccess;
  const long long want = (nblk + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 16384 ? want : 16384);
  hipLaunchKernelGGL(quantize_fp4_kernel, dim3(grid), dim3(256), 0, s, x, codes, scales, nblk);
  return hipGetLastError();
}

}  // namespace rba
