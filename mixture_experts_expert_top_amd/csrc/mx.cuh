// MXFP8 element and scale codecs shared by the quantize kernels and the
// GEMM epilogues ("Efficient MoE Training for Biological Foundation
// Models", Challenge 2: 8-bit values with one scaling factor per block of
// 32 consecutive values; the element format is OCP E4M3 "FN", the scale an
// E8M0 power of two).
#pragma once

#include "common.cuh"

namespace moe {

constexpr int kMxBlock = 32;

// Scale exponent of a block from its largest magnitude (a finite float):
// e = clamp(floor(log2 amax) - 8, -127, 127), 8 being the exponent of
// E4M3's largest normal (448 = 1.75 * 2^8); zero and subnormal maxima give
// -127.  Read from the exponent field, so it is exact.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const int ef = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
  if (ef == 0) return -127;
  const int e = ef - 127 - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as a float, for the e that finite bf16 or fp32 block maxima give
// (-127 .. 119): always a normal float.
__device__ __forceinline__ float mx_inv_scale(int e) {
  return __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
}

// E4M3 codes of four values (already divided by the block scale), packed
// little-endian: round to nearest, ties to even mantissa, saturate at
// +-448, keep the sign (also of zero).  gfx950's v_cvt_pk_fp8_f32 converts
// two floats to OCP E4M3 with round-to-nearest-even; it returns NaN past
// the largest finite value, so the inputs are clamped to +-448 first.
// Checked against a software encoder of this rule on every float of
// magnitude below 512, both signs (no difference), and against the
// float64 codec on every finite bf16 value in the tests.
__device__ __forceinline__ float e4m3_clamp(float x) {
  return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f);
}

__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c,
                                               float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0,
                                          false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
  return static_cast<uint32_t>(w);
}

}  // namespace moe
