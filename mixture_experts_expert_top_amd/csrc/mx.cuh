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

// E4M3 code of x (already divided by the block scale): round to nearest,
// ties to even mantissa, saturate at +-448, keep the sign (also of zero).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7fffffffu);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7eu;                              // saturate (448 itself too)
  } else if (a < 0.015625f) {                  // below 2^-6: subnormal step
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));   // 0..8
  } else {
    const uint32_t b = u & 0x7fffffffu;
    uint32_t exp = (b >> 23) - 127 + 7;        // biased E4M3 exponent 1..15
    uint32_t man = (b >> 20) & 7u;
    const uint32_t rem = b & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (man & 1u))) {
      if (++man == 8u) { man = 0; ++exp; }
    }
    code = (exp << 3) | man;
    if (code > 0x7eu) code = 0x7eu;
  }
  return code | sign;
}

}  // namespace moe
