// MXFP8 element and scale codecs shared by the quantize kernels and the
// GEMM epilogues ("Efficient MoE Training for Biological Foundation
// Models", Challenge 2: 8-bit values with one scaling factor per block of
// 32 consecutive values; the element format is OCP E4M3 "FN", the scale an
// E8M0 power of two).
#pragma once

#include "common.cuh"
#include "internal.h"

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

// Exclusive prefix of the 128-padded segment lengths into s_pad[0..nseg]
// (one wave), from device offsets seg[0..nseg] (or one segment of `rows`).
__device__ inline void padded_prefix(const int32_t* seg, int nseg, int64_t rows,
                              int* s_pad) {
  const int lane = threadIdx.x;
  if (lane < 64) {
    constexpr int kPer = (kMaxExperts + 1 + 63) / 64;
    int loc[kPer];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = lane * kPer + q;
      int len = 0;
      if (i < nseg)
        len = seg ? seg[i + 1] - seg[i] : static_cast<int>(rows);
      loc[q] = (len + kMxPad - 1) / kMxPad * kMxPad;
      sum += loc[q];
    }
    int incl = sum;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(incl, m, 64);
      if (lane >= m) incl += o;
    }
    int run = incl - sum;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = lane * kPer + q;
      if (i <= nseg) s_pad[i] = run;
      run += loc[q];
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------- MXFP4
// The hgpu.org abstract of the MXFP4 MoE training recipe keeps activations
// and payloads as MXFP4: E2M1 elements (0, 0.5, 1, 1.5, 2, 3, 4, 6 and
// their negatives) with one E8M0 scale per 32 values, stored two codes a
// byte (the lower index in the low nibble).

// Block scale exponent: clamp(floor(log2 amax) - 2, -127, 127), 2 being
// the exponent of E2M1's largest value (6 = 1.5 * 2^2); zero and subnormal
// maxima give -127.
__device__ __forceinline__ int mx4_scale_exp(float amax) {
  const int ef = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
  if (ef == 0) return -127;
  const int e = ef - 127 - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// E2M1 codes of v[0..7] (already divided by the block scale): round to
// nearest, ties to the even code, saturate at +-6, keep the sign.  gfx950's
// v_cvt_scalef32_pk_fp4_f32 (scale 1) rounds this way; it was checked
// against a software encoder of the rule on every float of magnitude
// below 16, both signs, and the inputs are clamped to +-6 first.
__device__ __forceinline__ float e2m1_clamp(float x) {
  return __builtin_amdgcn_fmed3f(x, -6.0f, 6.0f);
}

__device__ __forceinline__ uint32_t e2m1_pack8(const float* v) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e2m1_clamp(v[0]),
                                               e2m1_clamp(v[1]), 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e2m1_clamp(v[2]),
                                               e2m1_clamp(v[3]), 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e2m1_clamp(v[4]),
                                               e2m1_clamp(v[5]), 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e2m1_clamp(v[6]),
                                               e2m1_clamp(v[7]), 1.0f, 3);
  return w;
}

// Value of an E2M1 code (bits 0-3).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  // m < 2: 0 or 0.5; else (1 + (m & 1) / 2) * 2^((m >> 1) - 1)
  const float v = (m < 2u) ? 0.5f * static_cast<float>(m)
                           : __uint_as_float(((126u + (m >> 1)) << 23) |
                                             ((m & 1u) << 22));
  return (c & 8u) ? -v : v;
}

// 2^(byte - 127) for a scale byte (2^-127 is a subnormal float).
__device__ __forceinline__ float e8m0_value(uint32_t byte) {
  return byte ? __uint_as_float(byte << 23) : __uint_as_float(0x00400000u);
}

}  // namespace moe
