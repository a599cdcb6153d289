// Device-side helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // IEEE bfloat16 bit pattern

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16, round to nearest even (hardware convert on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, b);
}

// Two floats -> packed pair of bfloat16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f2bf(lo)) |
         (static_cast<uint32_t>(f2bf(hi)) << 16);
}

__device__ __forceinline__ float bf_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// ---------------------------------------------------------------- buffers
// Raw buffer resource over [base, base + bytes).  Loads whose offset falls
// outside the range return zero, which implements tile masking.
constexpr uint32_t kBufferWord3 = 0x00020000u;
constexpr uint32_t kOob = 0x80000000u;  // an offset beyond every range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base),
                                           static_cast<short>(0),
                                           static_cast<int>(bytes),
                                           static_cast<int>(kBufferWord3));
}

__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r,
                                            uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r,
                                              uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// ---------------------------------------------------------------- math
__device__ __forceinline__ float sigmoidf_(float a) {
  return 1.0f / (1.0f + __expf(-a));
}

// ---------------------------------------------------------------- waves
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, kWave);
}

// Sum over groups of `width` consecutive lanes (power of two), fixed
// butterfly order, result in every lane of the group.
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

}  // namespace moe
