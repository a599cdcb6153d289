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

// base and bytes must be the same on every lane of the wave: they are read
// from the first active lane, which keeps the resource in scalar registers
// (a resource the compiler cannot prove uniform costs a readfirstlane loop
// around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(p & 0xffffffffu)));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(p >> 32)));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(
      ub, static_cast<short>(0),
      __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)),
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
// 1 / (1 + e^-a) with the hardware reciprocal (about 1 ulp) in place of an
// IEEE division: the result feeds bf16 or E4M3 values, and the division's
// scale/fixup sequence cost ten VALU instructions an element in the SwiGLU
// epilogues.  a -> -inf gives rcp(inf) = 0, a -> +inf gives 1.
__device__ __forceinline__ float sigmoidf_(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
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

// ---------------------------------------------------------------- DPP
// Lane exchanges inside a row of 16 lanes as DPP operand modifiers of a
// VALU move (no LDS round trip, unlike ds_bpermute).  Controls:
// quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane i of each 8 reads lane 7 - i) and row_mirror
// (lane i of each 16 reads lane 15 - i).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

// Sum over aligned groups of W lanes (W = 2, 4, 8 or 16), the sum in every
// lane of the group: pairs, then quads, then halves of a row (the mirror
// pairs lane i with the other quad), then the row.
template <int W>
__device__ __forceinline__ float dpp_group_sum(float v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group of 2..16");
  v += dpp_move<kDppXor1>(v);
  if constexpr (W >= 4) v += dpp_move<kDppXor2>(v);
  if constexpr (W >= 8) v += dpp_move<kDppHalfMirror>(v);
  if constexpr (W >= 16) v += dpp_move<kDppMirror>(v);
  return v;
}

// Maximum over aligned groups of W lanes, in every lane of the group.
template <int W>
__device__ __forceinline__ float dpp_group_max(float v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group of 2..16");
  v = fmaxf(v, dpp_move<kDppXor1>(v));
  if constexpr (W >= 4) v = fmaxf(v, dpp_move<kDppXor2>(v));
  if constexpr (W >= 8) v = fmaxf(v, dpp_move<kDppHalfMirror>(v));
  if constexpr (W >= 16) v = fmaxf(v, dpp_move<kDppMirror>(v));
  return v;
}

}  // namespace moe
