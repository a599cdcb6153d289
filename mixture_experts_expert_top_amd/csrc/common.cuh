// Device-side helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

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

// Two floats -> packed pair of bfloat16 (lo in bits 0..15), round to
// nearest even: one two-input hardware convert.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// Workgroup id -> logical id so that the workgroups one XCD receives (the
// hardware hands out ids round-robin over the 8 XCDs) form a contiguous
// range of logical ids, which share data in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int q = nb >> 3, r = nb & 7;
  const int x = bid & 7, i = bid >> 3;
  return x * q + min(x, r) + i;
}

// ---------------------------------------------------------------- buffers
// Raw buffer resource over [base, base + bytes), bytes <= kOob (internal.h).
// Loads whose offset falls outside the range return zero, which implements
// tile masking.
constexpr uint32_t kBufferWord3 = 0x00020000u;

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

// The same with a wave-uniform part of the offset in soffset (a scalar
// register, added without a vector instruction).  Callers keep every term
// that can reach past the resource in voff, so the range check holds
// whether or not the hardware counts soffset in it, and keep voff + soff
// below 2^32.
__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r,
                                            uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r,
                                              uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
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


// ---------------------------------------------------------------- [k][mn] tiles
// An LDS tile of 64 k-rows x 256 bf16 columns kept as it lies in memory
// (512-byte rows), the 16-byte chunk c of k-row r at chunk c ^ ((r & 3) << 2)
// of its row: 64 lanes storing two rows' 32 chunks, and 64 lanes of a
// transposed fragment read touching 8 rows x 4 chunks, both spread evenly
// over the LDS banks.  kmn_off is the byte offset of chunk c of row r.
__device__ __forceinline__ int kmn_off(int r, int c) {
  return r * 512 + ((c ^ ((r & 3) << 2)) << 4);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// MFMA 32x32x16 fragment (lane l: column l % 32, k = 8 (l / 32) + 0..7 of
// k-slice kk) of a [k][mn] LDS tile laid out by kmn_off, for the 32
// columns starting at 32 * blk.  ds_read_b64_tr_b16 works on groups of 16
// lanes: lane 4R + m of a group gives the address of 4 consecutive
// elements, which become columns 4m..4m+3 of row R of a 4 x 16 block, and
// lane j receives column j (rows 0..3).  Group g = l / 16 of the fragment
// covers k-rows 8 (g / 2) + 0..3 (first read) and + 4..7 (second read,
// 2048 bytes on) and columns 16 (g % 2) + 0..15.  lane_base and R come
// from KmnLane.
// frag_tr_at takes the lane's whole block offset, lane_base + ((blk ^ R)
// << 6), so a caller can compute it once for every k-slice and stage.
__device__ __forceinline__ bf16x8_v frag_tr_at(const uint8_t* tile,
                                               int lane_off, int kk) {
  const uint8_t* p = tile + lane_off + kk * 8192;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(p + 2048));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_v, v);
}

__device__ __forceinline__ bf16x8_v frag_tr(const bf16_t* tile, int lane_base,
                                            int R, int blk, int kk) {
  return frag_tr_at(reinterpret_cast<const uint8_t*>(tile),
                    lane_base + ((blk ^ R) << 6), kk);
}

// The lane's fixed part of a frag_tr address (its row R and chunk inside a
// 4 x 16 block, from its 16-lane group and position).
struct KmnLane {
  int base, R;
  __device__ __forceinline__ explicit KmnLane(int lane) {
    const int g = lane >> 4, j = lane & 15;
    R = j >> 2;
    const int m = j & 3;
    base = ((g >> 1) * 8 + R) * 512 + (2 * (g & 1) + (m >> 1)) * 16 +
           (m & 1) * 8;
  }
};

}  // namespace moe
