// MXFP4 block quantization for activations and dispatch payloads (the
// hgpu.org abstract of the MXFP4 MoE training recipe: GEMMs stay FP8,
// activations and expert-parallel payloads are MXFP4, and row-blocked FP4
// is turned into column blocks with new scales).
//
// Layouts (two E2M1 codes a byte, the lower index in the low nibble; one
// E8M0 scale byte per 32 values):
//   rows:   blocks of 32 consecutive columns of [rows][cols]: codes
//           [rows][cols/2], scales [rows][cols/32].
//   tokens: blocks of 32 consecutive rows restarting at every segment
//           start, transposed: codes [cols][rows_pad/2], scales
//           [cols][rows_pad/32]; segment s starts at padded row
//           sum over s' < s of round_up(len_s', 128); padding holds zero
//           codes with scale byte 0.
// The token-axis kernel reads either bf16 rows or MXFP4 rows; from MXFP4
// it is the row-to-column conversion: every value is decoded exactly and
// re-blocked along the rows with new scales.

#include "common.cuh"
#include "internal.h"
#include "mx.cuh"

namespace moe {
namespace {

// One thread per 32-block of a bf16 row: 64 bytes in, 16 code bytes and a
// scale byte out.
__global__ __launch_bounds__(256) void quant_rows4_kernel(
    const bf16_t* __restrict__ src, int64_t rows, int64_t cols,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t nb = cols / kMxBlock;
  const int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x +
                      threadIdx.x;
  if (blk >= rows * nb) return;
  const i32x4* p = reinterpret_cast<const i32x4*>(src + blk * kMxBlock);
  float v[kMxBlock];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const i32x4 w = p[q];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[q * 8 + 2 * c] = bf_lo(static_cast<uint32_t>(w[c]));
      v[q * 8 + 2 * c + 1] = bf_hi(static_cast<uint32_t>(w[c]));
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx4_scale_exp(amax);
  const float inv = mx_inv_scale(e);
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) v[i] *= inv;
  i32x4 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) out[q] = static_cast<int>(e2m1_pack8(v + 8 * q));
  *reinterpret_cast<i32x4*>(codes + blk * (kMxBlock / 2)) = out;
  scales[blk] = static_cast<uint8_t>(e + 127);
}

// Workgroup = one 128-row tile of the padded layout x kTok4Runs runs of 64
// columns (a tile never straddles a segment: segments start on multiples
// of 128), each run in three steps:
//   1. the tile's source rows go to LDS as fp32 (rows past the segment
//      read as zero): from bf16, thread t converts 8 columns of rows
//      t/8 + 32 i; from MXFP4, thread t decodes 32 columns (16 code bytes
//      and their scale) of row t/2;
//   2. thread (block b = t/64, column c = t%64) quantizes its 32-row block
//      of one column into 16 code bytes of an LDS staging line;
//   3. every column's 128 codes leave as one 64-byte line (4 lanes, 16
//      bytes each) and its 4 scale bytes as one word.
constexpr int kTok4Rows = 128;
constexpr int kTok4Cols = 64;
constexpr int kTok4Ld = kTok4Cols + 4;      // fp32 row stride of the tile
constexpr int kTok4Runs = 4;                // column runs per workgroup

template <bool kSrcFp4>
__global__ __launch_bounds__(256) void quant_tokens4_kernel(
    const void* __restrict__ src, const uint8_t* __restrict__ src_scales,
    int64_t rows, int64_t cols, const int32_t* __restrict__ seg, int nseg,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    int64_t rows_pad) {
  __shared__ int s_pad[kMaxExperts + 1];
  __shared__ float tile[kTok4Rows * kTok4Ld];
  __shared__ __attribute__((aligned(16))) uint8_t out[kTok4Cols]
                                                     [kTok4Rows / 2];
  __shared__ uint32_t sc_out[kTok4Cols];
  padded_prefix(seg, nseg, rows, s_pad);
  const int t = threadIdx.x;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kTok4Rows;
  int lo = 0, hi = nseg - 1;               // segment holding this tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pad[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  int64_t r0 = 0, r_end = 0;               // source rows [r0, r_end)
  if (p0 < s_pad[nseg]) {
    const int64_t sbeg = seg ? seg[lo] : 0;
    const int64_t send = seg ? seg[lo + 1] : rows;
    r0 = sbeg + (p0 - s_pad[lo]);
    r_end = r0 + kTok4Rows < send ? r0 + kTok4Rows : send;
  }
  for (int ct = 0; ct < kTok4Runs; ++ct) {
    const int64_t c0 =
        (static_cast<int64_t>(blockIdx.y) * kTok4Runs + ct) * kTok4Cols;
    if (c0 >= cols) break;
    if (ct > 0) __syncthreads();           // LDS of the previous run
    // 1. load
    if constexpr (!kSrcFp4) {
      const bf16_t* s16 = static_cast<const bf16_t*>(src);
      const int cc = (t & 7) * 8;
      const bool col_ok = c0 + cc < cols;  // cols % 32 == 0
#pragma unroll
      for (int i = 0; i < kTok4Rows / 32; ++i) {
        const int rr = (t >> 3) + 32 * i;
        i32x4 w = {0, 0, 0, 0};
        if (col_ok && r0 + rr < r_end)
          w = *reinterpret_cast<const i32x4*>(s16 + (r0 + rr) * cols + c0 +
                                              cc);
        float* d = tile + rr * kTok4Ld + cc;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          d[2 * c] = bf_lo(static_cast<uint32_t>(w[c]));
          d[2 * c + 1] = bf_hi(static_cast<uint32_t>(w[c]));
        }
      }
    } else {
      const uint8_t* s4 = static_cast<const uint8_t*>(src);
      const int rr = t >> 1, half = t & 1;
      const int64_t cbase = c0 + 32 * half;
      i32x4 w = {0, 0, 0, 0};
      float sc = 0.0f;
      if (cbase < cols && r0 + rr < r_end) {
        const int64_t r = r0 + rr;
        w = *reinterpret_cast<const i32x4*>(s4 + r * (cols / 2) + cbase / 2);
        sc = e8m0_value(src_scales[r * (cols / kMxBlock) + cbase / kMxBlock]);
      }
      float* d = tile + rr * kTok4Ld + 32 * half;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t word = static_cast<uint32_t>(w[q]);
#pragma unroll
        for (int n = 0; n < 8; ++n)
          d[8 * q + n] = e2m1_value(word >> (4 * n)) * sc;
      }
    }
    __syncthreads();
    // 2. quantize one 32-row block of one column
    {
      const int c = t & (kTok4Cols - 1);
      const int b = t / kTok4Cols;
      float v[kMxBlock];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < kMxBlock; ++i) {
        v[i] = tile[(b * kMxBlock + i) * kTok4Ld + c];
        amax = fmaxf(amax, fabsf(v[i]));
      }
      const int e = mx4_scale_exp(amax);   // all-zero block: byte 0
      const float inv = mx_inv_scale(e);
#pragma unroll
      for (int i = 0; i < kMxBlock; ++i) v[i] *= inv;
      i32x4 q;
#pragma unroll
      for (int k = 0; k < 4; ++k) q[k] = static_cast<int>(e2m1_pack8(v + 8 * k));
      *reinterpret_cast<i32x4*>(&out[c][b * (kMxBlock / 2)]) = q;
      reinterpret_cast<uint8_t*>(sc_out)[c * 4 + b] =
          static_cast<uint8_t>(e + 127);
    }
    __syncthreads();
    // 3. write: 64 columns x 64 code bytes, 4 lanes a line
    {
      const int col = t >> 2, chunk = t & 3;
      if (c0 + col < cols)
        *reinterpret_cast<i32x4*>(codes + (c0 + col) * (rows_pad / 2) +
                                  p0 / 2 + chunk * 16) =
            *reinterpret_cast<const i32x4*>(&out[col][chunk * 16]);
    }
    if (t < kTok4Cols && c0 + t < cols)
      *reinterpret_cast<uint32_t*>(scales + (c0 + t) * (rows_pad / kMxBlock) +
                                   p0 / kMxBlock) = sc_out[t];
  }
}

}  // namespace

hipError_t launch_mx4_quant_rows(const bf16_t* src, int64_t rows,
                                 int64_t cols, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s) {
  const int64_t blocks = rows * (cols / kMxBlock);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows4_kernel,
                     dim3(static_cast<unsigned>((blocks + 255) / 256)),
                     dim3(256), 0, s, src, rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx4_quant_tokens(const void* src,
                                   const uint8_t* src_scales, int64_t rows,
                                   int64_t cols, const int32_t* seg, int nseg,
                                   uint8_t* codes, uint8_t* scales,
                                   int64_t rows_pad, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(rows_pad / kTok4Rows),
            static_cast<unsigned>((cols + kTok4Cols * kTok4Runs - 1) /
                                  (kTok4Cols * kTok4Runs)));
  if (src_scales)
    hipLaunchKernelGGL(quant_tokens4_kernel<true>, grid, dim3(256), 0, s, src,
                       src_scales, rows, cols, seg, nseg, codes, scales,
                       rows_pad);
  else
    hipLaunchKernelGGL(quant_tokens4_kernel<false>, grid, dim3(256), 0, s,
                       src, src_scales, rows, cols, seg, nseg, codes, scales,
                       rows_pad);
  return hipGetLastError();
}

}  // namespace moe
