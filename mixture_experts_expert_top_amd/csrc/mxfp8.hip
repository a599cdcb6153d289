// MXFP8 block quantization ("Efficient MoE Training for Biological
// Foundation Models", Challenge 2: one scaling factor per block of 32
// consecutive values; Challenge 3: BF16 activations and weights are
// quantized before the low-precision GEMMs).
//
// Two layouts, both giving each GEMM operand its 32-blocks along the GEMM's
// reduction axis with the blocks contiguous in memory:
//   rows:   blocks of 32 consecutive columns of a row-major [rows][cols]
//           tensor; codes keep the layout, scales are [rows][cols/32].
//   tokens: blocks of 32 consecutive rows, restarting at every segment
//           (expert) start; the output is transposed, codes [cols][rows_pad]
//           and scales [cols][rows_pad/32], where segment s starts at
//           column pad_off[s] = sum over s' < s of round_up(len_s', 128)
//           and padding holds code 0 with scale byte 0.

#include "common.cuh"
#include "internal.h"
#include "mx.cuh"

namespace moe {
namespace {

// One thread per 32-block of a row.
__global__ __launch_bounds__(256) void quant_rows_kernel(
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
  const int e = mx_scale_exp(amax);
  const float inv = mx_inv_scale(e);
  i32x4 out[2];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      word |= e4m3_encode(v[q * 4 + b] * inv) << (8 * b);
    out[q >> 2][q & 3] = static_cast<int>(word);
  }
  i32x4* o = reinterpret_cast<i32x4*>(codes + blk * kMxBlock);
  o[0] = out[0];
  o[1] = out[1];
  scales[blk] = static_cast<uint8_t>(e + 127);
}

// Exclusive prefix of the 128-padded segment lengths into s_pad[0..nseg]
// (one wave), from device offsets seg[0..nseg] (or one segment of `rows`).
__device__ void padded_prefix(const int32_t* seg, int nseg, int64_t rows,
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

// Workgroup = one padded 32-row block x 256 columns; thread = column.
__global__ __launch_bounds__(256) void quant_tokens_kernel(
    const bf16_t* __restrict__ src, const int32_t* __restrict__ gather,
    int64_t rows, int64_t cols,
    const int32_t* __restrict__ seg, int nseg, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int64_t rows_pad) {
  __shared__ int s_pad[kMaxExperts + 1];
  padded_prefix(seg, nseg, rows, s_pad);
  const int64_t pb = blockIdx.x;                 // padded 32-row block
  const int64_t c = static_cast<int64_t>(blockIdx.y) * blockDim.x +
                    threadIdx.x;
  const int64_t p0 = pb * kMxBlock;              // first padded row
  // segment holding this block: largest s with s_pad[s] <= p0
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pad[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  int64_t r0 = 0, r_end = 0;                     // source rows [r0, r_end)
  if (p0 < s_pad[nseg]) {
    const int64_t sbeg = seg ? seg[s] : 0;
    const int64_t send = seg ? seg[s + 1] : rows;
    r0 = sbeg + (p0 - s_pad[s]);
    r_end = r0 + kMxBlock < send ? r0 + kMxBlock : send;
  }
  if (c >= cols) return;
  float v[kMxBlock];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) {
    const int64_t r = r0 + i;
    float x = 0.0f;
    if (r < r_end) {
      const int64_t sr = gather ? static_cast<int64_t>(gather[r]) : r;
      x = bf2f(src[sr * cols + c]);
    }
    v[i] = x;
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const int e = mx_scale_exp(amax);
  const float inv = mx_inv_scale(e);
  i32x4 out[2];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int i = q * 4 + b;
      const uint32_t cd = (r0 + i < r_end) ? e4m3_encode(v[i] * inv) : 0u;
      word |= cd << (8 * b);
    }
    out[q >> 2][q & 3] = static_cast<int>(word);
  }
  i32x4* o = reinterpret_cast<i32x4*>(codes + c * rows_pad + p0);
  o[0] = out[0];
  o[1] = out[1];
  scales[c * (rows_pad / kMxBlock) + pb] =
      static_cast<uint8_t>(r_end > r0 ? e + 127 : 0);
}

}  // namespace

hipError_t launch_mx_quant_rows(const bf16_t* src, int64_t rows, int64_t cols,
                                uint8_t* codes, uint8_t* scales,
                                hipStream_t s) {
  const int64_t blocks = rows * (cols / kMxBlock);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel,
                     dim3(static_cast<unsigned>((blocks + 255) / 256)),
                     dim3(256), 0, s, src, rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quant_tokens(const bf16_t* src, const int32_t* gather,
                                  int64_t rows, int64_t cols,
                                  const int32_t* seg, int nseg,
                                  uint8_t* codes, uint8_t* scales,
                                  int64_t rows_pad, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(rows_pad / kMxBlock),
            static_cast<unsigned>((cols + 255) / 256));
  hipLaunchKernelGGL(quant_tokens_kernel, grid, dim3(256), 0, s, src, gather,
                     rows, cols, seg, nseg, codes, scales, rows_pad);
  return hipGetLastError();
}

}  // namespace moe
