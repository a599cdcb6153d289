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
  for (int q = 0; q < 8; ++q)
    out[q >> 2][q & 3] = static_cast<int>(
        e4m3_pack4(v[q * 4] * inv, v[q * 4 + 1] * inv, v[q * 4 + 2] * inv,
                   v[q * 4 + 3] * inv));
  i32x4* o = reinterpret_cast<i32x4*>(codes + blk * kMxBlock);
  o[0] = out[0];
  o[1] = out[1];
  scales[blk] = static_cast<uint8_t>(e + 127);
}


// Workgroup = one 128-row tile of the padded layout x kTokTiles runs of 64
// columns (kTokTilesRows with the row-wise outputs; a tile never straddles
// a segment: segments start on multiples of 128), each run in three steps:
//   1. 256 threads load the tile's source rows with 16-byte loads (8
//      columns each; rows past the segment read as zero) into LDS;
//   2. thread (block b = t/64, column c = t%64) quantizes its 32-row block
//      of one column and writes the 32 codes to an LDS staging line;
//   3. every column's 128 codes leave as one 128-byte line (8 lanes, 16
//      bytes each) and its 4 scale bytes as one 4-byte word.
// With kRows (one segment, no gather: a weight quantized for both of its
// GEMMs from one read) thread (row t/2, half t%2) also quantizes its 32
// columns of the tile along the row, as quant_rows_kernel does, into
// row_codes [rows][cols] and row_scales [rows][cols/32].  Those are kept in
// LDS over the workgroup's column runs and leave at the end as whole rows
// of the runs (128 code bytes, 8 lanes a row, and one 4-byte scale word a
// row), so the row-wise outputs go out in full lines instead of 64-byte
// pieces and single bytes.
constexpr int kTokRows = 128;
constexpr int kTokCols = 64;
constexpr int kTokLd = kTokCols + 8;       // bf16 row stride of the tile
constexpr int kTokTiles = 4;               // column runs per workgroup
constexpr int kTokTilesRows = 2;           // ... with the row-wise outputs

template <bool kRows>
__global__ __launch_bounds__(256) void quant_tokens_kernel(
    const bf16_t* __restrict__ src, const int32_t* __restrict__ gather,
    int64_t rows, int64_t cols, const int32_t* __restrict__ seg, int nseg,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    int64_t rows_pad, uint8_t* __restrict__ row_codes,
    uint8_t* __restrict__ row_scales) {
  __shared__ int s_pad[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) bf16_t tile[kTokRows * kTokLd];
  __shared__ __attribute__((aligned(16))) uint8_t out[kTokCols][kTokRows];
  __shared__ uint32_t sc_out[kTokCols];
  constexpr int kRuns = kRows ? kTokTilesRows : kTokTiles;
  // kRows: the row-wise codes and scales of all the column runs
  constexpr int kRowBytes = kTokCols * kRuns;
  __shared__ __attribute__((aligned(16)))
  uint8_t rcodes[kRows ? kTokRows : 1][kRows ? kRowBytes : 16];
  __shared__ __attribute__((aligned(4)))
  uint8_t rscales[kRows ? kTokRows : 1][kRows ? kRowBytes / kMxBlock : 4];
  padded_prefix(seg, nseg, rows, s_pad);
  const int t = threadIdx.x;
  // Workgroup order: each XCD takes a contiguous range of (row tile,
  // column group) pairs, column group fastest, so the 4-byte scale pieces
  // that neighbouring workgroups write into one 32-byte sector (row-wise:
  // the column groups of a row tile; along tokens: consecutive row tiles)
  // leave one XCD close together and can merge in its L2.
  const int ngy = static_cast<int>(gridDim.y);
  const int lin = xcd_remap(
      static_cast<int>(blockIdx.y * gridDim.x + blockIdx.x),
      static_cast<int>(gridDim.x) * ngy);
  const int bx = lin / ngy, by = lin % ngy;
  const int64_t p0 = static_cast<int64_t>(bx) * kTokRows;
  // segment holding this tile: largest s with s_pad[s] <= p0
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pad[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  int64_t r0 = 0, r_end = 0;                     // source rows [r0, r_end)
  if (p0 < s_pad[nseg]) {
    const int64_t sbeg = seg ? seg[lo] : 0;
    const int64_t send = seg ? seg[lo + 1] : rows;
    r0 = sbeg + (p0 - s_pad[lo]);
    r_end = r0 + kTokRows < send ? r0 + kTokRows : send;
  }
  // 1. load: thread t covers columns 8 (t%8) .. +7 of rows t/8 + 32 i of
  // column run ct; the next run's loads are issued as soon as this run is
  // in LDS, so they land while this run is quantized and written
  const int cc = (t & 7) * 8;
  i32x4 nxt[kTokRows / 32];
  auto load_run = [&](int ct) {
    const int64_t c0 =
        (static_cast<int64_t>(by) * kRuns + ct) * kTokCols;
    const bool col_ok = c0 + cc < cols;            // cols % 8 == 0
#pragma unroll
    for (int i = 0; i < kTokRows / 32; ++i) {
      const int rr = (t >> 3) + 32 * i;
      nxt[i] = i32x4{0, 0, 0, 0};
      if (col_ok && r0 + rr < r_end) {
        const int64_t r = r0 + rr;
        const int64_t sr = gather ? static_cast<int64_t>(gather[r]) : r;
        nxt[i] = *reinterpret_cast<const i32x4*>(src + sr * cols + c0 + cc);
      }
    }
  };
  load_run(0);
  for (int ct = 0; ct < kRuns; ++ct) {
    const int64_t c0 =
        (static_cast<int64_t>(by) * kRuns + ct) * kTokCols;
    if (c0 >= cols) break;
    if (ct > 0) __syncthreads();                   // LDS of the previous run
#pragma unroll
    for (int i = 0; i < kTokRows / 32; ++i)
      *reinterpret_cast<i32x4*>(tile + ((t >> 3) + 32 * i) * kTokLd + cc) =
          nxt[i];
    __syncthreads();
    if (ct + 1 < kRuns) load_run(ct + 1);
    if constexpr (kRows) {
      // along the row: 32 columns of row t/2 (c0 is a multiple of 64)
      const int rr = t >> 1, half = t & 1;
      const int64_t r = r0 + rr;
      if (r < r_end && c0 + 32 * half < cols) {
        float v[kMxBlock];
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x4 w = *reinterpret_cast<const i32x4*>(
              tile + rr * kTokLd + 32 * half + 8 * q);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            v[q * 8 + 2 * c] = bf_lo(static_cast<uint32_t>(w[c]));
            v[q * 8 + 2 * c + 1] = bf_hi(static_cast<uint32_t>(w[c]));
          }
        }
#pragma unroll
        for (int i = 0; i < kMxBlock; ++i) amax = fmaxf(amax, fabsf(v[i]));
        const int e = mx_scale_exp(amax);
        const float inv = mx_inv_scale(e);
        i32x4 w[2];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          w[q >> 2][q & 3] = static_cast<int>(
              e4m3_pack4(v[q * 4] * inv, v[q * 4 + 1] * inv,
                         v[q * 4 + 2] * inv, v[q * 4 + 3] * inv));
        const int lc = ct * kTokCols + 32 * half;     // column in the runs
        i32x4* o = reinterpret_cast<i32x4*>(&rcodes[rr][lc]);
        o[0] = w[0];
        o[1] = w[1];
        rscales[rr][lc / kMxBlock] = static_cast<uint8_t>(e + 127);
      }
    }
    // 2. quantize one 32-row block of one column
    {
      const int c = t & (kTokCols - 1);
      const int b = t / kTokCols;                  // block 0..3 of the tile
      float v[kMxBlock];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < kMxBlock; ++i) {
        v[i] = bf2f(tile[(b * kMxBlock + i) * kTokLd + c]);
        amax = fmaxf(amax, fabsf(v[i]));
      }
      const int e = mx_scale_exp(amax);           // all-zero block: byte 0
      const float inv = mx_inv_scale(e);
      i32x4 w[2];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[q >> 2][q & 3] = static_cast<int>(
            e4m3_pack4(v[q * 4] * inv, v[q * 4 + 1] * inv,
                       v[q * 4 + 2] * inv, v[q * 4 + 3] * inv));
      *reinterpret_cast<i32x4*>(&out[c][b * kMxBlock]) = w[0];
      *reinterpret_cast<i32x4*>(&out[c][b * kMxBlock + 16]) = w[1];
      reinterpret_cast<uint8_t*>(sc_out)[c * 4 + b] =
          static_cast<uint8_t>(e + 127);
    }
    __syncthreads();
    // 3. write: 64 columns x 128 code bytes, 8 lanes a line
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int id = t + 256 * j;
      const int col = id >> 3, chunk = id & 7;
      if (c0 + col < cols)
        *reinterpret_cast<i32x4*>(codes + (c0 + col) * rows_pad + p0 +
                                  chunk * 16) =
            *reinterpret_cast<const i32x4*>(&out[col][chunk * 16]);
    }
    if (t < kTokCols && c0 + t < cols)
      *reinterpret_cast<uint32_t*>(scales + (c0 + t) * (rows_pad / kMxBlock) +
                                   p0 / kMxBlock) = sc_out[t];
  }
  if constexpr (kRows) {
    // the runs' row-wise codes: kChunks lanes a row, 16 bytes each; scales:
    // kRowBytes / 32 bytes a row (cols is a multiple of 64, so a run is all
    // in or all out)
    __syncthreads();
    constexpr int kChunks = kRowBytes / 16;
    const int64_t cw0 = static_cast<int64_t>(by) * kRowBytes;
    const int64_t ncols = cols - cw0 < kRowBytes ? cols - cw0 : kRowBytes;
#pragma unroll
    for (int j = 0; j < kTokRows * kChunks / 256; ++j) {
      const int id = t + 256 * j;
      const int rr = id / kChunks, ch = id % kChunks;
      const int64_t r = r0 + rr;
      if (r < r_end && ch * 16 < ncols)
        *reinterpret_cast<i32x4*>(row_codes + r * cols + cw0 + ch * 16) =
            *reinterpret_cast<const i32x4*>(&rcodes[rr][ch * 16]);
    }
    if (t < kTokRows) {
      const int64_t r = r0 + t;
      const int nsc = static_cast<int>(ncols / kMxBlock);
      uint8_t* dst = row_scales + r * (cols / kMxBlock) + cw0 / kMxBlock;
      if (r < r_end) {
        if (nsc == 4 && kRowBytes / kMxBlock == 4 &&
            ((reinterpret_cast<uintptr_t>(dst) & 3) == 0))
          *reinterpret_cast<uint32_t*>(dst) =
              *reinterpret_cast<const uint32_t*>(&rscales[t][0]);
        else
          for (int i = 0; i < nsc; ++i) dst[i] = rscales[t][i];
      }
    }
  }
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
  dim3 grid(static_cast<unsigned>(rows_pad / kTokRows),
            static_cast<unsigned>((cols + kTokCols * kTokTiles - 1) /
                                  (kTokCols * kTokTiles)));
  hipLaunchKernelGGL(quant_tokens_kernel<false>, grid, dim3(256), 0, s, src,
                     gather, rows, cols, seg, nseg, codes, scales, rows_pad,
                     nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_mx_quant_both(const bf16_t* src, int64_t rows,
                                int64_t cols, uint8_t* row_codes,
                                uint8_t* row_scales, uint8_t* col_codes,
                                uint8_t* col_scales, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(rows / kTokRows),
            static_cast<unsigned>((cols + kTokCols * kTokTilesRows - 1) /
                                  (kTokCols * kTokTilesRows)));
  hipLaunchKernelGGL(quant_tokens_kernel<true>, grid, dim3(256), 0, s, src,
                     nullptr, rows, cols, nullptr, 1, col_codes, col_scales,
                     rows, row_codes, row_scales);
  return hipGetLastError();
}

}  // namespace moe
