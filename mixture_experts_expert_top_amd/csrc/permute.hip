// Dispatch plan, token permutation, un-permute combine and the routing
// weight gradient reduction on gfx950.
//
// "Efficient MoE Training for Biological Foundation Models", Challenge 1:
// every expert gathers the tokens that chose it (GroupedLinear takes the
// per-expert token counts, split_sizes) and the expert outputs are
// index-added back into each token's output.  Here the grouping is a stable
// counting sort of the flat slot index t*k+j (integer, exact, ordered by
// token inside each expert) and the combine is a gather in ascending expert
// order with fp32 accumulation -- no atomics, so results are deterministic.

#include "common.cuh"
#include "internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- plan
// Pass 1: one wavefront per chunk of kPlanChunk slots walks its chunk in
// 64-slot steps.  For each step the lanes that share an expert id are
// grouped with ballots; a lane's rank is the number of lower lanes in its
// group plus the chunk's running count of that expert (LDS).  The rank
// within the chunk is stashed in pos; the chunk's counts go to ws.
__global__ __launch_bounds__(64) void plan_rank_kernel(
    const int32_t* __restrict__ idx, int64_t TK, int E,
    int32_t* __restrict__ rank_out, int32_t* __restrict__ chunk_counts) {
  __shared__ int cnt[kMaxExperts];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kPlanChunk;
  const int64_t c1 = min(TK, c0 + kPlanChunk);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t s0 = c0; s0 < c1; s0 += 64) {
    const int64_t s = s0 + lane;
    const bool valid = s < c1;
    const int e = valid ? idx[s] : -1;
    uint64_t active = __ballot(valid);
    int rank = 0, grp = 0;
    while (active) {
      const int leader = __ffsll(static_cast<unsigned long long>(active)) - 1;
      const int le = __shfl(e, leader, 64);
      const uint64_t mask = __ballot(valid && e == le);
      if (valid && e == le) {
        rank = __popcll(mask & below);
        grp = __popcll(mask);
      }
      active &= ~mask;
    }
    const int base = valid ? cnt[e] : 0;
    __syncthreads();
    if (valid && rank == grp - 1) cnt[e] = base + grp;
    if (valid) rank_out[s] = base + rank;
    __syncthreads();
  }
  for (int e = lane; e < E; e += 64)
    chunk_counts[static_cast<int64_t>(blockIdx.x) * E + e] = cnt[e];
}

// Pass 2: one workgroup.  Each expert's column of chunk counts is turned
// into exclusive chunk bases (in place) and the expert total by a group of
// G lanes (G = 64 halved until G * E <= 1024): lane g sums its contiguous
// range of chunks, the group scans those sums, and each lane rewrites its
// range from its base.  An exclusive scan over experts then gives the
// offsets.  Integer sums, so the result does not depend on the split.
__global__ __launch_bounds__(1024) void plan_scan_kernel(
    int32_t* __restrict__ chunk_counts, int nchunks, int E,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int wsum[16];
  int G = 64;
  while (G > 1 && G * E > 1024) G >>= 1;
  const int t = threadIdx.x;
  const int e = t / G, g = t - (t / G) * G;
  const int per = (nchunks + G - 1) / G;
  const int c0 = min(nchunks, g * per), c1 = min(nchunks, c0 + per);
  int sum = 0;
  if (e < E)
    for (int c = c0; c < c1; ++c)
      sum += chunk_counts[static_cast<int64_t>(c) * E + e];
  int gincl = sum;
  for (int m = 1; m < G; m <<= 1) {
    const int o = __shfl_up(gincl, m, G);
    if (g >= m) gincl += o;
  }
  if (e < E) {
    int run = gincl - sum;
    for (int c = c0; c < c1; ++c) {
      int32_t* p = chunk_counts + static_cast<int64_t>(c) * E + e;
      const int v = *p;
      *p = run;
      run += v;
    }
    if (g == G - 1) {
      s_cnt[e] = gincl;
      counts[e] = gincl;
    }
  }
  __syncthreads();
  // block-wide exclusive scan over experts: thread t holds expert t
  const int tot = t < E ? s_cnt[t] : 0;
  const int lane = t & 63, w = t >> 6;
  int incl = tot;
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m, 64);
    if (lane >= m) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int i = 0; i < 16; ++i) {
      const int v = wsum[i];
      wsum[i] = acc;
      acc += v;
    }
  }
  __syncthreads();
  const int excl = wsum[w] + incl - tot;
  if (t < E) offsets[t] = excl;
  if (t == E - 1) offsets[E] = excl + tot;
}

// ---------------------------------------------------------------- rows
// Copy one row of `bytes` (multiple of 16) from src to the k rows
// dst_base + rows[j] * stride.  rows[] lives in LDS.
__device__ __forceinline__ void copy_row16(const uint8_t* __restrict__ src,
                                           uint8_t* __restrict__ dst_base,
                                           const int* rows, int k,
                                           int64_t bytes) {
  const int64_t n16 = bytes >> 4;
  for (int64_t q = threadIdx.x; q < n16; q += blockDim.x) {
    const i32x4 v = reinterpret_cast<const i32x4*>(src)[q];
    for (int j = 0; j < k; ++j)
      reinterpret_cast<i32x4*>(dst_base + static_cast<int64_t>(rows[j]) *
                                              bytes)[q] = v;
  }
}

__device__ __forceinline__ void copy_row1(const uint8_t* __restrict__ src,
                                          uint8_t* __restrict__ dst_base,
                                          const int* rows, int k,
                                          int64_t bytes) {
  for (int64_t q = threadIdx.x; q < bytes; q += blockDim.x) {
    const uint8_t v = src[q];
    for (int j = 0; j < k; ++j)
      dst_base[static_cast<int64_t>(rows[j]) * bytes + q] = v;
  }
}

// Pass 3: one workgroup per token: final positions, src, w_perm, then the
// token's row (and side bytes) copied to its k permuted rows.
__global__ __launch_bounds__(256) void scatter_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ topk_w, int k,
    int E, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ chunk_base, int32_t* __restrict__ pos,
    int32_t* __restrict__ src, float* __restrict__ w_perm,
    const uint8_t* __restrict__ x, int64_t row_bytes, uint8_t* __restrict__ xp,
    const uint8_t* __restrict__ side, int64_t side_bytes,
    uint8_t* __restrict__ side_p) {
  __shared__ int s_pos[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    const int64_t s = t * k + j;
    const int e = idx[s];
    const int64_t c = s / kPlanChunk;
    const int p = offsets[e] + chunk_base[c * E + e] + pos[s];
    pos[s] = p;
    src[p] = static_cast<int32_t>(t);
    if (w_perm) w_perm[p] = topk_w[s];
    s_pos[j] = p;
  }
  __syncthreads();
  copy_row16(x + t * row_bytes, xp, s_pos, k, row_bytes);
  if (side) copy_row1(side + t * side_bytes, side_p, s_pos, k, side_bytes);
}

__global__ __launch_bounds__(256) void permute_rows_kernel(
    const int32_t* __restrict__ pos, int k, const uint8_t* __restrict__ x,
    int64_t row_bytes, uint8_t* __restrict__ xp,
    const uint8_t* __restrict__ side, int64_t side_bytes,
    uint8_t* __restrict__ side_p) {
  __shared__ int s_pos[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) s_pos[threadIdx.x] = pos[t * k + threadIdx.x];
  __syncthreads();
  copy_row16(x + t * row_bytes, xp, s_pos, k, row_bytes);
  if (side) copy_row1(side + t * side_bytes, side_p, s_pos, k, side_bytes);
}

// ---------------------------------------------------------------- combine
// y[t] = sum_j wt_j * O[pos[t][j]] with the slots taken in ascending
// permuted row (= ascending expert id).  One workgroup per token; a thread
// owns 8 consecutive columns.  O rows are bf16 or fp32 (OF32).
template <bool OF32>
__device__ __forceinline__ void load8(const void* o, int64_t row, int64_t d,
                                      int64_t q, float* v) {
  if (OF32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(
                         static_cast<const float*>(o) + row * d) + 2 * q;
    const f32x4 a = p[0], b = p[1];
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else {
    const i32x4 x = reinterpret_cast<const i32x4*>(
        static_cast<const bf16_t*>(o) + row * d)[q];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[2 * c] = bf_lo(static_cast<uint32_t>(x[c]));
      v[2 * c + 1] = bf_hi(static_cast<uint32_t>(x[c]));
    }
  }
}

template <bool OF32>
__global__ __launch_bounds__(256) void unpermute_kernel(
    const void* __restrict__ o, int planes, int64_t plane,
    const int32_t* __restrict__ pos, const float* __restrict__ w, int k,
    int64_t d, int y_fp32, void* __restrict__ y) {
  __shared__ int s_pos[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x == 0) {
    // insertion sort of the token's k rows (k <= 32)
    for (int j = 0; j < k; ++j) {
      const int p = pos[t * k + j];
      const float wj = w ? w[t * k + j] : 1.0f;
      int i = j;
      while (i > 0 && s_pos[i - 1] > p) {
        s_pos[i] = s_pos[i - 1];
        s_w[i] = s_w[i - 1];
        --i;
      }
      s_pos[i] = p;
      s_w[i] = wj;
    }
  }
  __syncthreads();
  const int64_t n8 = d >> 3;
  for (int64_t q = threadIdx.x; q < n8; q += blockDim.x) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      float v[8];
      load8<OF32>(o, s_pos[j], d, q, v);
      // further partial-sum planes of the same row, in plane order
      for (int pl = 1; pl < planes; ++pl) {
        float u[8];
        load8<OF32>(static_cast<const float*>(o) + pl * plane, s_pos[j], d, q,
                    u);
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] += u[c];
      }
      if (w) {
        const float wj = s_w[j];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += wj * v[c];
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += v[c];
      }
    }
    if (y_fp32) {
      f32x4* yp = reinterpret_cast<f32x4*>(static_cast<float*>(y) + t * d) + 2 * q;
      yp[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
      yp[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      i32x4 out;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        out[c] = static_cast<int>(pack_bf16x2(acc[2 * c], acc[2 * c + 1]));
      reinterpret_cast<i32x4*>(static_cast<bf16_t*>(y) + t * d)[q] = out;
    }
  }
}

// dp[t][j] = sum over n-tiles (ascending) of dp_part[pos[t][j]][n]
__global__ __launch_bounds__(256) void dp_reduce_kernel(
    const float* __restrict__ part, int ntn, const int32_t* __restrict__ pos,
    int64_t TK, float* __restrict__ dp) {
  const int64_t s = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (s >= TK) return;
  const float* p = part + static_cast<int64_t>(pos[s]) * ntn;
  float acc = 0.0f;
  for (int n = 0; n < ntn; ++n) acc += p[n];
  dp[s] = acc;
}

}  // namespace

size_t plan_workspace_bytes(int64_t Tk, int E) {
  const int64_t nchunks = (Tk + kPlanChunk - 1) / kPlanChunk;
  return static_cast<size_t>(nchunks * E * sizeof(int32_t));
}

hipError_t launch_plan(const int32_t* idx, int64_t T, int E, int k,
                       int32_t* counts, int32_t* offsets, int32_t* pos,
                       void* ws, hipStream_t s) {
  const int64_t TK = T * k;
  const int nchunks = static_cast<int>((TK + kPlanChunk - 1) / kPlanChunk);
  int32_t* chunk = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(plan_rank_kernel, dim3(nchunks), dim3(64), 0, s, idx, TK,
                     E, pos, chunk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, s, chunk,
                     nchunks, E, counts, offsets);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* idx, const float* topk_w, int64_t T,
                          int E, int k, const int32_t* offsets, int32_t* pos,
                          int32_t* src, float* w_perm, const void* x,
                          int64_t row_bytes, void* x_perm, const void* side,
                          int64_t side_bytes, void* side_perm, const void* ws,
                          hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3(static_cast<unsigned>(T)), dim3(256),
                     0, s, idx, topk_w, k, E, offsets,
                     static_cast<const int32_t*>(ws), pos, src, w_perm,
                     static_cast<const uint8_t*>(x), row_bytes,
                     static_cast<uint8_t*>(x_perm),
                     static_cast<const uint8_t*>(side), side_bytes,
                     static_cast<uint8_t*>(side_perm));
  return hipGetLastError();
}

hipError_t launch_permute_rows(const int32_t* pos, int64_t T, int k,
                               const void* x, int64_t row_bytes, void* x_perm,
                               const void* side, int64_t side_bytes,
                               void* side_perm, hipStream_t s) {
  hipLaunchKernelGGL(permute_rows_kernel, dim3(static_cast<unsigned>(T)),
                     dim3(256), 0, s, pos, k, static_cast<const uint8_t*>(x),
                     row_bytes, static_cast<uint8_t*>(x_perm),
                     static_cast<const uint8_t*>(side), side_bytes,
                     static_cast<uint8_t*>(side_perm));
  return hipGetLastError();
}

hipError_t launch_unpermute(const void* o, int o_fp32, int o_planes,
                            const int32_t* pos, const float* w, int64_t T,
                            int k, int64_t d, int y_fp32, void* y,
                            hipStream_t s) {
  const int64_t plane = T * k * d;
  if (o_fp32)
    hipLaunchKernelGGL(unpermute_kernel<true>, dim3(static_cast<unsigned>(T)),
                       dim3(256), 0, s, o, o_planes, plane, pos, w, k, d,
                       y_fp32, y);
  else
    hipLaunchKernelGGL(unpermute_kernel<false>, dim3(static_cast<unsigned>(T)),
                       dim3(256), 0, s, o, 1, plane, pos, w, k, d, y_fp32, y);
  return hipGetLastError();
}

hipError_t launch_dp_reduce(const float* dp_part, int ntn, const int32_t* pos,
                            int64_t T, int k, float* dp, hipStream_t s) {
  const int64_t TK = T * k;
  hipLaunchKernelGGL(dp_reduce_kernel,
                     dim3(static_cast<unsigned>((TK + 255) / 256)), dim3(256),
                     0, s, dp_part, ntn, pos, TK, dp);
  return hipGetLastError();
}

}  // namespace moe
