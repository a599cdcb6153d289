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

// An expert id outside [0, E) (the routing kernel never writes one; a
// caller's own idx might) is taken as the nearest valid id, so that no
// count, offset or row index leaves its buffer.
__device__ __forceinline__ int clamp_expert(int e, int E) {
  return min(max(e, 0), E - 1);
}

// ---------------------------------------------------------------- plan
// Pass 1: every wavefront ranks one chunk of `chunk` slots (a multiple of
// 64, see plan_chunk) in 64-slot steps.  For each step the lanes that share
// an expert id are grouped with ballots; a lane's rank is the number of
// lower lanes in its group plus the chunk's running count of that expert
// (the wave's own LDS row).  The rank within the chunk is stashed in pos;
// the chunk's counts go to ws.  Four waves a workgroup, each on its own
// chunk and LDS row, so only wave-level ordering is needed.
constexpr int kRankWaves = 4;

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(64 * kRankWaves) void plan_rank_kernel(
    const int32_t* __restrict__ idx, int64_t TK, int E, int chunk,
    int nchunks, int32_t* __restrict__ rank_out,
    int32_t* __restrict__ chunk_counts) {
  __shared__ int cnt_all[kRankWaves][kMaxExperts];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c = blockIdx.x * kRankWaves + w;
  if (c >= nchunks) return;                     // whole wave
  int* cnt = cnt_all[w];
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  wave_sync_lds();
  const int64_t c0 = static_cast<int64_t>(c) * chunk;
  const int64_t c1 = min(TK, c0 + chunk);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t s0 = c0; s0 < c1; s0 += 64) {
    const int64_t s = s0 + lane;
    const bool valid = s < c1;
    const int e = valid ? clamp_expert(idx[s], E) : -1;
    uint64_t active = __ballot(valid);
    int rank = 0, grp = 0;
    while (active) {
      const int leader = __ffsll(static_cast<unsigned long long>(active)) - 1;
      const int le = __builtin_amdgcn_readlane(e, leader);
      const uint64_t mask = __ballot(valid && e == le);
      if (valid && e == le) {
        rank = __popcll(mask & below);
        grp = __popcll(mask);
      }
      active &= ~mask;
    }
    const int base = valid ? cnt[e] : 0;
    wave_sync_lds();
    if (valid && rank == grp - 1) cnt[e] = base + grp;
    if (valid) rank_out[s] = base + rank;
    wave_sync_lds();
  }
  for (int e = lane; e < E; e += 64)
    chunk_counts[static_cast<int64_t>(c) * E + e] = cnt[e];
}

// Pass 2: one workgroup.  Each expert's column of chunk counts is turned
// into exclusive chunk bases (in place) and the expert total by a group of
// G lanes (G = 64 halved until G * E <= 1024); an exclusive scan over the
// experts' totals then gives the offsets.  Integer sums, so the result
// does not depend on how the work is split.  The kernel is one
// workgroup's latency.  A table that fits (kScanLds ints with its
// padding) is copied into LDS expert-major, rows of nchunks + 17 ints,
// with coalesced 16-byte loads all in flight together; the G lanes of an
// expert then walk its row G chunks a round (lane g takes chunk r G + g:
// a shuffle scan over the lanes plus the running carry), so the 64 lanes
// of a wave read distinct banks; the row is written back the same way.
// A larger table is scanned in place in global memory, lane g taking a
// contiguous range of chunks.
constexpr int kScanLds = 34816;       // ints of LDS table (136 KiB)
constexpr int kScanIn = 8;            // 16-byte loads in flight a thread
__global__ __launch_bounds__(1024) void plan_scan_kernel(
    int32_t* __restrict__ chunk_counts, int nchunks, int E,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int wsum[16];
  __shared__ int s_tab[kScanLds];
  const int t = threadIdx.x;
  const int n = nchunks * E;
  const int n4 = (E & 3) == 0 ? n >> 2 : 0;    // 16-byte moves need E % 4
  const int S = nchunks + 17;                   // LDS row stride (odd)
  const bool in_lds = S * E <= kScanLds;
  int G = 64;
  while (G > 1 && G * E > 1024) G >>= 1;
  const int e = t / G, g = t - (t / G) * G;
  if (in_lds) {
    // [chunk][expert] in global -> [expert][chunk] in LDS
    const i32x4* src = reinterpret_cast<const i32x4*>(chunk_counts);
    for (int b = t; b < n4; b += 1024 * kScanIn) {
      i32x4 v[kScanIn];
#pragma unroll
      for (int u = 0; u < kScanIn; ++u)
        v[u] = b + u * 1024 < n4 ? src[b + u * 1024] : i32x4{};
#pragma unroll
      for (int u = 0; u < kScanIn; ++u) {
        const int i = 4 * (b + u * 1024);
        if (i < n) {
          const int c = i / E, e4 = i - c * E;
#pragma unroll
          for (int q = 0; q < 4; ++q) s_tab[(e4 + q) * S + c] = v[u][q];
        }
      }
    }
    for (int i = 4 * n4 + t; i < n; i += 1024)
      s_tab[(i % E) * S + i / E] = chunk_counts[i];
    __syncthreads();
    int carry = 0;
    if (e < E) {
      int* row = s_tab + e * S;
      for (int c0 = 0; c0 < nchunks; c0 += G) {
        const int c = c0 + g;
        const int v = c < nchunks ? row[c] : 0;
        int incl = v;
        for (int m = 1; m < G; m <<= 1) {
          const int o = __shfl_up(incl, m, G);
          if (g >= m) incl += o;
        }
        if (c < nchunks) row[c] = carry + incl - v;
        carry += __shfl(incl, G - 1, G);
      }
      if (g == G - 1) {
        s_cnt[e] = carry;
        counts[e] = carry;
      }
    }
    __syncthreads();
    // back to [chunk][expert]
    for (int i = t; i < n; i += 1024) chunk_counts[i] = s_tab[(i % E) * S + i / E];
  } else {
    const int per = (nchunks + G - 1) / G;
    const int c0 = min(nchunks, g * per), c1 = min(nchunks, c0 + per);
    int32_t* col = chunk_counts + e;
    int sum = 0;
    if (e < E)
      for (int c = c0; c < c1; ++c) sum += col[static_cast<int64_t>(c) * E];
    int gincl = sum;
    for (int m = 1; m < G; m <<= 1) {
      const int o = __shfl_up(gincl, m, G);
      if (g >= m) gincl += o;
    }
    if (e < E) {
      int run = gincl - sum;
      for (int c = c0; c < c1; ++c) {
        const int v = col[static_cast<int64_t>(c) * E];
        col[static_cast<int64_t>(c) * E] = run;
        run += v;
      }
      if (g == G - 1) {
        s_cnt[e] = gincl;
        counts[e] = gincl;
      }
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
// A token's row of `bytes` (a multiple of 16) goes to the k rows
// dst_base + rows[j] * bytes (rows[] in LDS).  The first kRowPre 16-byte
// pieces of each thread are loaded before the destinations are known
// (RowPre::load, issued ahead of the position work) and stored after
// (RowPre::store); the rest of a long row is copied in a plain loop.
constexpr int kRowPre = 4;
struct RowPre {
  i32x4 v[kRowPre];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ src,
                                       int64_t bytes) {
    const int64_t n16 = bytes >> 4;
#pragma unroll
    for (int i = 0; i < kRowPre; ++i) {
      const int64_t q = threadIdx.x + static_cast<int64_t>(i) * blockDim.x;
      if (q < n16) v[i] = reinterpret_cast<const i32x4*>(src)[q];
    }
  }
  __device__ __forceinline__ void store(const uint8_t* __restrict__ src,
                                        uint8_t* __restrict__ dst_base,
                                        const int* rows, int k,
                                        int64_t bytes) const {
    const int64_t n16 = bytes >> 4;
#pragma unroll
    for (int i = 0; i < kRowPre; ++i) {
      const int64_t q = threadIdx.x + static_cast<int64_t>(i) * blockDim.x;
      if (q < n16)
        for (int j = 0; j < k; ++j)
          reinterpret_cast<i32x4*>(dst_base + static_cast<int64_t>(rows[j]) *
                                                  bytes)[q] = v[i];
    }
    for (int64_t q = threadIdx.x + static_cast<int64_t>(kRowPre) * blockDim.x;
         q < n16; q += blockDim.x) {
      const i32x4 w = reinterpret_cast<const i32x4*>(src)[q];
      for (int j = 0; j < k; ++j)
        reinterpret_cast<i32x4*>(dst_base + static_cast<int64_t>(rows[j]) *
                                                bytes)[q] = w;
    }
  }
};

// Side bytes (MX scales) of a row: 16 bytes at a time when the row length
// allows, else byte by byte.
__device__ __forceinline__ void copy_side(const uint8_t* __restrict__ src,
                                          uint8_t* __restrict__ dst_base,
                                          const int* rows, int k,
                                          int64_t bytes) {
  if ((bytes & 15) == 0) {
    const int64_t n16 = bytes >> 4;
    for (int64_t q = threadIdx.x; q < n16; q += blockDim.x) {
      const i32x4 v = reinterpret_cast<const i32x4*>(src)[q];
      for (int j = 0; j < k; ++j)
        reinterpret_cast<i32x4*>(dst_base + static_cast<int64_t>(rows[j]) *
                                                bytes)[q] = v;
    }
    return;
  }
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
    int E, int chunk, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ chunk_base, int32_t* __restrict__ pos,
    int32_t* __restrict__ src, float* __restrict__ w_perm,
    const uint8_t* __restrict__ x, int64_t row_bytes, uint8_t* __restrict__ xp,
    const uint8_t* __restrict__ side, int64_t side_bytes,
    uint8_t* __restrict__ side_p) {
  __shared__ int s_pos[kMaxTopK];
  const int64_t t = blockIdx.x;
  RowPre row;
  row.load(x + t * row_bytes, row_bytes);
  if (threadIdx.x < k) {
    const int j = threadIdx.x;
    const int64_t s = t * k + j;
    const int e = clamp_expert(idx[s], E);
    const int64_t c = s / chunk;
    const int p = offsets[e] + chunk_base[c * E + e] + pos[s];
    pos[s] = p;
    src[p] = static_cast<int32_t>(t);
    if (w_perm) w_perm[p] = topk_w[s];
    s_pos[j] = p;
  }
  __syncthreads();
  row.store(x + t * row_bytes, xp, s_pos, k, row_bytes);
  if (side) copy_side(side + t * side_bytes, side_p, s_pos, k, side_bytes);
}

__global__ __launch_bounds__(256) void permute_rows_kernel(
    const int32_t* __restrict__ pos, int k, const uint8_t* __restrict__ x,
    int64_t row_bytes, uint8_t* __restrict__ xp,
    const uint8_t* __restrict__ side, int64_t side_bytes,
    uint8_t* __restrict__ side_p) {
  __shared__ int s_pos[kMaxTopK];
  const int64_t t = blockIdx.x;
  RowPre row;
  row.load(x + t * row_bytes, row_bytes);
  if (threadIdx.x < k) s_pos[threadIdx.x] = pos[t * k + threadIdx.x];
  __syncthreads();
  row.store(x + t * row_bytes, xp, s_pos, k, row_bytes);
  if (side) copy_side(side + t * side_bytes, side_p, s_pos, k, side_bytes);
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

// slot of flattened (slot, plane) row r: planes is 1 or 2 in practice,
// which needs no division
__device__ __forceinline__ int slot_of(int r, int planes) {
  return planes == 1 ? r : planes == 2 ? (r >> 1) : r / planes;
}

// With dl (router score gradients [T][E] fp32) and wg (router weight
// [E][d] bf16), the router's share of the token's input gradient,
// sum over e in order of dl[t][e] * wg[e], is added to the fp32 sum before
// the one rounding, as moe_router_backward adds it to a given fp32 dx.  A
// workgroup takes TPB consecutive tokens, so each w_g row it loads serves
// TPB tokens (many experts would otherwise read w_g once per token).
template <bool OF32, int TPB>
__global__ __launch_bounds__(256) void unpermute_kernel(
    const void* __restrict__ o, int planes, int64_t plane,
    const int32_t* __restrict__ pos, const float* __restrict__ w, int k,
    int64_t T, int64_t d, int y_fp32, void* __restrict__ y,
    const float* __restrict__ dl, const bf16_t* __restrict__ wg, int E) {
  __shared__ int s_pos[TPB][kMaxTopK];
  __shared__ float s_w[TPB][kMaxTopK];
  __shared__ float s_dl[TPB > 1 ? TPB : 1][kMaxExperts];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TPB;
  const int nt = static_cast<int>(T - t0 < TPB ? T - t0 : TPB);
  if (dl)
    for (int i = threadIdx.x; i < nt * E; i += blockDim.x)
      s_dl[i / E][i % E] = dl[t0 * E + i];
  if (threadIdx.x < nt) {
    // insertion sort of the token's k rows (k <= 32)
    const int tt = threadIdx.x;
    const int64_t t = t0 + tt;
    for (int j = 0; j < k; ++j) {
      const int p = pos[t * k + j];
      const float wj = w ? w[t * k + j] : 1.0f;
      int i = j;
      while (i > 0 && s_pos[tt][i - 1] > p) {
        s_pos[tt][i] = s_pos[tt][i - 1];
        s_w[tt][i] = s_w[tt][i - 1];
        --i;
      }
      s_pos[tt][i] = p;
      s_w[tt][i] = wj;
    }
  }
  __syncthreads();
  // A token's rows, taken as (slot, plane) pairs in order (slots
  // ascending, a slot's planes in plane order), are loaded kUnBatch at a
  // time with every load of a batch in flight before any is added; the
  // additions keep that order.
  constexpr int kUnBatch = 8;
  const int nrow = k * planes;
  const int64_t n8 = d >> 3;
  for (int64_t q = threadIdx.x; q < n8; q += blockDim.x) {
    float acc[TPB][8];
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[tt][c] = 0.0f;
      if (tt >= nt) continue;
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int r0 = 0; r0 < nrow; r0 += kUnBatch) {
        float u[kUnBatch][8];
#pragma unroll
        for (int b = 0; b < kUnBatch; ++b) {
          const int r = r0 + b;
          if (r < nrow) {
            const int j = slot_of(r, planes), pl = r - j * planes;
            load8<OF32>(OF32 ? static_cast<const void*>(
                                   static_cast<const float*>(o) + pl * plane)
                             : o,
                        s_pos[tt][j], d, q, u[b]);
          }
        }
#pragma unroll
        for (int b = 0; b < kUnBatch; ++b) {
          const int r = r0 + b;
          if (r >= nrow) break;
          const int j = slot_of(r, planes), pl = r - j * planes;
          if (pl == 0) {
#pragma unroll
            for (int c = 0; c < 8; ++c) v[c] = u[b][c];
          } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) v[c] += u[b][c];
          }
          if (pl == planes - 1) {
            if (w) {
              const float wj = s_w[tt][j];
#pragma unroll
              for (int c = 0; c < 8; ++c) acc[tt][c] += wj * v[c];
            } else {
#pragma unroll
              for (int c = 0; c < 8; ++c) acc[tt][c] += v[c];
            }
          }
        }
      }
    }
    if (dl) {
      // w_g rows of kUnBatch experts in flight at a time, experts in order
      const int64_t col = q * 8;
      for (int e0 = 0; e0 < E; e0 += kUnBatch) {
        i32x4 wr[kUnBatch];
#pragma unroll
        for (int b = 0; b < kUnBatch; ++b)
          wr[b] = e0 + b < E ? *reinterpret_cast<const i32x4*>(
                                   wg + static_cast<int64_t>(e0 + b) * d + col)
                             : i32x4{};
#pragma unroll
        for (int b = 0; b < kUnBatch; ++b) {
          if (e0 + b >= E) break;
          float wv[8];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            wv[2 * c] = bf_lo(static_cast<uint32_t>(wr[b][c]));
            wv[2 * c + 1] = bf_hi(static_cast<uint32_t>(wr[b][c]));
          }
#pragma unroll
          for (int tt = 0; tt < TPB; ++tt) {
            const float g = s_dl[TPB > 1 ? tt : 0][e0 + b];
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[tt][c] += g * wv[c];
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt) {
      if (tt >= nt) break;
      const int64_t t = t0 + tt;
      if (y_fp32) {
        f32x4* yp =
            reinterpret_cast<f32x4*>(static_cast<float*>(y) + t * d) + 2 * q;
        yp[0] = f32x4{acc[tt][0], acc[tt][1], acc[tt][2], acc[tt][3]};
        yp[1] = f32x4{acc[tt][4], acc[tt][5], acc[tt][6], acc[tt][7]};
      } else {
        i32x4 out;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          out[c] = static_cast<int>(
              pack_bf16x2(acc[tt][2 * c], acc[tt][2 * c + 1]));
        reinterpret_cast<i32x4*>(static_cast<bf16_t*>(y) + t * d)[q] = out;
      }
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
  // 8 tiles' loads in flight at a time, added in tile order
  float acc = 0.0f;
  for (int n0 = 0; n0 < ntn; n0 += 8) {
    float v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) v[b] = n0 + b < ntn ? p[n0 + b] : 0.0f;
#pragma unroll
    for (int b = 0; b < 8; ++b)
      if (n0 + b < ntn) acc += v[b];
  }
  dp[s] = acc;
}

}  // namespace

// Slots per chunk of the counting pass: a power of two at least 64, E and
// Tk / 512.  So there are at most 512 chunks (their counts fill at most
// 512 * E * 4 bytes, 2 MiB at E = 1024), and each wave ranks few 64-slot
// steps while the small problems still spread over many waves.
int plan_chunk(int64_t Tk, int E) {
  int64_t c = 64;
  while (c < E || c * 512 < Tk) c <<= 1;
  return static_cast<int>(c);
}

size_t plan_workspace_bytes(int64_t Tk, int E) {
  const int64_t chunk = plan_chunk(Tk, E);
  const int64_t nchunks = (Tk + chunk - 1) / chunk;
  return static_cast<size_t>(nchunks * E * sizeof(int32_t));
}

hipError_t launch_plan(const int32_t* idx, int64_t T, int E, int k,
                       int32_t* counts, int32_t* offsets, int32_t* pos,
                       void* ws, hipStream_t s) {
  const int64_t TK = T * k;
  const int chunk = plan_chunk(TK, E);
  const int nchunks = static_cast<int>((TK + chunk - 1) / chunk);
  int32_t* chunk_counts = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(plan_rank_kernel,
                     dim3((nchunks + kRankWaves - 1) / kRankWaves),
                     dim3(64 * kRankWaves), 0, s, idx, TK, E, chunk, nchunks,
                     pos, chunk_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, s,
                     chunk_counts, nchunks, E, counts, offsets);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* idx, const float* topk_w, int64_t T,
                          int E, int k, const int32_t* offsets, int32_t* pos,
                          int32_t* src, float* w_perm, const void* x,
                          int64_t row_bytes, void* x_perm, const void* side,
                          int64_t side_bytes, void* side_perm, const void* ws,
                          hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3(static_cast<unsigned>(T)), dim3(256),
                     0, s, idx, topk_w, k, E, plan_chunk(T * k, E), offsets,
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
                            const float* dl, const bf16_t* wg, int E,
                            hipStream_t s) {
  const int64_t plane = T * k * d;
  const int planes = o_fp32 ? o_planes : 1;
  // with the router's share of many experts, 4 tokens a workgroup share
  // each w_g row they load
  if (dl && E > 8) {
    constexpr int kTpb = 4;
    const dim3 grid(static_cast<unsigned>((T + kTpb - 1) / kTpb));
    if (o_fp32)
      hipLaunchKernelGGL((unpermute_kernel<true, kTpb>), grid, dim3(256), 0,
                         s, o, planes, plane, pos, w, k, T, d, y_fp32, y, dl,
                         wg, E);
    else
      hipLaunchKernelGGL((unpermute_kernel<false, kTpb>), grid, dim3(256), 0,
                         s, o, planes, plane, pos, w, k, T, d, y_fp32, y, dl,
                         wg, E);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(T));
  if (o_fp32)
    hipLaunchKernelGGL((unpermute_kernel<true, 1>), grid, dim3(256), 0, s, o,
                       planes, plane, pos, w, k, T, d, y_fp32, y, dl, wg, E);
  else
    hipLaunchKernelGGL((unpermute_kernel<false, 1>), grid, dim3(256), 0, s, o,
                       planes, plane, pos, w, k, T, d, y_fp32, y, dl, wg, E);
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
