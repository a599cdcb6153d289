// Router scores and top-k routing on gfx950.
//
// "How MoE Architecture Cuts Costs and Boosts Efficiency", section "Why
// Biology Is Especially Well-Suited for MoE": the router gives every expert
// a score and only the K best-scoring experts run for a token.
// "Efficient MoE Training for Biological Foundation Models", Challenge 1:
// the chosen experts' outputs are scaled by routing weights.

#include <math.h>

#include "common.cuh"
#include "internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- logits
// logits[t][e] = x[t] . w_g[e] (+ bias[e]); a skinny GEMM (N = E) on bf16
// MFMA 32x32x16.  A workgroup owns 32 tokens x 32 experts; its 4 waves
// split d into 4 contiguous quarters and their partial tiles are summed in
// LDS in wave order (fixed, deterministic).
constexpr int kLogitThreads = 256;

__global__ __launch_bounds__(kLogitThreads) void router_logits_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
    const float* __restrict__ bias, int T, int d, int E,
    float* __restrict__ logits) {
  __shared__ float part[4][32 * 32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int row = lane & 31, kh = lane >> 5;
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(x, static_cast<uint32_t>(static_cast<int64_t>(T) * d * 2));
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(wg, static_cast<uint32_t>(static_cast<int64_t>(E) * d * 2));
  const int tok = t0 + row, ex = e0 + row;
  const bool tok_ok = tok < T, ex_ok = ex < E;
  // quarter of the reduction owned by this wave, in steps of 16
  const int steps = (d + 15) / 16;
  const int q = (steps + 3) / 4;
  const int s_begin = wave * q, s_end = min(steps, s_begin + q);
  f32x16 acc = {};
  for (int s = s_begin; s < s_end; ++s) {
    const int kk = s * 16 + kh * 8;
    const bool kok = kk < d;
    const uint32_t ox = (tok_ok && kok)
        ? static_cast<uint32_t>((static_cast<int64_t>(tok) * d + kk) * 2) : kOob;
    const uint32_t ow = (ex_ok && kok)
        ? static_cast<uint32_t>((static_cast<int64_t>(ex) * d + kk) * 2) : kOob;
    const bf16x8_v a = __builtin_bit_cast(bf16x8_v, buf_load16(rx, ox));
    const bf16x8_v b = __builtin_bit_cast(bf16x8_v, buf_load16(rw, ow));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  // acc[v] = C[token i][expert j], i = (v/4)*8 + kh*4 + v%4, j = lane%32
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int i = (v >> 2) * 8 + kh * 4 + (v & 3);
    part[wave][i * 32 + row] = acc[v];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 32 * 32; idx += kLogitThreads) {
    const int i = idx >> 5, j = idx & 31;
    const int t = t0 + i, e = e0 + j;
    if (t < T && e < E) {
      float s = part[0][idx];
      s += part[1][idx];
      s += part[2][idx];
      s += part[3][idx];
      if (bias) s += bias[e];
      logits[static_cast<int64_t>(t) * E + e] = s;
    }
  }
}

// ---------------------------------------------------------------- top-k
// G lanes (a power of two <= 64) own one token; lane g holds the scores of
// experts g, g+G, ..., (VPL of them).  k rounds of a butterfly arg-max over
// the G lanes pick the experts in order; the comparison is "larger score,
// or equal score and smaller id", so ties go to the lower id and +0 == -0.
__device__ __forceinline__ bool better(float va, int ea, float vb, int eb) {
  return (va > vb) || (va == vb && ea < eb);
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int G,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int gwave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int tpw = 64 / G;
  const int sub = lane / G, gl = lane % G;
  const int t = gwave * tpw + sub;
  const bool tok_ok = t < T;
  float v[VPL];
  bool live[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = gl + i * G;
    live[i] = tok_ok && e < E;
    v[i] = live[i] ? logits[static_cast<int64_t>(t) * E + e] : 0.0f;
  }
  float top = 0.0f, zsum = 0.0f;
  float z[kMaxTopK];
  int ids[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    // local best among live values
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = gl + i * G;
      if (live[i] && better(v[i], e, bv, be)) { bv = v[i]; be = e; }
    }
    for (int m = 1; m < G; m <<= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oe = __shfl_xor(be, m, 64);
      if (better(ov, oe, bv, be)) { bv = ov; be = oe; }
    }
    // the owner retires the chosen expert
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (gl + i * G == be) live[i] = false;
    if (j == 0) top = bv;
    z[j] = expf(bv - top);
    ids[j] = be;
    zsum += z[j];
  }
  float denom = zsum;
  if (!renorm) {
    // softmax over all E: sum exp(l - top) over every expert of the token
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = gl + i * G;
      if (tok_ok && e < E) s += expf(v[i] - top);
    }
    for (int m = 1; m < G; m <<= 1) s += __shfl_xor(s, m, 64);
    denom = s;
  }
  if (!tok_ok) return;
  const float inv = 1.0f / denom;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    if ((j % G) == gl) {
      idx_out[static_cast<int64_t>(t) * k + j] = ids[j];
      w_out[static_cast<int64_t>(t) * k + j] = z[j] * inv;
    }
  }
}

}  // namespace

hipError_t launch_router_logits(const bf16_t* x, const bf16_t* w_g,
                                const float* bias, int64_t T, int64_t d, int E,
                                float* logits, hipStream_t s) {
  dim3 grid(static_cast<unsigned>((T + 31) / 32),
            static_cast<unsigned>((E + 31) / 32));
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(kLogitThreads), 0, s, x,
                     w_g, bias, static_cast<int>(T), static_cast<int>(d), E,
                     logits);
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, int64_t T, int E, int k,
                        int renorm, int32_t* idx, float* w, hipStream_t s) {
  int G = 1;
  while (G < E && G < 64) G <<= 1;
  const int vpl_needed = (E + G - 1) / G;
  const int tokens_per_block = 256 / G;
  const unsigned grid =
      static_cast<unsigned>((T + tokens_per_block - 1) / tokens_per_block);
  const int Ti = static_cast<int>(T);
#define MOE_ROUTE_CASE(V)                                                     \
  if (vpl_needed <= V) {                                                      \
    hipLaunchKernelGGL(route_kernel<V>, dim3(grid), dim3(256), 0, s, logits,  \
                       Ti, E, k, renorm, G, idx, w);                          \
    return hipGetLastError();                                                 \
  }
  MOE_ROUTE_CASE(1)
  MOE_ROUTE_CASE(2)
  MOE_ROUTE_CASE(4)
  MOE_ROUTE_CASE(8)
  MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
