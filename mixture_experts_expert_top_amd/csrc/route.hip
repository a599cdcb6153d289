// Router scores and top-k routing on gfx950.
//
// "How MoE Architecture Cuts Costs and Boosts Efficiency", section "Why
// Biology Is Especially Well-Suited for MoE": the router gives every expert
// a score and only the K best-scoring experts run for a token.
// "Efficient MoE Training for Biological Foundation Models", Challenge 1:
// the chosen experts' outputs are scaled by routing weights.

#include <math.h>

#include <algorithm>

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

// ---------------------------------------------------------------- backward
// dlogits of one token (G lanes, as in route_kernel): the routing-weight
// gradient of the chosen experts (renormalised: p_j (dp_j - s), s =
// sum_j p_j dp_j; full softmax: P_e (g_e - s)) plus, with counts, the
// balancing term's alpha E / T * P_e (f_e - sum_e' f_e' P_e').  Each token's
// sum_e f_e P_e is kept per block (fixed order) for the loss value.
template <int VPL>
__global__ __launch_bounds__(256) void router_dlogits_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ p, const float* __restrict__ dp,
    const int32_t* __restrict__ counts, float alpha, int T, int E, int k,
    int renorm, int G, float* __restrict__ dlogits,
    float* __restrict__ q_part) {
  __shared__ float s_q[256];
  const int lane = threadIdx.x & 63;
  const int gwave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int tpw = 64 / G;
  const int sub = lane / G, gl = lane % G;
  const int t = gwave * tpw + sub;
  const bool tok_ok = t < T;
  const int64_t tk = static_cast<int64_t>(tok_ok ? t : 0) * k;
  float s = 0.0f;
  for (int j = 0; j < k; ++j) s += tok_ok ? p[tk + j] * dp[tk + j] : 0.0f;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = gl + i * G;
    v[i] = (tok_ok && e < E) ? logits[static_cast<int64_t>(t) * E + e]
                             : -INFINITY;
  }
  const bool need_p = !renorm || counts != nullptr;
  float P[VPL];
  float qf = 0.0f;
  if (need_p) {
    float top = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPL; ++i) top = fmaxf(top, v[i]);
    for (int m = 1; m < G; m <<= 1) top = fmaxf(top, __shfl_xor(top, m, 64));
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      P[i] = (gl + i * G < E && tok_ok) ? expf(v[i] - top) : 0.0f;
      z += P[i];
    }
    for (int m = 1; m < G; m <<= 1) z += __shfl_xor(z, m, 64);
    const float inv = tok_ok ? 1.0f / z : 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) P[i] *= inv;
    if (counts) {
      const float rtk = 1.0f / (static_cast<float>(T) * k);
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = gl + i * G;
        if (e < E) qf += counts[e] * rtk * P[i];
      }
      for (int m = 1; m < G; m <<= 1) qf += __shfl_xor(qf, m, 64);
    }
  }
  const float aux_scale = alpha * static_cast<float>(E) / static_cast<float>(T);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = gl + i * G;
    if (!tok_ok || e >= E) continue;
    float g = 0.0f, pj = 0.0f;
    bool chosen = false;
    for (int j = 0; j < k; ++j) {
      if (idx[tk + j] == e) { g = dp[tk + j]; pj = p[tk + j]; chosen = true; }
    }
    float r;
    if (renorm) r = chosen ? pj * (g - s) : 0.0f;
    else r = P[i] * (g - s);
    if (counts) {
      const float fe = counts[e] / (static_cast<float>(T) * k);
      r += aux_scale * P[i] * (fe - qf);
    }
    dlogits[static_cast<int64_t>(t) * E + e] = r;
  }
  // the block's tokens' sum_e f_e P_e, added in token order
  const int tb = threadIdx.x / G;             // token slot in the block
  if (gl == 0) s_q[tb] = tok_ok ? qf : 0.0f;
  __syncthreads();
  if (threadIdx.x == 0) {
    float acc = 0.0f;
    for (int i = 0; i < 256 / G; ++i) acc += s_q[i];
    q_part[blockIdx.x] = acc;
  }
}

// Partial dW_g over one chunk of 256 tokens, 512 columns and up to kExp
// experts (8 when E <= 8, else 32 a block): part[chunk][e][c] = sum over
// the chunk's tokens, in order, of dlogits[t][e] * x[t][c]; the y == 0
// blocks also sum dlogits over the chunk (db).  With part == nullptr only
// the db sums are made (x unread).  The x values of kAhead tokens are
// loaded before any of them is used, so the loads overlap; the sums still
// take the tokens one by one in order.
constexpr int kRbTok = 256;
constexpr int kRbExp = 32;
constexpr int kRbCols = 512;          // columns of a block, two a thread
template <int kExp>
__global__ __launch_bounds__(256) void router_dwg_partial_kernel(
    const float* __restrict__ dlogits, const bf16_t* __restrict__ x, int T,
    int E, int d, float* __restrict__ part, float* __restrict__ db_part) {
  constexpr int kRbExp = kExp;
  __shared__ __attribute__((aligned(16))) float s_dl[kRbTok][kRbExp];
  const int tc = blockIdx.x;
  const int c = blockIdx.y * kRbCols + threadIdx.x * 2;
  const int e0 = blockIdx.z * kRbExp;
  const int t0 = tc * kRbTok;
  const int ne = min(kRbExp, E - e0), nt = min(kRbTok, T - t0);
  for (int i = threadIdx.x; i < kRbTok * kRbExp; i += 256) {
    const int tt = i / kRbExp, ee = i % kRbExp;
    s_dl[tt][ee] = (tt < nt && ee < ne)
        ? dlogits[static_cast<int64_t>(t0 + tt) * E + e0 + ee] : 0.0f;
  }
  __syncthreads();
  if (blockIdx.y == 0 && threadIdx.x < ne) {
    float acc = 0.0f;
    for (int tt = 0; tt < nt; ++tt) acc += s_dl[tt][threadIdx.x];
    db_part[static_cast<int64_t>(tc) * E + e0 + threadIdx.x] = acc;
  }
  if (part == nullptr || c >= d) return;
  // columns c and c+1 (d is a multiple of 8), tokens added in order
  float acc0[kRbExp], acc1[kRbExp];
#pragma unroll
  for (int ee = 0; ee < kRbExp; ++ee) { acc0[ee] = 0.0f; acc1[ee] = 0.0f; }
  const bf16_t* xc = x + static_cast<int64_t>(t0) * d + c;
  constexpr int kAhead = 8;
  for (int tb = 0; tb < nt; tb += kAhead) {
    uint32_t xv[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u)
      xv[u] = (tb + u < nt) ? *reinterpret_cast<const uint32_t*>(
                                  xc + static_cast<int64_t>(tb + u) * d)
                            : 0u;
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      if (tb + u >= nt) break;
      const int tt = tb + u;
      const float x0 = bf_lo(xv[u]), x1 = bf_hi(xv[u]);
#pragma unroll
      for (int q = 0; q < kRbExp / 4; ++q) {
        const f32x4 g = *reinterpret_cast<const f32x4*>(&s_dl[tt][4 * q]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc0[4 * q + r] += g[r] * x0;
          acc1[4 * q + r] += g[r] * x1;
        }
      }
    }
  }
  for (int ee = 0; ee < ne; ++ee) {
    float2 o;
    o.x = acc0[ee];
    o.y = acc1[ee];
    *reinterpret_cast<float2*>(part + (static_cast<int64_t>(tc) * E + e0 + ee) * d + c) = o;
  }
}

// dW_g[e][c] = sum over chunks, in order, of part[chunk][e][c]; db likewise.
__global__ __launch_bounds__(256) void router_dwg_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ db_part,
    int chunks, int E, int d, float* __restrict__ dw, float* __restrict__ db) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(E) * d;
  if (dw && i < n) {
    float acc = 0.0f;
    for (int tc = 0; tc < chunks; ++tc) acc += part[tc * n + i];
    dw[i] = acc;
  }
  if (db && i < E) {
    float acc = 0.0f;
    for (int tc = 0; tc < chunks; ++tc) acc += db_part[static_cast<int64_t>(tc) * E + i];
    db[i] = acc;
  }
}

// dx_out[t] = bf16(dx_in[t] + sum_e dlogits[t][e] w_g[e]), experts added
// in order: a block owns kDxTok tokens and 2048 columns, a thread 8
// columns of each of the tokens, so every w_g chunk it loads serves
// kDxTok tokens.
constexpr int kDxTok = 8;
__global__ __launch_bounds__(256) void router_dx_kernel(
    const float* __restrict__ dlogits, const bf16_t* __restrict__ wg,
    const float* __restrict__ dx_in, int T, int E, int d,
    bf16_t* __restrict__ dx_out) {
  __shared__ __attribute__((aligned(16))) float s_dl[kMaxExperts * kDxTok];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kDxTok;
  const int nt = min(kDxTok, static_cast<int>(T - t0));
  // s_dl[e][tt]: the block's dlogits, expert-major
  for (int i = threadIdx.x; i < kDxTok * E; i += 256) {
    const int tt = i / E, e = i - (i / E) * E;
    s_dl[e * kDxTok + tt] = tt < nt ? dlogits[(t0 + tt) * E + e] : 0.0f;
  }
  __syncthreads();
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= d) return;
  float acc[kDxTok][8];
#pragma unroll
  for (int tt = 0; tt < kDxTok; ++tt) {
    if (dx_in && tt < nt) {
      const float* src = dx_in + (t0 + tt) * d + c;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
      acc[tt][0] = a[0]; acc[tt][1] = a[1]; acc[tt][2] = a[2]; acc[tt][3] = a[3];
      acc[tt][4] = b[0]; acc[tt][5] = b[1]; acc[tt][6] = b[2]; acc[tt][7] = b[3];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[tt][i] = 0.0f;
    }
  }
  for (int e = 0; e < E; ++e) {
    const i32x4 w =
        *reinterpret_cast<const i32x4*>(wg + static_cast<int64_t>(e) * d + c);
    float wv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wv[2 * q] = bf_lo(static_cast<uint32_t>(w[q]));
      wv[2 * q + 1] = bf_hi(static_cast<uint32_t>(w[q]));
    }
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(s_dl + e * kDxTok);
    const f32x4 g1 = *reinterpret_cast<const f32x4*>(s_dl + e * kDxTok + 4);
    const float g[kDxTok] = {g0[0], g0[1], g0[2], g0[3],
                             g1[0], g1[1], g1[2], g1[3]};
#pragma unroll
    for (int tt = 0; tt < kDxTok; ++tt)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[tt][i] += g[tt] * wv[i];
  }
#pragma unroll
  for (int tt = 0; tt < kDxTok; ++tt) {
    if (tt < nt) {
      uint4 o;
      o.x = pack_bf16x2(acc[tt][0], acc[tt][1]);
      o.y = pack_bf16x2(acc[tt][2], acc[tt][3]);
      o.z = pack_bf16x2(acc[tt][4], acc[tt][5]);
      o.w = pack_bf16x2(acc[tt][6], acc[tt][7]);
      *reinterpret_cast<uint4*>(dx_out + (t0 + tt) * d + c) = o;
    }
  }
}

// aux_loss = alpha * E / T * sum of q_part: thread j adds blocks j, j+256,
// ... in order, then the 256 partial sums are added pairwise in a fixed
// tree (deterministic).
__global__ __launch_bounds__(256) void router_aux_final_kernel(
    const float* __restrict__ q_part, int blocks, float scale,
    float* __restrict__ loss) {
  __shared__ float s_sum[256];
  float acc = 0.0f;
  for (int b = threadIdx.x; b < blocks; b += 256) acc += q_part[b];
  s_sum[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w)
      s_sum[threadIdx.x] += s_sum[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = scale * s_sum[0];
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

size_t router_backward_workspace(int64_t T, int E, int64_t d) {
  const int64_t chunks = (T + kRbTok - 1) / kRbTok;
  const size_t a = static_cast<size_t>(chunks * E * d * 4);
  const size_t b = static_cast<size_t>(chunks * E * 4);
  const size_t c = static_cast<size_t>(T * 4);
  auto up = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  return up(a) + up(b) + up(c);
}

hipError_t launch_router_backward(const float* logits, const int32_t* idx,
                                  const float* p, const float* dp,
                                  const int32_t* counts, float alpha,
                                  int64_t T, int E, int k, int renorm,
                                  const bf16_t* x, const bf16_t* w_g,
                                  int64_t d, float* dlogits, float* dw_g,
                                  float* db, const float* dx_in,
                                  bf16_t* dx_out, float* aux_loss, void* ws,
                                  hipStream_t s) {
  const int64_t chunks = (T + kRbTok - 1) / kRbTok;
  auto up = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* part = reinterpret_cast<float*>(w);
  w += up(static_cast<size_t>(chunks * E * d * 4));
  float* db_part = reinterpret_cast<float*>(w);
  w += up(static_cast<size_t>(chunks * E * 4));
  float* q_part = reinterpret_cast<float*>(w);
  int G = 1;
  while (G < E && G < 64) G <<= 1;
  const int vpl_needed = (E + G - 1) / G;
  const int tokens_per_block = 256 / G;
  const unsigned grid =
      static_cast<unsigned>((T + tokens_per_block - 1) / tokens_per_block);
  const int Ti = static_cast<int>(T);
  hipError_t err = hipErrorInvalidValue;
#define MOE_RB_CASE(V)                                                        \
  if (err == hipErrorInvalidValue && vpl_needed <= V) {                       \
    hipLaunchKernelGGL(router_dlogits_kernel<V>, dim3(grid), dim3(256), 0, s, \
                       logits, idx, p, dp, counts, alpha, Ti, E, k, renorm,   \
                       G, dlogits, q_part);                                   \
    err = hipGetLastError();                                                  \
  }
  MOE_RB_CASE(1)
  MOE_RB_CASE(2)
  MOE_RB_CASE(4)
  MOE_RB_CASE(8)
  MOE_RB_CASE(16)
#undef MOE_RB_CASE
  if (err != hipSuccess) return err;
  if (dw_g || db) {
    // without dw_g only the db sums are wanted: one column block, x unread
    const int64_t dd = dw_g ? d : 0;
    // experts a block: 8 when they all fit, else 32 (grid.z covers E)
    const int eb = E <= 8 ? 8 : kRbExp;
    dim3 g2(static_cast<unsigned>(chunks),
            static_cast<unsigned>(dw_g ? (d + kRbCols - 1) / kRbCols : 1),
            static_cast<unsigned>((E + eb - 1) / eb));
    if (eb == 8)
      hipLaunchKernelGGL(router_dwg_partial_kernel<8>, g2, dim3(256), 0, s,
                         dlogits, x, Ti, E, static_cast<int>(dd),
                         dw_g ? part : nullptr, db_part);
    else
      hipLaunchKernelGGL(router_dwg_partial_kernel<kRbExp>, g2, dim3(256), 0,
                         s, dlogits, x, Ti, E, static_cast<int>(dd),
                         dw_g ? part : nullptr, db_part);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t n = std::max<int64_t>(static_cast<int64_t>(E) * dd, E);
    hipLaunchKernelGGL(router_dwg_reduce_kernel,
                       dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                       0, s, part, db_part, static_cast<int>(chunks), E,
                       static_cast<int>(dd), dw_g, db);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (dx_out) {
    dim3 g4(static_cast<unsigned>((T + kDxTok - 1) / kDxTok),
            static_cast<unsigned>((d + 2047) / 2048));
    hipLaunchKernelGGL(router_dx_kernel, g4, dim3(256), 0, s, dlogits, w_g,
                       dx_in, Ti, E, static_cast<int>(d), dx_out);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (aux_loss && counts) {
    hipLaunchKernelGGL(router_aux_final_kernel, dim3(1), dim3(256), 0, s,
                       q_part, static_cast<int>(grid),
                       alpha * static_cast<float>(E) / static_cast<float>(T),
                       aux_loss);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moe
