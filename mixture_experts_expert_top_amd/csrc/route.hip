// Router scores and top-k routing on gfx950.
//
// "How MoE Architecture Cuts Costs and Boosts Efficiency", section "Why
// Biology Is Especially Well-Suited for MoE": the router gives every expert
// a score and only the K best-scoring experts run for a token.
// "Efficient MoE Training for Biological Foundation Models", Challenge 1:
// the chosen experts' outputs are scaled by routing weights.

#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.cuh"
#include "internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- logits
// logits[t][e] = x[t] . w_g[e] (+ bias[e]); a skinny GEMM (N = E) on bf16
// MFMA 32x32x16, bound by the one read of x.  A workgroup owns 32 tokens x
// 64 experts (two 32-expert blocks; one when the experts end sooner), so
// x is read once for E <= 64; its 8 waves split d into 8 contiguous ranges
// and their partial tiles are summed in LDS in wave order (fixed,
// deterministic).  Each wave issues the loads of AH k-steps before their
// MFMAs so that enough of x is in flight to keep HBM busy: 16 when E <= 32
// (one expert block, so the registers of the second serve the loads), else
// 8.  The workgroups are one per CU at these token counts, so the loads
// in flight are what sets the rate.
constexpr int kLogitThreads = 512;
constexpr int kLogitWaves = kLogitThreads / 64;
constexpr int kLogitExp = 64;

template <int AH, bool TWO>
__global__ __launch_bounds__(kLogitThreads) void router_logits_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
    const float* __restrict__ bias, int T, int d, int E,
    float* __restrict__ logits) {
  __shared__ float part[kLogitWaves][2][32 * 32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * kLogitExp;
  const int row = lane & 31, kh = lane >> 5;
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(x, static_cast<uint32_t>(static_cast<int64_t>(T) * d * 2));
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(wg, static_cast<uint32_t>(static_cast<int64_t>(E) * d * 2));
  const int tok = t0 + row;
  const bool tok_ok = tok < T;
  const bool two = TWO && e0 + 32 < E;    // uniform: second expert block
  const bool ex_ok0 = e0 + row < E, ex_ok1 = e0 + 32 + row < E;
  // the range of the reduction owned by this wave, in steps of 16
  const int steps = (d + 15) / 16;
  const int q = (steps + kLogitWaves - 1) / kLogitWaves;
  const int s_begin = wave * q, s_end = min(steps, s_begin + q);
  const int64_t xrow = static_cast<int64_t>(tok) * d;
  const int64_t wrow0 = static_cast<int64_t>(e0 + row) * d;
  const int64_t wrow1 = wrow0 + static_cast<int64_t>(32) * d;
  f32x16 acc0 = {}, acc1 = {};
  for (int s0 = s_begin; s0 < s_end; s0 += AH) {
    bf16x8_v a[AH], b0[AH], b1[TWO ? AH : 1];
#pragma unroll
    for (int u = 0; u < AH; ++u) {
      // steps past the wave's range (or d) read zeros through kOob
      const int kk = (s0 + u) * 16 + kh * 8;
      const bool kok = s0 + u < s_end && kk < d;
      const uint32_t ox = (tok_ok && kok)
          ? static_cast<uint32_t>((xrow + kk) * 2) : kOob;
      const uint32_t ow0 = (ex_ok0 && kok)
          ? static_cast<uint32_t>((wrow0 + kk) * 2) : kOob;
      a[u] = __builtin_bit_cast(bf16x8_v, buf_load16(rx, ox));
      b0[u] = __builtin_bit_cast(bf16x8_v, buf_load16(rw, ow0));
      if (two) {
        const uint32_t ow1 = (ex_ok1 && kok)
            ? static_cast<uint32_t>((wrow1 + kk) * 2) : kOob;
        b1[TWO ? u : 0] = __builtin_bit_cast(bf16x8_v, buf_load16(rw, ow1));
      }
    }
    // every load of the group is issued before the first MFMA waits
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < AH; ++u) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b0[u], acc0, 0, 0, 0);
      if (two)
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b1[TWO ? u : 0],
                                                       acc1, 0, 0, 0);
    }
  }
  // acc[v] = C[token i][expert j], i = (v/4)*8 + kh*4 + v%4, j = lane%32
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int i = (v >> 2) * 8 + kh * 4 + (v & 3);
    part[wave][0][i * 32 + row] = acc0[v];
    part[wave][1][i * 32 + row] = acc1[v];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 2 * 32 * 32; idx += kLogitThreads) {
    const int h = idx >> 10, i = (idx >> 5) & 31, j = idx & 31;
    const int t = t0 + i, e = e0 + 32 * h + j;
    if (t < T && e < E) {
      float s = part[0][h][idx & 1023];
#pragma unroll
      for (int w = 1; w < kLogitWaves; ++w) s += part[w][h][idx & 1023];
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
// A NaN score ranks below every number (NaNs among themselves by id), so
// every round picks a real expert whatever the scores hold; kNoExpert marks
// a lane with nothing left and loses to any expert.
constexpr int kNoExpert = 0x7fffffff;
__device__ __forceinline__ bool better(float va, int ea, float vb, int eb) {
  if (ea == kNoExpert) return false;
  if (eb == kNoExpert) return true;
  const bool na = va != va, nb = vb != vb;
  if (na || nb) return na && nb ? ea < eb : nb;
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
    int be = kNoExpert;
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

// Partial dW_g over one chunk of kRbTok tokens on bf16 MFMA:
// part[chunk][e][c] = the sum over the chunk's tokens of
// dlogits[t][e] * x[t][c].  Each fp32 dlogits value is split into three
// bf16 terms whose sum is the value exactly (the top 8 significant bits
// rounded to nearest, then the next 8 of the remainder, then the last
// 8), so every product with the bf16 x is exact in fp32 and the MFMA sums
// them in fp32: the accuracy of an fp32 sum of the chunk's 3 * kRbTok
// products, at matrix-core rate.  A block owns kDwCols columns, kDwExp
// experts and the chunk; it stages kDwStep tokens at a time (x as a
// [token][column] tile read transposed by frag_tr, dlogits as [expert]
// [token]), and wave w keeps the 64 columns 64w.. x the 64 experts in four
// 32 x 32 accumulators.  The y == 0 blocks also sum dlogits over the chunk
// in token order (db).  With part == nullptr only the db sums are made (x
// unread).
constexpr int kRbTok = 256;
constexpr int kDwCols = 256;
constexpr int kDwExp = 64;
constexpr int kDwStep = 64;
typedef float f32x8_v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split_bf16x3(f32x8_v v, bf16x8_v* hi,
                                             bf16x8_v* mid, bf16x8_v* lo) {
  *hi = __builtin_convertvector(v, bf16x8_v);
  const f32x8_v r1 = v - __builtin_convertvector(*hi, f32x8_v);
  *mid = __builtin_convertvector(r1, bf16x8_v);
  const f32x8_v r2 = r1 - __builtin_convertvector(*mid, f32x8_v);
  *lo = __builtin_convertvector(r2, bf16x8_v);
}

__global__ __launch_bounds__(256) void router_dwg_partial_kernel(
    const float* __restrict__ dlogits, const bf16_t* __restrict__ x, int T,
    int E, int d, float* __restrict__ part, float* __restrict__ db_part) {
  __shared__ __attribute__((aligned(16))) bf16_t s_x[kDwStep * kDwCols];
  // [expert][token], rows padded to 68 floats (16-byte aligned, and the
  // transposing stores spread over the banks)
  __shared__ __attribute__((aligned(16))) float s_dl[kDwExp][kDwStep + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tc = blockIdx.x;
  const int c0 = blockIdx.y * kDwCols, e0 = blockIdx.z * kDwExp;
  const int t0 = tc * kRbTok;
  const int nt = min(kRbTok, T - t0), ne = min(kDwExp, E - e0);
  const bool want_x = part != nullptr;
  const bool do_db = blockIdx.y == 0 && tid < ne;
  const KmnLane kl(lane);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  float db = 0.0f;
  // thread t moves the 16-byte column chunk t % 32 of token rows
  // 8 (t / 32) + i of a step, and experts 16 (t % 4) + 0..15 of token t / 4;
  // a step's values are loaded into registers during the step before
  const int cc = tid & 31, kr0 = (tid >> 5) * 8;
  const int col = c0 + cc * 8;
  const int tt4 = tid >> 2, eb = (tid & 3) * 16;
  i32x4 v[8];
  float g[16];
  auto load_step = [&](int s0) {
    if (want_x) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = s0 + kr0 + i;
        v[i] = (row < nt && col < d)
            ? *reinterpret_cast<const i32x4*>(
                  x + static_cast<int64_t>(t0 + row) * d + col)
            : i32x4{};
      }
    }
    const bool tok = s0 + tt4 < nt;
    const float* src = dlogits + static_cast<int64_t>(t0 + s0 + tt4) * E + e0;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      g[q] = (tok && eb + q < ne) ? src[eb + q] : 0.0f;
  };
  load_step(0);
  for (int s0 = 0; s0 < nt; s0 += kDwStep) {
    if (want_x) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<i32x4*>(reinterpret_cast<uint8_t*>(s_x) +
                                  kmn_off(kr0 + i, cc)) = v[i];
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) s_dl[eb + q][tt4] = g[q];
    __syncthreads();
    if (s0 + kDwStep < nt) load_step(s0 + kDwStep);
    // the next step's loads stay ahead of this step's MFMAs
    __builtin_amdgcn_sched_barrier(0);
    if (do_db)
      for (int tt = 0; tt < kDwStep; ++tt) db += s_dl[tid][tt];
    if (want_x) {
#pragma unroll
      for (int kk = 0; kk < kDwStep / 16; ++kk) {
        bf16x8_v a[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          a[i] = frag_tr(s_x, kl.base, kl.R, wave * 2 + i, kk);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (32 * j >= ne) break;              // no expert in this block
          const float* p = &s_dl[32 * j + (lane & 31)][16 * kk + 8 * (lane >> 5)];
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(p);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(p + 4);
          const f32x8_v g = {g0[0], g0[1], g0[2], g0[3],
                             g1[0], g1[1], g1[2], g1[3]};
          bf16x8_v hi, mid, lo;
          split_bf16x3(g, &hi, &mid, &lo);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a[i], hi, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a[i], mid, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a[i], lo, acc[i][j], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }
  if (do_db) db_part[static_cast<int64_t>(tc) * E + e0 + tid] = db;
  if (!want_x) return;
  // acc[i][j][v] = column c0 + 64 wave + 32 i + 8 (v / 4) + 4 (lane / 32)
  // + v % 4 (rows of the MFMA) for expert e0 + 32 j + lane % 32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = 32 * j + (lane & 31);
    if (e >= ne) continue;
    float* dst = part + (static_cast<int64_t>(tc) * E + e0 + e) * d;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + wave * 64 + 32 * i + 8 * q + 4 * (lane >> 5);
        if (c < d) {
          const f32x4 o = {acc[i][j][4 * q], acc[i][j][4 * q + 1],
                           acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          *reinterpret_cast<f32x4*>(dst + c) = o;
        }
      }
  }
}

// dW_g[e][c] = sum over chunks, in order, of part[chunk][e][c]; db likewise.
__global__ __launch_bounds__(256) void router_dwg_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ db_part,
    int chunks, int E, int d, float* __restrict__ dw, float* __restrict__ db) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(E) * d;
  if (dw && i < n) {
    // kAhead chunks' loads in flight at a time, added in chunk order
    constexpr int kAhead = 8;
    float acc = 0.0f;
    for (int tb = 0; tb < chunks; tb += kAhead) {
      float v[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u)
        v[u] = tb + u < chunks ? part[(tb + u) * n + i] : 0.0f;
#pragma unroll
      for (int u = 0; u < kAhead; ++u)
        if (tb + u < chunks) acc += v[u];
    }
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
  // the w_g rows of kDxAhead experts are loaded before any is used
  constexpr int kDxAhead = 4;
  for (int eb = 0; eb < E; eb += kDxAhead) {
    i32x4 wr[kDxAhead];
#pragma unroll
    for (int u = 0; u < kDxAhead; ++u)
      wr[u] = eb + u < E ? *reinterpret_cast<const i32x4*>(
                               wg + static_cast<int64_t>(eb + u) * d + c)
                         : i32x4{};
#pragma unroll
    for (int u = 0; u < kDxAhead; ++u) {
      if (eb + u >= E) break;
      const int e = eb + u;
      float wv[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wv[2 * q] = bf_lo(static_cast<uint32_t>(wr[u][q]));
        wv[2 * q + 1] = bf_hi(static_cast<uint32_t>(wr[u][q]));
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
            static_cast<unsigned>((E + kLogitExp - 1) / kLogitExp));
  if (E <= 32)
    hipLaunchKernelGGL((router_logits_kernel<16, false>), grid,
                       dim3(kLogitThreads), 0, s, x, w_g, bias,
                       static_cast<int>(T), static_cast<int>(d), E, logits);
  else
    hipLaunchKernelGGL((router_logits_kernel<8, true>), grid,
                       dim3(kLogitThreads), 0, s, x, w_g, bias,
                       static_cast<int>(T), static_cast<int>(d), E, logits);
  return hipGetLastError();
}

// Lanes that share one token in the routing kernels: the smallest power of
// two that leaves each lane at most 8 experts (at most 64 lanes; 16 experts
// a lane at E = 1024) -- a lane's own experts are compared in registers and
// only log2(G) shuffle steps a round cross lanes -- but more, up to one
// expert a lane, while the grid (256 / G tokens a block) would leave
// compute units idle.
int route_lanes(int E, int64_t T) {
  int G = 1;
  while (G * 8 < E && G < 64) G <<= 1;
  while (G < 64 && G < E && T * G < 256 * 256) G <<= 1;
  return G;
}

hipError_t launch_route(const float* logits, int64_t T, int E, int k,
                        int renorm, int32_t* idx, float* w, hipStream_t s) {
  const int G = route_lanes(E, T);
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
  const int G = route_lanes(E, T);
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
    dim3 g2(static_cast<unsigned>(chunks),
            static_cast<unsigned>(dw_g ? (d + kDwCols - 1) / kDwCols : 1),
            static_cast<unsigned>((E + kDwExp - 1) / kDwExp));
    hipLaunchKernelGGL(router_dwg_partial_kernel, g2, dim3(256), 0, s,
                       dlogits, x, Ti, E, static_cast<int>(dd),
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
