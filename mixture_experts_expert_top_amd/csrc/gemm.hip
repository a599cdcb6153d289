// Grouped GEMM over expert segments on gfx950 bf16 MFMA.
//
// One submission covers every expert ("Efficient MoE Training for
// Biological Foundation Models", Challenge 1: GroupedLinear submits all
// local experts' work together, driven by per-expert token counts).  The
// per-expert row offsets stay on the device; each workgroup decodes its
// (expert, m-tile, n-tile) from them, so no host synchronisation is needed.
//
// Two grouping modes:
//   SegM: rows of the product are an expert's permuted rows (forward and
//         dgrad): M_e = counts[e], K fixed, B = that expert's weight.
//   SegK: the reduction runs over an expert's permuted rows (wgrad):
//         K_e = counts[e], M and N fixed, C = that expert's weight grad.
// Operands are either K-contiguous (row-major [M][K]) or MN-contiguous
// (row-major [K][M]); MN-contiguous tiles are transposed in registers on
// the way into LDS so every LDS tile is K-contiguous and one MFMA inner
// loop serves all six GEMMs of the layer.
//
// Epilogues (Challenge 3 of the same page: gate_up -> ScaledSwiGLU -> down
// with the routing probabilities as the SwiGLU scales, plus a matching
// fused backward):
//   kStore   : C = bf16(acc)
//   kStoreF32: C = acc (fp32; rows later summed by the combine)
//   kSwiglu  : dual-B tile (gate and up columns of the same index in one
//              workgroup); stores AB (bf16) and S = w * silu(gate) * up
//   kDSwiglu : acc = dS; reads AB and w, writes dAB = (dA_g, dA_u) and
//              per-tile partial sums of dS * H for the routing-weight grad
//
// Tile: 256 x 256 x 64, 256 threads = 4 waves in 2 x 2, each wave a
// 128 x 128 sub-tile of 4 x 4 MFMA 32x32x16 blocks (256 fp32 accumulators
// per lane).  LDS: two stages of (256 + 256) x 64 bf16 = 128 KiB, rows of
// 128 B with a 16-byte-chunk XOR swizzle that keeps both the tile stores
// and the MFMA fragment reads free of bank conflicts.

#include "common.cuh"
#include "internal.h"

namespace moe {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kTileElems = BM * BK;       // one operand stage (A or B)
constexpr int kStageElems = 2 * kTileElems;
constexpr int kGroupN = 4;                // n-tiles per scheduling group
constexpr int kEpiLd = 132;               // fp32 row stride of the epilogue stage
constexpr int kSmemBytes = 4 * 64 * kEpiLd * 4;  // >= the two operand stages

enum Mode { kSegM = 0, kSegK = 1 };
enum Epi { kStore = 0, kSwiglu = 1, kDSwiglu = 2, kStoreF32 = 3 };

struct Params {
  const bf16_t* A;
  int64_t lda;
  const bf16_t* B;
  int64_t ldb;
  int64_t b_stride;  // elements between experts' B
  bf16_t* C;         // bf16 output (kStore, kSwiglu, kDSwiglu)
  float* Cf;         // fp32 output (kStoreF32)
  int64_t ldc;
  int64_t c_stride;  // SegK: elements between experts' C
  const int32_t* offsets;
  int E;
  int64_t Tk;
  int M;             // SegK: rows of C
  int N;             // columns of C (kSwiglu: f, the gate width)
  int K;             // SegM: reduction length
  int ntn;           // n-tiles
  int b_rows;        // rows of one expert's B as stored (SegM)
  // epilogue operands
  const float* w;    // per permuted row weight (kSwiglu, kDSwiglu), or null
  bf16_t* S;         // kSwiglu: S [Tk][f]
  const bf16_t* AB;  // kDSwiglu: saved [Tk][2f]
  float* dp_part;    // kDSwiglu: [Tk][ntn]
  int f;
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Element offset of (row, chunk) inside one LDS operand tile.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * BK + ((chunk ^ swz(row)) << 3);
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo,
                                             uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Workgroup id -> logical tile id so that the blocks one XCD receives
// (hardware hands out ids round-robin over the 8 XCDs) form a contiguous
// range of tiles that share operands in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int q = nb >> 3, r = nb & 7;
  const int x = bid & 7, i = bid >> 3;
  return x * q + min(x, r) + i;
}

template <bool KC>
struct Loader;

// K-contiguous operand: 256 rows x 64 k; thread loads 8 chunks of 16 B at
// (row = tid/8 + 32*i, chunk = tid%8).
template <>
struct Loader<true> {
  i32x4 v[8];
  template <typename RowMap>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t ld,
                                       int k0, int kmax, RowMap rowmap,
                                       int tid) {
    const int chunk = tid & 7;
    const int kk = k0 + chunk * 8;
    const bool kok = kk < kmax;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 3) + 32 * i;
      const int64_t grow = rowmap(row);
      uint32_t off = kOob;
      if (kok && grow >= 0)
        off = static_cast<uint32_t>((grow * ld + kk) * 2);
      v[i] = buf_load16(rs, off);
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
    const int chunk = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (tid >> 3) + 32 * i;
      *reinterpret_cast<i32x4*>(lds + lds_off(row, chunk)) = v[i];
    }
  }
};

// MN-contiguous operand: 64 k-rows x 256 columns; thread loads an 8x8
// block (k = kr*8 .. +7, columns mc*8 .. +7), kr = tid/32, mc = tid%32, and
// transposes it so that each column's 8 k-values become one LDS chunk.
template <>
struct Loader<false> {
  i32x4 v[8];
  template <typename ColMap>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t ld,
                                       int k0, int kmax, ColMap colmap,
                                       int tid) {
    const int kr = tid >> 5, mc = tid & 31;
    const int64_t gcol = colmap(mc * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + kr * 8 + i;
      uint32_t off = kOob;
      if (k < kmax && gcol >= 0)
        off = static_cast<uint32_t>((static_cast<int64_t>(k) * ld + gcol) * 2);
      v[i] = buf_load16(rs, off);
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
    const int kr = tid >> 5, mc = tid & 31;
    // v[i] holds k = kr*8+i, columns mc*8+0..7 (dword q: columns 2q, 2q+1).
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int q = m >> 1;
      const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
      i32x4 o;
      o[0] = perm_b32(v[1][q], v[0][q], sel);
      o[1] = perm_b32(v[3][q], v[2][q], sel);
      o[2] = perm_b32(v[5][q], v[4][q], sel);
      o[3] = perm_b32(v[7][q], v[6][q], sel);
      *reinterpret_cast<i32x4*>(lds + lds_off(mc * 8 + m, kr)) = o;
    }
  }
};

__device__ __forceinline__ int find_segment(const int* pref, int E, int key) {
  // largest e in [0, E) with pref[e] <= key (pref non-decreasing)
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= key) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int MODE, bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(Params P) {
  static_assert(kSmemBytes >= 2 * kStageElems * 2, "stage fits");
  __shared__ __attribute__((aligned(16))) bf16_t smem[kSmemBytes / 2];
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ float s_dp[2 * BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int E = P.E;

  // ---------------------------------------------------------- tile decode
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int e, mt, nt;
  int64_t seg0;      // first permuted row of the expert
  int seg_len;       // rows of the expert
  if (MODE == kSegM) {
    // prefix of m-tiles per expert
    for (int i = tid; i <= E; i += kThreads) {
      int c = 0;
      if (i < E) c = (P.offsets[i + 1] - P.offsets[i] + BM - 1) / BM;
      s_pref[i] = c;
    }
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int i = 0; i <= E; ++i) {
        const int c = s_pref[i];
        s_pref[i] = run;
        run += c;
      }
    }
    __syncthreads();
    const int total = s_pref[E] * P.ntn;
    if (bid >= total) return;
    e = find_segment(s_pref, E, bid / P.ntn);
    // the expert's tiles: groups of kGroupN n-tiles, m fastest inside
    const int mte = s_pref[e + 1] - s_pref[e];
    const int local = bid - s_pref[e] * P.ntn;
    const int grp = local / (mte * kGroupN);
    const int within = local - grp * mte * kGroupN;
    mt = within % mte;
    nt = grp * kGroupN + within / mte;
    seg0 = P.offsets[e];
    seg_len = P.offsets[e + 1] - P.offsets[e];
  } else {
    const int mtiles = (P.M + BM - 1) / BM;
    const int per_e = mtiles * P.ntn;
    e = bid / per_e;
    const int local = bid - e * per_e;
    const int grp = local / (mtiles * kGroupN);
    const int within = local - grp * mtiles * kGroupN;
    mt = within % mtiles;
    nt = grp * kGroupN + within / mtiles;
    seg0 = P.offsets[e];
    seg_len = P.offsets[e + 1] - P.offsets[e];
  }
  const int m0 = mt * BM;
  const int n0 = nt * BN;               // kSwiglu: gate column tile = nt*BN/2
  const int Mvalid = (MODE == kSegM) ? seg_len : P.M;
  const int Kdim = (MODE == kSegM) ? P.K : seg_len;

  // ---------------------------------------------------------- operands
  __amdgpu_buffer_rsrc_t rsA, rsB;
  if (MODE == kSegM) {
    const bf16_t* a = P.A + seg0 * P.lda;
    const int64_t bytes = (P.Tk - seg0) * P.lda * 2;
    rsA = make_rsrc(a, static_cast<uint32_t>(bytes));
    const bf16_t* b = P.B + static_cast<int64_t>(e) * P.b_stride;
    rsB = make_rsrc(b, static_cast<uint32_t>(static_cast<int64_t>(P.b_rows) *
                                             P.ldb * 2));
  } else {
    const bf16_t* a = P.A + seg0 * P.lda;
    rsA = make_rsrc(a, static_cast<uint32_t>(seg_len * P.lda * 2));
    const bf16_t* b = P.B + seg0 * P.ldb;
    rsB = make_rsrc(b, static_cast<uint32_t>(seg_len * P.ldb * 2));
  }

  // row/column maps: tile-local index -> global row of the operand
  const int f = P.f;
  const int n0g = nt * (BN / 2);
  auto amap = [&](int r) -> int64_t { return m0 + r; };
  auto bmap = [&](int q) -> int64_t {
    if (EPI == kSwiglu) {
      const int w_n = q >> 7, jj = (q >> 5) & 3, c = q & 31;
      return static_cast<int64_t>((jj >> 1) * f + n0g + w_n * 64 +
                                  (jj & 1) * 32 + c);
    }
    return n0 + q;
  };

  Loader<AKC> la;
  Loader<BKC> lb;
  const int nk = (Kdim + BK - 1) / BK;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  if (nk > 0) {
    la.load(rsA, P.lda, 0, Kdim, amap, tid);
    lb.load(rsB, P.ldb, 0, Kdim, bmap, tid);
    la.store(smem, tid);
    lb.store(smem + kTileElems, tid);
    __syncthreads();
  }

  const int fr = lane & 31;      // fragment row inside a 32-block
  const int fk = lane >> 5;      // which 8-wide k half
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bf16_t* sa = smem + cur * kStageElems;
    const bf16_t* sb = sa + kTileElems;
    if (kt + 1 < nk) {
      la.load(rsA, P.lda, (kt + 1) * BK, Kdim, amap, tid);
      lb.load(rsB, P.ldb, (kt + 1) * BK, Kdim, bmap, tid);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int chunk = kk * 2 + fk;
      bf16x8_v af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + fr;
        af[i] = __builtin_bit_cast(
            bf16x8_v, *reinterpret_cast<const i32x4*>(sa + lds_off(r, chunk)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 128 + j * 32 + fr;
        bfr[j] = __builtin_bit_cast(
            bf16x8_v, *reinterpret_cast<const i32x4*>(sb + lds_off(r, chunk)));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],
                                                              acc[i][j], 0, 0,
                                                              0);
    }
    if (kt + 1 < nk) {
      bf16_t* nxt = smem + (cur ^ 1) * kStageElems;
      la.store(nxt, tid);
      lb.store(nxt + kTileElems, tid);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------- epilogue
  // acc[i][j][v] is C[row][col] of the wave's 128 x 128 sub-tile with
  //   row = i*32 + (v/4)*8 + (lane/32)*4 + v%4,  col = j*32 + lane%32.
  // Each half (64 rows) is staged through the wave's own LDS region as
  // fp32 [64][kEpiLd] and then processed row by row: a lane owns 4
  // consecutive columns, so global reads and bf16 stores are contiguous.
  float* stage = reinterpret_cast<float*>(smem) + wave * (64 * kEpiLd);
  const int64_t cbase = (MODE == kSegM) ? seg0 * P.ldc
                                        : static_cast<int64_t>(e) * P.c_stride;
  const float* w = ((EPI == kSwiglu || EPI == kDSwiglu) && P.w) ? P.w + seg0
                                                                : nullptr;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = ii * 32 + (v >> 2) * 8 + fk * 4 + (v & 3);
          stage[r * kEpiLd + j * 32 + fr] = acc[2 * h + ii][j][v];
        }
    __syncthreads();
    const int row_base = m0 + wm * 128 + h * 64;   // tile-relative + m0
    if (EPI == kStore) {
      // 32 lanes x 4 columns per row, 2 rows per pass
      const int c4 = (lane & 31) * 4;
      const int col = n0 + wn * 128 + c4;
      for (int r = lane >> 5; r < 64; r += 2) {
        const int row = row_base + r;
        if (row < Mvalid && col < P.N) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(stage + r * kEpiLd + c4);
          uint2 o;
          o.x = pack_bf16x2(x[0], x[1]);
          o.y = pack_bf16x2(x[2], x[3]);
          *reinterpret_cast<uint2*>(P.C + cbase + static_cast<int64_t>(row) * P.ldc + col) = o;
        }
      }
    } else if (EPI == kStoreF32) {
      const int c4 = (lane & 31) * 4;
      const int col = n0 + wn * 128 + c4;
      for (int r = lane >> 5; r < 64; r += 2) {
        const int row = row_base + r;
        if (row < Mvalid && col < P.N)
          *reinterpret_cast<f32x4*>(P.Cf + cbase + static_cast<int64_t>(row) * P.ldc + col) =
              *reinterpret_cast<const f32x4*>(stage + r * kEpiLd + c4);
      }
    } else if (EPI == kSwiglu) {
      // stage columns [0,64) are gate, [64,128) the matching up columns
      bf16_t* AB = P.C + cbase;                       // [rows][2f]
      bf16_t* S = P.S + seg0 * static_cast<int64_t>(f);
      const int c4 = (lane & 15) * 4;
      const int col = n0g + wn * 64 + c4;             // gate column
      for (int r = lane >> 4; r < 64; r += 4) {
        const int row = row_base + r;
        if (row < Mvalid && col < f) {
          const f32x4 g = *reinterpret_cast<const f32x4*>(stage + r * kEpiLd + c4);
          const f32x4 u = *reinterpret_cast<const f32x4*>(stage + r * kEpiLd + 64 + c4);
          const float wr = w ? w[row] : 1.0f;
          float sv[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) sv[c] = wr * (g[c] * sigmoidf_(g[c]) * u[c]);
          const int64_t ro = static_cast<int64_t>(row);
          uint2 og, ou, os;
          og.x = pack_bf16x2(g[0], g[1]); og.y = pack_bf16x2(g[2], g[3]);
          ou.x = pack_bf16x2(u[0], u[1]); ou.y = pack_bf16x2(u[2], u[3]);
          os.x = pack_bf16x2(sv[0], sv[1]); os.y = pack_bf16x2(sv[2], sv[3]);
          *reinterpret_cast<uint2*>(AB + ro * P.ldc + col) = og;
          *reinterpret_cast<uint2*>(AB + ro * P.ldc + f + col) = ou;
          *reinterpret_cast<uint2*>(S + ro * f + col) = os;
        }
      }
    } else {  // kDSwiglu
      const bf16_t* AB = P.AB + seg0 * static_cast<int64_t>(2 * f);
      bf16_t* dAB = P.C + cbase;
      const int c4 = (lane & 31) * 4;
      const int col = n0 + wn * 128 + c4;
      for (int r = lane >> 5; r < 64; r += 2) {
        const int row = row_base + r;
        float part = 0.0f;
        if (row < Mvalid && col < f) {
          const int64_t ro = static_cast<int64_t>(row);
          const f32x4 ds = *reinterpret_cast<const f32x4*>(stage + r * kEpiLd + c4);
          const uint2 gb = *reinterpret_cast<const uint2*>(AB + ro * 2 * f + col);
          const uint2 ub = *reinterpret_cast<const uint2*>(AB + ro * 2 * f + f + col);
          const float g[4] = {bf_lo(gb.x), bf_hi(gb.x), bf_lo(gb.y), bf_hi(gb.y)};
          const float u[4] = {bf_lo(ub.x), bf_hi(ub.x), bf_lo(ub.y), bf_hi(ub.y)};
          const float wr = w ? w[row] : 1.0f;
          float dg[4], du[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float sg = sigmoidf_(g[c]);
            const float sl = g[c] * sg;
            part += ds[c] * (sl * u[c]);
            const float dh = wr * ds[c];
            dg[c] = dh * u[c] * sg * (1.0f + g[c] * (1.0f - sg));
            du[c] = dh * sl;
          }
          uint2 og, ou;
          og.x = pack_bf16x2(dg[0], dg[1]); og.y = pack_bf16x2(dg[2], dg[3]);
          ou.x = pack_bf16x2(du[0], du[1]); ou.y = pack_bf16x2(du[2], du[3]);
          *reinterpret_cast<uint2*>(dAB + ro * P.ldc + col) = og;
          *reinterpret_cast<uint2*>(dAB + ro * P.ldc + f + col) = ou;
        }
        // row sum over the 32 lanes of this row, fixed butterfly order
        part += __shfl_xor(part, 1, 64);
        part += __shfl_xor(part, 2, 64);
        part += __shfl_xor(part, 4, 64);
        part += __shfl_xor(part, 8, 64);
        part += __shfl_xor(part, 16, 64);
        if ((lane & 31) == 0) s_dp[wn * BM + wm * 128 + h * 64 + r] = part;
      }
    }
    __syncthreads();
  }
  if (EPI == kDSwiglu) {
    // the tile's two column halves, added in order (wn = 0 then wn = 1)
    for (int lr = tid; lr < BM; lr += kThreads) {
      const int row = m0 + lr;
      if (row < Mvalid)
        P.dp_part[(seg0 + row) * P.ntn + nt] = s_dp[lr] + s_dp[BM + lr];
    }
  }
}

template <int MODE, bool AKC, bool BKC, int EPI>
hipError_t launch(const Params& P, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<MODE, AKC, BKC, EPI>), dim3(grid),
                     dim3(kThreads), 0, s, P);
  return hipGetLastError();
}

int segm_grid(int64_t Tk, int E, int ntn) {
  const int64_t mt = (Tk + BM - 1) / BM + E;
  return static_cast<int>(mt * ntn);
}

}  // namespace

int gemm_dp_tiles(int64_t f) { return static_cast<int>((f + BN - 1) / BN); }

// fc1 forward: AB = Xp . W_gu^T (dual gate/up tile), S = w*silu(g)*u
hipError_t gemm_fc1_fwd(const bf16_t* xp, const bf16_t* w_gu,
                        const int32_t* offsets, int E, int64_t Tk, int64_t d,
                        int64_t f, const float* w_perm, bf16_t* ab, bf16_t* s,
                        hipStream_t st) {
  Params P{};
  P.A = xp; P.lda = d;
  P.B = w_gu; P.ldb = d; P.b_stride = 2 * f * d; P.b_rows = 2 * f;
  P.C = ab; P.ldc = 2 * f;
  P.offsets = offsets; P.E = E; P.Tk = Tk;
  P.N = f; P.K = d; P.f = f;
  P.ntn = static_cast<int>((f + BN / 2 - 1) / (BN / 2));
  P.w = w_perm; P.S = s;
  return launch<kSegM, true, true, kSwiglu>(P, segm_grid(Tk, E, P.ntn), st);
}

// fc2 forward: O = S . W2^T (fp32 rows)
hipError_t gemm_fc2_fwd(const bf16_t* s, const bf16_t* w2,
                        const int32_t* offsets, int E, int64_t Tk, int64_t d,
                        int64_t f, float* o, hipStream_t st) {
  Params P{};
  P.A = s; P.lda = f;
  P.B = w2; P.ldb = f; P.b_stride = d * f; P.b_rows = d;
  P.Cf = o; P.ldc = d;
  P.offsets = offsets; P.E = E; P.Tk = Tk;
  P.N = d; P.K = f; P.f = f;
  P.ntn = static_cast<int>((d + BN - 1) / BN);
  return launch<kSegM, true, true, kStoreF32>(P, segm_grid(Tk, E, P.ntn), st);
}

// fc2 dgrad + dSwiGLU: dS = dO . W2 (W2 is [d][f]: MN-contiguous B)
hipError_t gemm_fc2_dgrad(const bf16_t* dO, const bf16_t* w2,
                          const int32_t* offsets, int E, int64_t Tk,
                          int64_t d, int64_t f, const bf16_t* ab,
                          const float* w_perm, bf16_t* dab, float* dp_part,
                          hipStream_t st) {
  Params P{};
  P.A = dO; P.lda = d;
  P.B = w2; P.ldb = f; P.b_stride = d * f; P.b_rows = d;
  P.C = dab; P.ldc = 2 * f;
  P.offsets = offsets; P.E = E; P.Tk = Tk;
  P.N = f; P.K = d; P.f = f;
  P.ntn = gemm_dp_tiles(f);
  P.AB = ab; P.w = w_perm; P.dp_part = dp_part;
  return launch<kSegM, true, false, kDSwiglu>(P, segm_grid(Tk, E, P.ntn), st);
}

// fc1 dgrad: dXp = dAB . W_gu (W_gu is [2f][d]: MN-contiguous B), fp32 rows
hipError_t gemm_fc1_dgrad(const bf16_t* dab, const bf16_t* w_gu,
                          const int32_t* offsets, int E, int64_t Tk,
                          int64_t d, int64_t f, float* dxp, hipStream_t st) {
  Params P{};
  P.A = dab; P.lda = 2 * f;
  P.B = w_gu; P.ldb = d; P.b_stride = 2 * f * d; P.b_rows = 2 * f;
  P.Cf = dxp; P.ldc = d;
  P.offsets = offsets; P.E = E; P.Tk = Tk;
  P.N = d; P.K = 2 * f; P.f = f;
  P.ntn = static_cast<int>((d + BN - 1) / BN);
  return launch<kSegM, true, false, kStoreF32>(P, segm_grid(Tk, E, P.ntn), st);
}

// wgrad: C[e] (M x N) = sum over the expert's rows r of A[r][m] * B[r][n]
hipError_t gemm_wgrad(const bf16_t* a, int64_t lda, const bf16_t* b,
                      int64_t ldb, const int32_t* offsets, int E, int64_t Tk,
                      int64_t M, int64_t N, bf16_t* c, hipStream_t st) {
  Params P{};
  P.A = a; P.lda = lda;
  P.B = b; P.ldb = ldb;
  P.C = c; P.ldc = N; P.c_stride = M * N;
  P.offsets = offsets; P.E = E; P.Tk = Tk;
  P.M = static_cast<int>(M); P.N = static_cast<int>(N);
  P.ntn = static_cast<int>((N + BN - 1) / BN);
  const int64_t mtiles = (M + BM - 1) / BM;
  const int grid = static_cast<int>(E * mtiles * P.ntn);
  return launch<kSegK, false, false, kStore>(P, grid, st);
}

}  // namespace moe
