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
//              wave); stores AB (bf16) and S = w * silu(gate) * up
//   kDSwiglu : acc = dS; reads AB and w, writes dAB = (dA_g, dA_u) and
//              per-tile partial sums of dS * H for the routing-weight grad
//
// Tile: 256 x 256 x 64 on MFMA 32x32x16.  The waves of a workgroup form a
// WM x WN grid over the tile (each wave owns (256/WM) x (256/WN) outputs):
// 4 waves as 2 x 2 (one wave per SIMD, 256 accumulators a lane) or 8 waves
// as 2 x 4 (two waves per SIMD, so one wave's LDS and global traffic
// overlaps the other's MFMAs).  LDS: two stages of (256 + 256) x 64 bf16,
// rows of 128 B with a 16-byte-chunk XOR swizzle that keeps both the tile
// stores and the MFMA fragment reads free of bank conflicts.

#include <type_traits>

#include "common.cuh"
#include "internal.h"

namespace moe {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kTileElems = BM * BK;       // one operand stage (A or B)
constexpr int kStageElems = 2 * kTileElems;
constexpr int kGroupN = 4;                // n-tiles per scheduling group
constexpr int kEpiRows = 64;              // rows per epilogue pass of a wave

enum Mode { kSegM = 0, kSegK = 1 };
enum Epi { kStore = 0, kSwiglu = 1, kDSwiglu = 2, kStoreF32 = 3 };

template <int WM_, int WN_>
struct Cfg {
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int TM = BM / WM, TN = BN / WN;   // wave tile
  static constexpr int BI = TM / 32, BJ = TN / 32;   // 32x32 blocks
  static constexpr int kEpiLd = TN + 4;              // fp32 stage stride
  static constexpr int kSmemBytes =
      (kWaves * kEpiRows * kEpiLd * 4 > 2 * kStageElems * 2)
          ? kWaves * kEpiRows * kEpiLd * 4
          : 2 * kStageElems * 2;
  // operand moving: 4 waves move both tiles, 8 waves split them (the first
  // 256 threads move A, the other 256 B)
  static constexpr bool kSplitLoad = kThreads == 512;
};

using Cfg4 = Cfg<2, 2>;
using Cfg8 = Cfg<2, 4>;

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
  // SegM split-K (kStoreF32 only): the reduction is cut into ksplit
  // contiguous ranges; range s writes its partial sums to plane s of C
  // (plane = elements between planes).  The combine adds the planes.
  int ksplit;
  int64_t plane;
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Instruction classes for the scheduling-group hints of the K-loop.
constexpr int kSgMfma = 0x008;
constexpr int kSgVmemRead = 0x020;
constexpr int kSgDsRead = 0x100;
constexpr int kSgDsWrite = 0x200;
#define sched_group(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

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

// One operand tile of 256 rows (M or N) x 64 k is moved by 256 threads
// (t = 0 .. 255) as 8 pieces of 16 B each, held in registers between the
// global load and the LDS store.  The pieces are moved in two halves
// (part 0: pieces 0-3, part 1: pieces 4-7) so the traffic can be spread
// over the k-slices of the pipeline.  Byte offsets are split into a
// per-thread part, computed once, and a per-piece part that is the same
// for the whole workgroup.
constexpr int kMoveThreads = 256;

template <bool KC>
struct Mover;

// K-contiguous operand: piece i is the 16-byte chunk (row = t/8 + 32 i,
// chunk = t%8).  blk(i) gives the operand row of the first row of the
// 32-row block i.
template <>
struct Mover<true> {
  uint32_t tpart;   // (t/8) * ld * 2 + (t%8) * 16
  int koff;         // (t%8) * 8
  __device__ __forceinline__ void init(int t, int64_t ld) {
    tpart = static_cast<uint32_t>(((t >> 3) * ld + (t & 7) * 8) * 2);
    koff = (t & 7) * 8;
  }
  template <typename Blk>
  __device__ __forceinline__ void load(i32x4* v, __amdgpu_buffer_rsrc_t rs,
                                       int64_t ld, int k0, int kmax, Blk blk,
                                       int part) const {
    const bool kok = k0 + koff < kmax;
#pragma unroll
    for (int i = 4 * part; i < 4 * part + 4; ++i) {
      const uint32_t off =
          tpart + static_cast<uint32_t>((blk(i) * ld + k0) * 2);
      v[i] = buf_load16(rs, kok ? off : kOob);
    }
  }
  __device__ __forceinline__ static void store(const i32x4* v, bf16_t* lds,
                                               int t, int part) {
    const int chunk = t & 7;
#pragma unroll
    for (int i = 4 * part; i < 4 * part + 4; ++i) {
      const int row = (t >> 3) + 32 * i;
      *reinterpret_cast<i32x4*>(lds + lds_off(row, chunk)) = v[i];
    }
  }
};

// MN-contiguous operand: 64 k-rows x 256 columns as 256 blocks of 8x8;
// thread t loads block t (k = kr*8 + i, i = 0..7 is piece i; columns
// colbase + mc*8 .. +7) and transposes it so that each column's 8 k-values
// become one LDS chunk (part 0 writes columns 0-3 of the block, part 1
// columns 4-7).
template <>
struct Mover<false> {
  uint32_t tpart;   // (kr*8 * ld + mc*8) * 2
  int krow;         // kr * 8
  __device__ __forceinline__ void init(int t, int64_t ld) {
    krow = (t >> 5) * 8;
    tpart = static_cast<uint32_t>((krow * ld + (t & 31) * 8) * 2);
  }
  __device__ __forceinline__ void load(i32x4* v, __amdgpu_buffer_rsrc_t rs,
                                       int64_t ld, int k0, int kmax,
                                       int64_t colbase, int part) const {
#pragma unroll
    for (int i = 4 * part; i < 4 * part + 4; ++i) {
      const uint32_t off =
          tpart + static_cast<uint32_t>(((k0 + i) * ld + colbase) * 2);
      v[i] = buf_load16(rs, (k0 + krow + i < kmax) ? off : kOob);
    }
  }
  __device__ __forceinline__ static void store(const i32x4* v, bf16_t* lds,
                                               int t, int part) {
    const int kr = t >> 5, mc = t & 31;
    // v[i] holds k = kr*8+i, columns mc*8+0..7 (dword q: columns 2q, 2q+1)
#pragma unroll
    for (int m = 4 * part; m < 4 * part + 4; ++m) {
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

// Load part `part` of one operand with the mover of its layout: K-contig
// movers take the block map, MN-contig movers the first column.
template <bool KC, typename M, typename Blk>
__device__ __forceinline__ void load_one(const M& mv, i32x4* v,
                                         __amdgpu_buffer_rsrc_t rs, int64_t ld,
                                         int k0, int part, Blk blk,
                                         int64_t colbase, int kmax) {
  if constexpr (KC)
    mv.load(v, rs, ld, k0, kmax, blk, part);
  else
    mv.load(v, rs, ld, k0, kmax, colbase, part);
}

__device__ __forceinline__ int find_segment(const int* pref, int E, int key) {
  // largest e in [0, E) with pref[e] <= key (pref non-decreasing)
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= key) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <class C, int MODE, bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(C::kThreads, 1) void grouped_gemm_kernel(
    Params P) {
  constexpr int NT = C::kThreads;
  constexpr int BI = C::BI, BJ = C::BJ, TM = C::TM, TN = C::TN;
  __shared__ __attribute__((aligned(16))) bf16_t smem[C::kSmemBytes / 2];
  __shared__ int s_pref[kMaxExperts + 1];
  __shared__ float s_dp[C::WN * BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int E = P.E;

  // ---------------------------------------------------------- tile decode
  // SegM grids hold ksplit copies of an upper bound on the tile count;
  // copy s (the slowest index) computes reduction range s.
  const int lbid = xcd_remap(blockIdx.x, gridDim.x);
  const int per_split = gridDim.x / P.ksplit;
  const int split = lbid / per_split;
  const int bid = lbid - split * per_split;
  int e, mt, nt;
  int64_t seg0;      // first permuted row of the expert
  int seg_len;       // rows of the expert
  if (MODE == kSegM) {
    // prefix of m-tiles per expert
    for (int i = tid; i <= E; i += NT) {
      int c = 0;
      if (i < E) c = (P.offsets[i + 1] - P.offsets[i] + BM - 1) / BM;
      s_pref[i] = c;
    }
    __syncthreads();
    if (tid < 64) {
      // exclusive scan of the E+1 entries by one wave, kPer entries a lane
      constexpr int kPer = (kMaxExperts + 1 + 63) / 64;
      int loc[kPer];
      int sum = 0;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int i = tid * kPer + q;
        loc[q] = (i <= E) ? s_pref[i] : 0;
        sum += loc[q];
      }
      int incl = sum;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const int o = __shfl_up(incl, m, 64);
        if (tid >= m) incl += o;
      }
      int run = incl - sum;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int i = tid * kPer + q;
        if (i <= E) s_pref[i] = run;
        run += loc[q];
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
  // reduction range [kbeg, Kdim) of this workgroup
  const int kchunk =
      (MODE == kSegM) ? ((P.K + P.ksplit * BK - 1) / (P.ksplit * BK)) * BK : 0;
  const int kbeg = (MODE == kSegM) ? min(P.K, split * kchunk) : 0;
  const int Kdim = (MODE == kSegM) ? min(P.K, kbeg + kchunk) : seg_len;

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

  // Block maps: the operand row of the first row of 32-row block i of the
  // tile.  The dual-B tile of kSwiglu puts, inside every wave's TN
  // columns, TN/2 gate columns followed by the up columns of the same
  // indices.
  const int f = P.f;
  const int n0g = nt * (BN / 2);
  auto blk_a = [&](int i) -> int64_t { return m0 + 32 * i; };
  auto blk_b = [&](int i) -> int64_t {
    if (EPI == kSwiglu) {
      constexpr int half = BJ / 2;
      const int w_n = (32 * i) / TN, jj = i % BJ;
      return static_cast<int64_t>((jj / half) * f + n0g + w_n * (TN / 2) +
                                  (jj % half) * 32);
    }
    return n0 + 32 * i;
  };

  // which operand this thread moves: with 4 waves every thread moves a
  // piece of both tiles; with 8 waves the first 256 threads move A and the
  // other 256 move B (one register set per thread either way).  The choice
  // is uniform over a wave.
  const bool mv_a = !C::kSplitLoad ||
                    __builtin_amdgcn_readfirstlane(tid) < kMoveThreads;
  const int lt = tid & (kMoveThreads - 1);
  const int nk = (Kdim - kbeg + BK - 1) / BK;
  Mover<AKC> ma;
  Mover<BKC> mb;
  ma.init(lt, P.lda);
  mb.init(lt, P.ldb);
  // with 8 waves and one layout for both operands, one mover serves either
  const __amdgpu_buffer_rsrc_t rs_own = mv_a ? rsA : rsB;
  const int64_t ld_own = mv_a ? P.lda : P.ldb;
  Mover<AKC> mown;
  mown.init(lt, ld_own);

  f32x16 acc[BI][BJ];
#pragma unroll
  for (int i = 0; i < BI; ++i)
#pragma unroll
    for (int j = 0; j < BJ; ++j) acc[i][j] = f32x16{};

  const int fr = lane & 31;      // fragment row inside a 32-block
  const int fk = lane >> 5;      // which 8-wide k half

  // Fragments of k-slice kk (16 wide) of one LDS stage.
  auto read_frags = [&](const bf16_t* sa, int kk, bf16x8_v* af,
                        bf16x8_v* bf) {
    const bf16_t* sb = sa + kTileElems;
    const int chunk = kk * 2 + fk;
#pragma unroll
    for (int i = 0; i < BI; ++i)
      af[i] = __builtin_bit_cast(
          bf16x8_v, *reinterpret_cast<const i32x4*>(
                        sa + lds_off(wm * TM + i * 32 + fr, chunk)));
#pragma unroll
    for (int j = 0; j < BJ; ++j)
      bf[j] = __builtin_bit_cast(
          bf16x8_v, *reinterpret_cast<const i32x4*>(
                        sb + lds_off(wn * TN + j * 32 + fr, chunk)));
  };
  auto mfmas = [&](const bf16x8_v* af, const bf16x8_v* bf) {
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
      for (int j = 0; j < BJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j],
                                                            acc[i][j], 0, 0,
                                                            0);
  };
  i32x4 va[8];
  i32x4 vb[C::kSplitLoad ? 1 : 8];
  // part p of this thread's operand(s): global -> registers, and
  // registers -> LDS stage st
  auto gload = [&](int k0, int part) {
    if (C::kSplitLoad) {
      if constexpr (AKC)
        mown.load(va, rs_own, ld_own, k0, Kdim,
                  [&](int i) { return mv_a ? blk_a(i) : blk_b(i); }, part);
      else
        mown.load(va, rs_own, ld_own, k0, Kdim, mv_a ? m0 : n0, part);
    } else {
      load_one<AKC>(ma, va, rsA, P.lda, k0, part, blk_a, m0, Kdim);
      load_one<BKC>(mb, vb, rsB, P.ldb, k0, part, blk_b, n0, Kdim);
    }
  };
  auto lstore = [&](bf16_t* st, int part) {
    if (C::kSplitLoad) {
      Mover<AKC>::store(va, st + (mv_a ? 0 : kTileElems), lt, part);
    } else {
      Mover<AKC>::store(va, st, lt, part);
      Mover<BKC>::store(vb, st + kTileElems, lt, part);
    }
  };
  // 8 waves with different layouts: each wave role gets its own copy of
  // the K-loop, so neither carries the other's mover state
  auto gload_a = [&](int k0, int part) {
    load_one<AKC>(ma, va, rsA, P.lda, k0, part, blk_a, m0, Kdim);
  };
  auto lstore_a = [&](bf16_t* st, int part) {
    Mover<AKC>::store(va, st, lt, part);
  };
  auto gload_b = [&](int k0, int part) {
    load_one<BKC>(mb, va, rsB, P.ldb, k0, part, blk_b, n0, Kdim);
  };
  auto lstore_b = [&](bf16_t* st, int part) {
    Mover<BKC>::store(va, st + kTileElems, lt, part);
  };

  // Software pipeline over k-steps of BK.  At iteration kt the mover
  // registers hold stage kt+1 (loaded one iteration earlier); they are
  // written to the other LDS buffer during k-slices 0 and 1, and stage
  // kt+2 is loaded into them during k-slices 2 and 3.  MFMA fragments are
  // double-buffered so the next slice's LDS reads overlap the current
  // slice's MFMAs.  Loads past K return zeros and the one stray store of
  // the last iteration lands in the buffer no one reads any more.
  auto kloop = [&](auto&& gload, auto&& lstore) {
    constexpr int kMf = BI * BJ;                   // MFMAs per k-slice
    constexpr int kRd = BI + BJ;                   // fragment reads per slice
    constexpr int kMv = C::kSplitLoad ? 4 : 8;     // moves per slice
    bf16x8_v a0[BI], b0[BJ], a1[BI], b1[BJ];
    if (nk > 0) {
      gload(kbeg, 0);
      gload(kbeg, 1);
      lstore(smem, 0);
      lstore(smem, 1);
      gload(kbeg + BK, 0);
      gload(kbeg + BK, 1);
      __syncthreads();
      read_frags(smem, 0, a0, b0);
    }
    for (int kt = 0; kt < nk; ++kt) {
      const bf16_t* cur = smem + (kt & 1) * kStageElems;
      bf16_t* nxt = smem + ((kt + 1) & 1) * kStageElems;
      const int k2 = kbeg + (kt + 2) * BK;
      // slice 0: MFMAs on (a0,b0); reads of slice 1; stores of stage kt+1
      read_frags(cur, 1, a1, b1);
      lstore(nxt, 0);
      mfmas(a0, b0);
  #pragma unroll
      for (int i = 0; i < kMf; ++i) {
        sched_group(kSgMfma, 1);
        if (i < kRd) sched_group(kSgDsRead, 1);
        if (i < kMv) sched_group(kSgDsWrite, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice 1: MFMAs on (a1,b1); reads of slice 2; stores of stage kt+1
      read_frags(cur, 2, a0, b0);
      lstore(nxt, 1);
      mfmas(a1, b1);
  #pragma unroll
      for (int i = 0; i < kMf; ++i) {
        sched_group(kSgMfma, 1);
        if (i < kRd) sched_group(kSgDsRead, 1);
        if (i < kMv) sched_group(kSgDsWrite, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice 2: MFMAs on (a0,b0); reads of slice 3; loads of stage kt+2
      read_frags(cur, 3, a1, b1);
      gload(k2, 0);
      mfmas(a0, b0);
  #pragma unroll
      for (int i = 0; i < kMf; ++i) {
        sched_group(kSgMfma, 1);
        if (i < kRd) sched_group(kSgDsRead, 1);
        if (i < kMv) sched_group(kSgVmemRead, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice 3: MFMAs on (a1,b1); loads of stage kt+2
      gload(k2, 1);
      mfmas(a1, b1);
  #pragma unroll
      for (int i = 0; i < kMf; ++i) {
        sched_group(kSgMfma, 1);
        if (i < kMv) sched_group(kSgVmemRead, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      read_frags(nxt, 0, a0, b0);
    }
  };

  if constexpr (C::kSplitLoad && AKC != BKC) {
    if (mv_a) kloop(gload_a, lstore_a);
    else kloop(gload_b, lstore_b);
  } else {
    kloop(gload, lstore);
  }

  // ---------------------------------------------------------- epilogue
  // acc[i][j][v] is C[row][col] of the wave's TM x TN sub-tile with
  //   row = i*32 + (v/4)*8 + (lane/32)*4 + v%4,  col = j*32 + lane%32.
  // Each pass of 64 rows is staged through the wave's own LDS region as
  // fp32 [64][kEpiLd] and then processed row by row: a lane owns 4
  // consecutive columns, so global reads and bf16 stores are contiguous.
  constexpr int LD = C::kEpiLd;
  float* stage = reinterpret_cast<float*>(smem) + wave * (kEpiRows * LD);
  const int64_t cbase = (MODE == kSegM) ? seg0 * P.ldc
                                        : static_cast<int64_t>(e) * P.c_stride;
  const float* w = ((EPI == kSwiglu || EPI == kDSwiglu) && P.w) ? P.w + seg0
                                                                : nullptr;
  constexpr int kLanesPerRow = TN / 4;             // 4 columns a lane
  constexpr int kRowsPerPass = 64 / kLanesPerRow;
#pragma unroll
  for (int h = 0; h < TM / kEpiRows; ++h) {
#pragma unroll
    for (int ii = 0; ii < kEpiRows / 32; ++ii)
#pragma unroll
      for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = ii * 32 + (v >> 2) * 8 + fk * 4 + (v & 3);
          stage[r * LD + j * 32 + fr] = acc[h * (kEpiRows / 32) + ii][j][v];
        }
    __syncthreads();
    const int row_base = m0 + wm * TM + h * kEpiRows;   // absolute row
    if (EPI == kStore || EPI == kStoreF32) {
      const int c4 = (lane % kLanesPerRow) * 4;
      const int col = n0 + wn * TN + c4;
      for (int r = lane / kLanesPerRow; r < kEpiRows; r += kRowsPerPass) {
        const int row = row_base + r;
        if (row < Mvalid && col < P.N) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(stage + r * LD + c4);
          const int64_t o = cbase + static_cast<int64_t>(row) * P.ldc + col;
          if (EPI == kStoreF32) {
            *reinterpret_cast<f32x4*>(P.Cf + split * P.plane + o) = x;
          } else {
            uint2 u;
            u.x = pack_bf16x2(x[0], x[1]);
            u.y = pack_bf16x2(x[2], x[3]);
            *reinterpret_cast<uint2*>(P.C + o) = u;
          }
        }
      }
    } else if (EPI == kSwiglu) {
      // stage columns [0, TN/2) are gate, [TN/2, TN) the matching up
      bf16_t* AB = P.C + cbase;                       // [rows][2f]
      bf16_t* S = P.S + seg0 * static_cast<int64_t>(f);
      constexpr int kLanesG = TN / 8;                 // lanes per row
      constexpr int kRowsG = 64 / kLanesG;
      const int c4 = (lane % kLanesG) * 4;
      const int col = n0g + wn * (TN / 2) + c4;       // gate column
      for (int r = lane / kLanesG; r < kEpiRows; r += kRowsG) {
        const int row = row_base + r;
        if (row < Mvalid && col < f) {
          const f32x4 g = *reinterpret_cast<const f32x4*>(stage + r * LD + c4);
          const f32x4 u =
              *reinterpret_cast<const f32x4*>(stage + r * LD + TN / 2 + c4);
          const float wr = w ? w[row] : 1.0f;
          float sv[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            sv[c] = wr * (g[c] * sigmoidf_(g[c]) * u[c]);
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
      const int c4 = (lane % kLanesPerRow) * 4;
      const int col = n0 + wn * TN + c4;
      for (int r = lane / kLanesPerRow; r < kEpiRows; r += kRowsPerPass) {
        const int row = row_base + r;
        float part = 0.0f;
        if (row < Mvalid && col < f) {
          const int64_t ro = static_cast<int64_t>(row);
          const f32x4 ds = *reinterpret_cast<const f32x4*>(stage + r * LD + c4);
          const uint2 gb = *reinterpret_cast<const uint2*>(AB + ro * 2 * f + col);
          const uint2 ub =
              *reinterpret_cast<const uint2*>(AB + ro * 2 * f + f + col);
          const float g[4] = {bf_lo(gb.x), bf_hi(gb.x), bf_lo(gb.y),
                              bf_hi(gb.y)};
          const float u[4] = {bf_lo(ub.x), bf_hi(ub.x), bf_lo(ub.y),
                              bf_hi(ub.y)};
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
        // row sum over the lanes of this row, fixed butterfly order
#pragma unroll
        for (int m = 1; m < kLanesPerRow; m <<= 1)
          part += __shfl_xor(part, m, 64);
        if ((lane % kLanesPerRow) == 0)
          s_dp[wn * BM + wm * TM + h * kEpiRows + r] = part;
      }
    }
    __syncthreads();
  }
  if (EPI == kDSwiglu) {
    // the tile's column groups, added in order (wn = 0, 1, ...)
    for (int lr = tid; lr < BM; lr += NT) {
      const int row = m0 + lr;
      if (row < Mvalid) {
        float sum = s_dp[lr];
#pragma unroll
        for (int q = 1; q < C::WN; ++q) sum += s_dp[q * BM + lr];
        P.dp_part[(seg0 + row) * P.ntn + nt] = sum;
      }
    }
  }
}

// Tile configuration per GEMM.  Measured on MI355X at the Mixtral shape,
// 8 waves beat 4 for every GEMM of the layer (forward +4-10%, wgrad
// +2-15%, dgrad +15-30%); the 4-wave configuration is kept selectable.
#ifndef MOE_GEMM_WAVES
#define MOE_GEMM_WAVES 8
#endif
using CfgFwd = std::conditional_t<MOE_GEMM_WAVES == 4, Cfg4, Cfg8>;
#ifndef MOE_DGRAD_WAVES
#define MOE_DGRAD_WAVES 8
#endif
using CfgDgrad = std::conditional_t<MOE_DGRAD_WAVES == 8, Cfg8, Cfg4>;
using CfgWgrad = Cfg8;

template <class C, int MODE, bool AKC, bool BKC, int EPI>
hipError_t launch(Params P, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (P.ksplit < 1) P.ksplit = 1;
  grid *= P.ksplit;
  hipLaunchKernelGGL((grouped_gemm_kernel<C, MODE, AKC, BKC, EPI>),
                     dim3(grid), dim3(C::kThreads), 0, s, P);
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
  return launch<CfgFwd, kSegM, true, true, kSwiglu>(P, segm_grid(Tk, E, P.ntn), st);
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
  P.ksplit = kOutPlanes; P.plane = Tk * d;
  P.ntn = static_cast<int>((d + BN - 1) / BN);
  return launch<CfgFwd, kSegM, true, true, kStoreF32>(P, segm_grid(Tk, E, P.ntn), st);
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
  return launch<CfgDgrad, kSegM, true, false, kDSwiglu>(P, segm_grid(Tk, E, P.ntn), st);
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
  P.ksplit = kOutPlanes; P.plane = Tk * d;
  P.ntn = static_cast<int>((d + BN - 1) / BN);
  return launch<CfgDgrad, kSegM, true, false, kStoreF32>(P, segm_grid(Tk, E, P.ntn), st);
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
  return launch<CfgWgrad, kSegK, false, false, kStore>(P, grid, st);
}

}  // namespace moe
