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
//
// MXFP8 (Challenge 2 of the same page: 8-bit values, one scale per block
// of 32 along the reduction axis): the same kernel with MX = true runs on
// E4M3 codes and E8M0 scale bytes through gfx950's block-scaled MFMA
// (32x32x64: per operand and row, lanes 0-31 supply the scale byte of the
// slice's first 32-block and lanes 32-63 that of its second; every lane
// holds 16 codes of each block).  Both operands are K-contiguous; their addresses and K
// coordinates count pairs of codes, so a 64-unit stage holds 128 codes and
// the movers and LDS tiles are shared unchanged with the bf16 kernel.  Each
// lane loads the scale dwords of its fragment rows (4 blocks = one stage)
// straight from global memory one stage ahead.  The epilogues can also
// emit their bf16 result MX-quantized along the columns (S for the down
// GEMM, dAB for the gate_up data gradient).  A third grouping mode serves
// the MX weight gradients: operands transposed by the token-axis quantizer
// ([rows][padded tokens], blocks restarting at every expert), reduced over
// each expert's padded token range.

#include <type_traits>

#include "common.cuh"
#include "internal.h"
#include "mx.cuh"

namespace moe {
namespace {

// Epilogue output stores of the MX kernels' fc1 outputs (AB, S codes) and
// plain tile stores are streaming (non-temporal): on MI355X that made the
// MX fc1 GEMM 9% and the MX weight gradient 9% faster.  The bf16 kernels
// keep ordinary stores: streaming left their time unchanged but raised
// fc1's HBM reads from 3.6x to 4.1x the algorithmic bytes.  The dSwiGLU
// outputs keep ordinary stores everywhere (streaming made that GEMM 20%
// slower).
template <bool kStream>
__device__ __forceinline__ void st_epi(uint2* p, uint2 v) {
  if constexpr (kStream)
    __builtin_nontemporal_store((static_cast<uint64_t>(v.y) << 32) | v.x,
                                reinterpret_cast<uint64_t*>(p));
  else
    *p = v;
}
template <bool kStream>
__device__ __forceinline__ void st_epi(i32x4* p, i32x4 v) {
  if constexpr (kStream) __builtin_nontemporal_store(v, p);
  else *p = v;
}
template <bool kStream>
__device__ __forceinline__ void st_epi(uint32_t* p, uint32_t v) {
  if constexpr (kStream) __builtin_nontemporal_store(v, p);
  else *p = v;
}

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kTileElems = BM * BK;       // one operand stage (A or B)
constexpr int kStageElems = 2 * kTileElems;
constexpr int kGroupN = 4;                // n-tiles per scheduling group
constexpr int kGroupM = 8;                // m-tiles per block of a group
constexpr int kGroupMOne = 12;            // ... or all, up to this many
constexpr int kEpiRows = 64;              // rows per epilogue pass of a wave
#ifndef MOE_INDEP_LOOP
#define MOE_INDEP_LOOP 1
#endif
constexpr bool kIndepLoop = MOE_INDEP_LOOP != 0;
#ifndef MOE_SCALE_GROUP
#define MOE_SCALE_GROUP 4
#endif
// MX K-loop: stages whose scale dwords one thread loads together (a power
// of two; 4 measured best: 8, with the loop unrolled eight times, made
// the MXFP8 step 8% slower)
constexpr int kScaleGroup = MOE_SCALE_GROUP;

enum Mode { kSegM = 0, kSegK = 1, kSegKT = 2 };
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
  // SegM split-K (kStoreF32 only): the reduction is cut into ksplit (1 or
  // 2) contiguous ranges; range s writes its partial sums to plane s of C
  // (plane = elements between planes).  The combine adds the planes.
  int ksplit;
  int64_t plane;
  int xcd_cus;       // compute units of one XCD (split-K piece sizing)
  // MX operands: scale bytes [rows][lds_*] (one per 32 codes along K),
  // bs_stride = bytes between experts' B scales (SegM)
  const uint8_t* sA;
  int64_t lds_a;
  const uint8_t* sB;
  int64_t lds_b;
  int64_t bs_stride;
  // MX epilogue outputs: codes [rows][ldq] and scales [rows][ldq / 32] of
  // S (kSwiglu, ldq = f) or dAB (kDSwiglu, ldq = 2f); null to skip
  uint8_t* Qc;
  uint8_t* Qs;
  // MX token-axis epilogue outputs (kSwiglu: S, f columns; kDSwiglu: dAB,
  // 2f columns), quantized from the bf16 values the epilogue rounds to, in
  // blocks of 32 rows restarting at each expert's first row: codes
  // [cols][ldt] and scales [cols][ldt / 32], expert e's rows starting at
  // its padded start (the sum over e' < e of counts rounded up to 128);
  // null to skip
  uint8_t* Tc;
  uint8_t* Ts;
  int64_t ldt;
};

// 16-byte chunk swizzle of a [row][64 k] bf16 operand tile (128-byte
// rows): chunk c of row r sits at chunk c ^ swz(r).  A fragment read (one
// chunk of 32 consecutive rows) and a mover store (all 8 chunks of 8 rows)
// are then spread evenly over the LDS banks, and swz is the same for rows
// 16 apart, so the 32-row blocks of a tile differ by a constant offset and
// every per-lane address is computed once per tile.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

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
constexpr int kTileBytes = kTileElems * 2;
constexpr int kBlkBytes = 32 * BK * 2;     // one 32-row block of a tile

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo,
                                             uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Orders a wave's LDS writes before its own later LDS reads of other
// lanes' data.  The epilogue needs no more: each wave stages through its
// own LDS region.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


// k-steps of the second piece of a two-piece split reduction of nk steps,
// on an XCD whose c CUs run ntx tiles: first all first pieces, then all
// second pieces, each CU taking the next piece as it frees.  With b = ntx
// mod c, b CUs run one first piece more than the others; second pieces of
// 1/m of the reduction let both groups end together at ntx/c tiles' time
// when m is a multiple of c / gcd(b, c) (and m >= 2).  m is kept to at
// most 8: a shorter piece would be mostly fixed per-tile cost.  b = 0
// needs no balancing and keeps two halves.
__device__ __forceinline__ int split_second_steps(int ntx, int nk, int c) {
  const int b = ntx % c;
  int m = 2;
  if (b != 0) {
    int u = b, v = c;
    while (v != 0) {
      const int t = u % v;
      u = v;
      v = t;
    }
    m = max(2, min(8, c / u));
  }
  return max(1, (nk + m / 2) / m);
}

// One operand tile of 256 rows (M or N) x 64 k is moved by 256 threads
// (t = 0 .. 255) as 8 pieces of 16 B each, held in registers between the
// global load and the LDS store.  The pieces are moved in two halves
// (part 0: pieces 0-3, part 1: pieces 4-7) so the traffic can be spread
// over the k-slices of the pipeline.  Byte offsets are split into a
// per-thread part, computed once, and a per-piece part that is the same
// for the whole workgroup; LDS offsets are per-thread bases plus
// constants.  init's tile_bytes places the operand's tile (A at 0, B at
// 2 kTileBytes) inside a stage; store takes the stage's base.
//
// Loads come in two forms.  The masked form tests every lane's k range
// against kmax, for the one stage that may end inside a tile.  The full
// form serves a stage that lies wholly inside [0, kmax) or wholly past it
// (its data is never read): no mask, the k offset in soffset (clamped to
// 0 past kmax, so the load stays inside the buffer), and rows past the
// buffer still caught by the range check on voffset.
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
  int lds0;         // LDS byte offset of piece 0 in a stage
  __device__ __forceinline__ void init(int t, int64_t ld, int tile_bytes) {
    tpart = static_cast<uint32_t>(((t >> 3) * ld + (t & 7) * 8) * 2);
    koff = (t & 7) * 8;
    lds0 = tile_bytes + lds_off(t >> 3, t & 7) * 2;
  }
  template <bool kFull, typename Blk>
  __device__ __forceinline__ void load(i32x4* v, __amdgpu_buffer_rsrc_t rs,
                                       int64_t ld, int k0, int kmax, Blk blk,
                                       int part) const {
    if constexpr (kFull) {
      const uint32_t ks = k0 < kmax ? static_cast<uint32_t>(k0) * 2 : 0u;
#pragma unroll
      for (int i = 4 * part; i < 4 * part + 4; ++i)
        v[i] = buf_load16(rs, tpart + static_cast<uint32_t>(blk(i) * ld * 2),
                          ks);
    } else {
      const bool kok = k0 + koff < kmax;
#pragma unroll
      for (int i = 4 * part; i < 4 * part + 4; ++i) {
        const uint32_t off =
            tpart + static_cast<uint32_t>((blk(i) * ld + k0) * 2);
        v[i] = buf_load16(rs, kok ? off : kOob);
      }
    }
  }
  // rows t/8 + 32 i share the swizzle: piece i is 32 rows on
  __device__ __forceinline__ void store(const i32x4* v, uint8_t* stage,
                                        int part) const {
#pragma unroll
    for (int i = 4 * part; i < 4 * part + 4; ++i)
      *reinterpret_cast<i32x4*>(stage + lds0 + i * kBlkBytes) = v[i];
  }
};

// MN-contiguous operand: 64 k-rows x 256 columns, kept in LDS as it lies
// in memory (the [k][mn] tile of kmn_off) and transposed by the fragment
// reads (ds_read_b64_tr_b16, see frag_tr).  Thread t moves the 16-byte
// column chunk t % 32 of k-rows 8 (t / 32) + i, i = 0..7 (piece i); part 0
// holds pieces 0-3, part 1 pieces 4-7.  A full load keeps the k-row in
// voffset: on a segment's last k-row, the chunks past the last column are
// past the buffer's end.
template <>
struct Mover<false> {
  uint32_t tpart;   // (kr*8 * ld + mc*8) * 2
  int krow;         // kr * 8
  int lds0[4];      // LDS byte offsets of pieces 0-3 in a stage
  __device__ __forceinline__ void init(int t, int64_t ld, int tile_bytes) {
    krow = (t >> 5) * 8;
    tpart = static_cast<uint32_t>((krow * ld + (t & 31) * 8) * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      lds0[q] = tile_bytes + kmn_off(krow + q, t & 31);
  }
  template <bool kFull>
  __device__ __forceinline__ void load(i32x4* v, __amdgpu_buffer_rsrc_t rs,
                                       int64_t ld, int k0, int kmax,
                                       int64_t colbase, int part) const {
    if constexpr (kFull) {
      const int kc = k0 < kmax ? k0 : 0;
#pragma unroll
      for (int i = 4 * part; i < 4 * part + 4; ++i)
        v[i] = buf_load16(
            rs, tpart + static_cast<uint32_t>(((kc + i) * ld + colbase) * 2),
            0u);
    } else {
#pragma unroll
      for (int i = 4 * part; i < 4 * part + 4; ++i) {
        const uint32_t off =
            tpart + static_cast<uint32_t>(((k0 + i) * ld + colbase) * 2);
        v[i] = buf_load16(rs, (k0 + krow + i < kmax) ? off : kOob);
      }
    }
  }
  // k-row krow + i: the chunk XOR repeats every 4 rows (krow is a multiple
  // of 8)
  __device__ __forceinline__ void store(const i32x4* v, uint8_t* stage,
                                        int part) const {
#pragma unroll
    for (int i = 4 * part; i < 4 * part + 4; ++i)
      *reinterpret_cast<i32x4*>(stage + lds0[i & 3] + (i & ~3) * 512) = v[i];
  }
};


// E2M1 codes two a byte -> E4M3 codes one a byte, exactly (every E2M1
// value is an E4M3 value): through f16 with gfx950's scaled conversions at
// scale 1 (checked against the code table on every 16-bit input).
__device__ __forceinline__ i32x4 e2m1x16_to_e4m3(uint32_t w0, uint32_t w1) {
  typedef __attribute__((ext_vector_type(2))) short s2;
  const s2 z = {0, 0};
  s2 r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(
      z, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0), 1.0f, false);
  r0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(
      r0, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1), 1.0f, true);
  s2 r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(
      z, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2), 1.0f, false);
  r1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(
      r1, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3), 1.0f, true);
  s2 r2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(
      z, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 0), 1.0f, false);
  r2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(
      r2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 1), 1.0f, true);
  s2 r3 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(
      z, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 2), 1.0f, false);
  r3 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(
      r3, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 3), 1.0f, true);
  return i32x4{__builtin_bit_cast(int, r0), __builtin_bit_cast(int, r1),
               __builtin_bit_cast(int, r2), __builtin_bit_cast(int, r3)};
}

// K-contiguous MXFP4 operand (two codes a byte), widened to E4M3 on its
// way to LDS: the LDS tiles, fragments and MFMAs are then those of an E4M3
// operand with the same block scales.  Piece i of thread t is Mover<true>'s
// 16-code chunk (row t/8 + 32 i, chunk t%8), loaded as its 8 code bytes
// (into the low half of the piece register) and widened at the LDS store.
// k0 and kmax count code pairs, which are bytes here.
struct Mover4 {
  uint32_t tpart;   // (t/8) * row bytes + (t%8) * 8
  uint32_t ldb;     // operand row stride in bytes
  int koff;         // (t%8) * 8 code pairs
  int lds0;         // LDS byte offset of piece 0 in a stage
  __device__ __forceinline__ void init(int t, int64_t ld_units,
                                       int tile_bytes) {
    ldb = static_cast<uint32_t>(ld_units * 2);
    tpart = static_cast<uint32_t>(t >> 3) * ldb +
            static_cast<uint32_t>((t & 7) * 8);
    koff = (t & 7) * 8;
    lds0 = tile_bytes + lds_off(t >> 3, t & 7) * 2;
  }
  template <bool kFull, typename Blk>
  __device__ __forceinline__ void load(i32x4* v, __amdgpu_buffer_rsrc_t rs,
                                       int k0, int kmax, Blk blk,
                                       int part) const {
    const bool kok = k0 + koff < kmax;
    const uint32_t ks = k0 < kmax ? static_cast<uint32_t>(k0) : 0u;
#pragma unroll
    for (int i = 4 * part; i < 4 * part + 4; ++i) {
      const uint32_t row = tpart + static_cast<uint32_t>(blk(i)) * ldb;
      const auto w =
          kFull ? __builtin_amdgcn_raw_buffer_load_b64(rs, row, ks, 0)
                : __builtin_amdgcn_raw_buffer_load_b64(
                      rs, kok ? row + static_cast<uint32_t>(k0) : kOob, 0, 0);
      v[i] = i32x4{static_cast<int>(w[0]), static_cast<int>(w[1]), 0, 0};
    }
  }
  __device__ __forceinline__ void store(const i32x4* v, uint8_t* stage,
                                        int part) const {
#pragma unroll
    for (int i = 4 * part; i < 4 * part + 4; ++i)
      *reinterpret_cast<i32x4*>(stage + lds0 + i * kBlkBytes) =
          e2m1x16_to_e4m3(static_cast<uint32_t>(v[i][0]),
                          static_cast<uint32_t>(v[i][1]));
  }
};

// Load part `part` of one operand with the mover of its layout: K-contig
// movers take the block map, MN-contig movers the first column.
template <bool KC, bool kFull, typename M, typename Blk>
__device__ __forceinline__ void load_one(const M& mv, i32x4* v,
                                         __amdgpu_buffer_rsrc_t rs, int64_t ld,
                                         int k0, int part, Blk blk,
                                         int64_t colbase, int kmax) {
  if constexpr (KC)
    mv.template load<kFull>(v, rs, ld, k0, kmax, blk, part);
  else
    mv.template load<kFull>(v, rs, ld, k0, kmax, colbase, part);
}

// Runs k-steps 0 .. nk-1 of a K-loop whose iteration kt reads LDS stage
// kt & 1 and prefetches stage kt + 2, as step(kt, stage, full): pairs
// (even kt, kt + 1) with the stage a compile-time constant and full loads
// up to kt_part, the iteration that prefetches a last stage ending inside
// its tile (-1: none), then single steps with a run-time stage and masked
// loads (at most four).  One loop of pairs and one of single steps: a loop
// that picks between the two forms each time round keeps both forms'
// registers live and spills.
template <typename Step>
__device__ __forceinline__ void run_ksteps(int nk, int kt_part, Step&& step) {
  const int kf = kt_part >= 0 ? min(nk, kt_part) : nk;
  int kt = 0;
  for (; kt + 1 < kf; kt += 2) {
    step(kt, 0, std::true_type{});
    step(kt + 1, 1, std::true_type{});
  }
  for (; kt < nk; ++kt) step(kt, kt & 1, std::false_type{});
}

// run_ksteps for a loop that also needs kt mod G, as step(kt, stage,
// full, kt % G): groups of G steps with both as compile-time constants
// and full loads up to kt_part, then single steps with run-time values
// and masked loads.
template <int G, typename Step, int... Is>
__device__ __forceinline__ void ksteps_group(int kt, Step&& step,
                                             std::integer_sequence<int, Is...>) {
  (step(kt + Is, Is & 1, std::true_type{}, std::integral_constant<int, Is>{}),
   ...);
}
template <int G, typename Step>
__device__ __forceinline__ void run_ksteps_g(int nk, int kt_part,
                                             Step&& step) {
  const int kf = kt_part >= 0 ? min(nk, kt_part) : nk;
  int kt = 0;
  for (; kt + G - 1 < kf; kt += G)
    ksteps_group<G>(kt, step, std::make_integer_sequence<int, G>{});
  for (; kt < nk; ++kt) step(kt, kt & 1, std::false_type{}, kt & (G - 1));
}

// Tile order inside one expert's mt x nt tile grid: groups of kGroupN
// n-tiles; inside a group, blocks of kGroupM m-tiles (the last group and
// block may be narrower), m fastest inside a block.  Consecutive tiles --
// which run together on one XCD -- then share kGroupN B column blocks and
// kGroupM A row blocks in its L2, in both short (forward: a few m-tiles an
// expert) and tall (weight gradients: M = d or 2f) grids.  An expert of at
// most kGroupMOne m-tiles is a single block: split in two, its last few
// m-tiles would run a whole tile time after the first block and read every
// B column block of the group from HBM again.
__device__ __forceinline__ void tile_order(int local, int mtn, int ntn,
                                           int* mt, int* nt) {
  const int grp = local / (mtn * kGroupN);
  const int ng = min(kGroupN, ntn - grp * kGroupN);
  int rem = local - grp * mtn * kGroupN;
  const int gm = mtn <= kGroupMOne ? mtn : kGroupM;
  const int blk = rem / (gm * ng);
  const int mb = min(gm, mtn - blk * gm);
  rem -= blk * gm * ng;
  *mt = blk * gm + rem % mb;
  *nt = grp * kGroupN + rem / mb;
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

// E4M3 codes of 4 values of one row and the scale byte of their 32-block,
// the block being held by 8 consecutive lanes (4 values each).  All 64
// lanes must call it; lanes with valid == false contribute zeros.
__device__ __forceinline__ uint32_t mx_quant4(const float* v, bool valid,
                                              uint32_t* scale_byte) {
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) amax = fmaxf(amax, valid ? fabsf(v[c]) : 0.0f);
  amax = dpp_group_max<8>(amax);
  const int e = mx_scale_exp(amax);
  const float inv = mx_inv_scale(e);
  const uint32_t word =
      e4m3_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  *scale_byte = static_cast<uint32_t>(e + 127);
  return word;
}

// Scaled MFMAs of one 64-code k-slice for A fragment rows [I0, I0 + NI)
// (af holds those NI fragments): the lane's scale byte is byte OPS of its
// (pre-shifted) scale dword.
template <int OPS, int I0, int NI, int BI, int BJ>
__device__ __forceinline__ void mx_mfmas(f32x16 (&acc)[BI][BJ],
                                         const i32x8* af, const i32x8* bf,
                                         const uint32_t* sa,
                                         const uint32_t* sb) {
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < BJ; ++j)
      acc[I0 + i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          af[i], bf[j], acc[I0 + i][j], 0, 0, OPS,
          static_cast<int>(sa[I0 + i]), OPS, static_cast<int>(sb[j]));
}

template <class C, int MODE, bool AKC, bool BKC, int EPI, bool MX, int FMT>
__global__ __launch_bounds__(C::kThreads, 1) void grouped_gemm_kernel(
    Params P) {
  // FMT bit 0 / bit 1: A / B holds MXFP4 (E2M1) codes, widened to E4M3 by
  // its movers
  static_assert(FMT == 0 || (MX && AKC && BKC && C::kSplitLoad),
                "E2M1 operands: MX kernels, K-contiguous, 8 waves");
  constexpr int NT = C::kThreads;
  constexpr int BI = C::BI, BJ = C::BJ, TM = C::TM, TN = C::TN;
  __shared__ __attribute__((aligned(16))) bf16_t smem[C::kSmemBytes / 2];
  __shared__ int s_pref[kMaxExperts + 1];
  // weight gradients: expert sizes and their descending order
  __shared__ int s_cnt[MODE == kSegM ? 1 : kMaxExperts];
  __shared__ int s_ord[MODE == kSegM ? 1 : kMaxExperts];
  __shared__ int s_stat[2];
  __shared__ float s_dp[C::WN * BM];
  // kDSwiglu: the routing weights of the tile's rows
  __shared__ float s_wrow[EPI == kDSwiglu ? BM : 1];
  // MX: scale dwords of the tile rows, [stage][A rows, B rows]
  __shared__ uint32_t s_scl[MX ? 2 * 2 * BM : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int E = P.E;

  // ---------------------------------------------------------- tile decode
  int e, mt, nt;
  int64_t seg0;      // first permuted row of the expert
  int seg_len;       // rows of the expert
  if (MODE == kSegM || MODE == kSegKT) {
    // SegM: prefix of m-tiles per expert; SegKT: prefix of the experts'
    // padded token ranges (units of two codes)
    for (int i = tid; i <= E; i += NT) {
      int c = 0;
      if (i < E) {
        const int n = P.offsets[i + 1] - P.offsets[i];
        c = (MODE == kSegM) ? (n + BM - 1) / BM
                            : (n + kMxPad - 1) / kMxPad * (kMxPad / 2);
      }
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
  }
  int split = 0;
  int ksplit_at = 0;    // SegM, two pieces: first k of the second piece
  if (MODE == kSegM) {
    // The grid holds an upper bound on the tile count (times two, rounded
    // to 16, with a split reduction) and only the first ids of each XCD
    // (the hardware deals ids round-robin over the 8 XCDs) carry a tile:
    // XCD x owns a contiguous range of the tiles, the same share for
    // every XCD, and the surplus ids exit at once.  A split reduction runs
    // the first pieces of all the XCD's tiles, then their second pieces,
    // whose length (split_second_steps) lets its CUs end together.
    const int total = s_pref[E] * P.ntn;
    int bid;
    if (P.ksplit == 1) {
      if (static_cast<int>(blockIdx.x) >= total) return;
      bid = xcd_remap(blockIdx.x, total);
    } else {
      const int q = total >> 3, r = total & 7;
      const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
      const int ntx = q + (x < r ? 1 : 0);
      if (i >= 2 * ntx) return;
      split = i >= ntx ? 1 : 0;
      bid = x * q + min(x, r) + i - split * ntx;
      const int nkf = (P.K + BK - 1) / BK;
      ksplit_at = (nkf - split_second_steps(ntx, nkf, P.xcd_cus)) * BK;
    }
    e = find_segment(s_pref, E, bid / P.ntn);
    const int mte = s_pref[e + 1] - s_pref[e];
    tile_order(bid - s_pref[e] * P.ntn, mte, P.ntn, &mt, &nt);
    seg0 = P.offsets[e];
    seg_len = P.offsets[e + 1] - P.offsets[e];
  } else {
    // A weight-gradient tile's depth is its expert's size (rows, or padded
    // token units), so with skewed routing the contiguous per-XCD tile
    // ranges would hand one XCD most of the work.  When the largest expert
    // is above twice the mean, experts are taken largest first (ties by
    // index) and tiles are dealt round-robin over the XCDs, in the order
    // the hardware hands out block ids; otherwise the L2-friendly
    // contiguous ranges stay.  Every workgroup reaches the same decision.
    const int mtiles = (P.M + BM - 1) / BM;
    const int per_e = mtiles * P.ntn;
    for (int i = tid; i < E; i += NT)
      s_cnt[i] = (MODE == kSegKT) ? s_pref[i + 1] - s_pref[i]
                                  : P.offsets[i + 1] - P.offsets[i];
    __syncthreads();
    if (tid < 64) {
      int mx = 0, sm = 0;
      for (int i = tid; i < E; i += 64) {
        mx = max(mx, s_cnt[i]);
        sm += s_cnt[i];
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        mx = max(mx, __shfl_xor(mx, m, 64));
        sm += __shfl_xor(sm, m, 64);
      }
      if (tid == 0) { s_stat[0] = mx; s_stat[1] = sm; }
    }
    __syncthreads();
    const bool skew = static_cast<int64_t>(s_stat[0]) * E >
                      2 * static_cast<int64_t>(s_stat[1]);
    if (skew) {
      for (int i = tid; i < E; i += NT) {
        const int ci = s_cnt[i];
        int r = 0;
        for (int j = 0; j < E; ++j) {
          const int cj = s_cnt[j];
          r += (cj > ci || (cj == ci && j < i)) ? 1 : 0;
        }
        s_ord[r] = i;
      }
      __syncthreads();
      const int t = blockIdx.x;
      e = s_ord[t / per_e];
      const int local = t - (t / per_e) * per_e;
      mt = local % mtiles;
      nt = local / mtiles;
    } else {
      const int bid = xcd_remap(blockIdx.x, gridDim.x);
      e = bid / per_e;
      tile_order(bid - e * per_e, mtiles, P.ntn, &mt, &nt);
    }
    seg0 = P.offsets[e];
    seg_len = P.offsets[e + 1] - P.offsets[e];
  }
  const int m0 = mt * BM;
  const int n0 = nt * BN;               // kSwiglu: gate column tile = nt*BN/2
  const int Mvalid = (MODE == kSegM) ? seg_len : P.M;
  // reduction range [kbeg, Kdim) of this workgroup
  const bool two = MODE == kSegM && P.ksplit == 2;
  const int kbeg = (MODE == kSegM)    ? (split ? min(P.K, ksplit_at) : 0)
                   : (MODE == kSegKT) ? s_pref[e]
                                      : 0;
  const int Kdim = (MODE == kSegM)    ? (two && !split ? min(P.K, ksplit_at)
                                                       : P.K)
                   : (MODE == kSegKT) ? s_pref[e + 1]
                                      : seg_len;

  // ---------------------------------------------------------- operands
  __amdgpu_buffer_rsrc_t rsA, rsB;
  // MX scale bytes (empty resources in the bf16 kernels)
  __amdgpu_buffer_rsrc_t rsSA = make_rsrc(P.sA, 0), rsSB = make_rsrc(P.sB, 0);
  // SegM: the A resource starts at the tile's first row and spans only the
  // expert's rows inside the tile (at most BM rows), so no tensor size
  // limits its 32-bit offsets; rows past the expert read as zero.
  const int a_row0 = (MODE == kSegM) ? 0 : m0;
  if (MODE == kSegM) {
    const int tile_rows = min(BM, seg_len - m0);
    const bf16_t* a = P.A + (seg0 + m0) * P.lda;
    const int64_t bytes = static_cast<int64_t>(tile_rows) * P.lda * 2;
    rsA = make_rsrc(a, static_cast<uint32_t>(bytes));
    const bf16_t* b = P.B + static_cast<int64_t>(e) * P.b_stride;
    // MX B may be a column range of a transposed weight: bound it by the
    // last byte the expert's rows reach
    const int64_t bbytes =
        MX ? ((static_cast<int64_t>(P.b_rows) - 1) * P.ldb + P.K) * 2
           : static_cast<int64_t>(P.b_rows) * P.ldb * 2;
    rsB = make_rsrc(b, static_cast<uint32_t>(bbytes));
    if (MX) {
      rsSA = make_rsrc(P.sA + (seg0 + m0) * P.lds_a,
                       static_cast<uint32_t>(tile_rows * P.lds_a));
      rsSB = make_rsrc(
          P.sB + static_cast<int64_t>(e) * P.bs_stride,
          static_cast<uint32_t>((static_cast<int64_t>(P.b_rows) - 1) *
                                    P.lds_b + P.K / 16));
    }
  } else if (MODE == kSegKT) {
    rsA = make_rsrc(P.A, static_cast<uint32_t>(P.M * P.lda * 2));
    rsB = make_rsrc(P.B, static_cast<uint32_t>(P.N * P.ldb * 2));
    rsSA = make_rsrc(P.sA, static_cast<uint32_t>(P.M * P.lds_a));
    rsSB = make_rsrc(P.sB, static_cast<uint32_t>(P.N * P.lds_b));
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
  auto blk_a = [&](int i) -> int64_t { return a_row0 + 32 * i; };
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
  ma.init(lt, P.lda, 0);
  mb.init(lt, P.ldb, 2 * kTileBytes);
  // with 8 waves and one layout for both operands, one mover serves either
  const __amdgpu_buffer_rsrc_t rs_own = mv_a ? rsA : rsB;
  const int64_t ld_own = mv_a ? P.lda : P.ldb;
  const int own_tile = mv_a ? 0 : 2 * kTileBytes;
  Mover<AKC> mown;
  mown.init(lt, ld_own, own_tile);

  f32x16 acc[BI][BJ];
#pragma unroll
  for (int i = 0; i < BI; ++i)
#pragma unroll
    for (int j = 0; j < BJ; ++j) acc[i][j] = f32x16{};

  const int fr = lane & 31;      // fragment row inside a 32-block
  const int fk = lane >> 5;      // which half of the fragment's k range

  // LDS tiles: [A stage 0][A stage 1][B stage 0][B stage 1]; stage st
  // of A starts at byte st * kTileBytes and of B 2 kTileBytes later.
  uint8_t* const smem8 = reinterpret_cast<uint8_t*>(smem);

  // Per-lane LDS byte offsets of the fragment reads, relative to a stage's
  // A tile; a stage, a 32-row block and (transposed) a k-slice add
  // constants, so that inside the unrolled K-loop every read address is
  // one of these registers plus an immediate.
  //  * K-contiguous: chunk 2 kk + fk of row fr of the wave's first block
  //    (swz is the same for rows 16 apart), kk = 0..3.
  //  * MN-contiguous: the frag_tr offset of each of the wave's blocks.
  int fa[4], fb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int c = lds_off(fr, 2 * kk + fk) * 2;
    fa[kk] = wm * TM * BK * 2 + c;
    fb[kk] = 2 * kTileBytes + wn * TN * BK * 2 + c;
  }
  const KmnLane kl(lane);
  int ta[BI], tb[BJ];
#pragma unroll
  for (int i = 0; i < BI; ++i)
    ta[i] = kl.base + (((wm * BI + i) ^ kl.R) << 6);
#pragma unroll
  for (int j = 0; j < BJ; ++j)
    tb[j] = 2 * kTileBytes + kl.base + (((wn * BJ + j) ^ kl.R) << 6);

  // bf16 fragments of k-slice kk (16 wide) of one LDS stage.
  auto read_frags = [&](int st, int kk, bf16x8_v* af, bf16x8_v* bf) {
    const uint8_t* s8 = smem8 + st * kTileBytes;
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      if constexpr (AKC)
        af[i] = __builtin_bit_cast(
            bf16x8_v,
            *reinterpret_cast<const i32x4*>(s8 + fa[kk] + i * kBlkBytes));
      else
        af[i] = frag_tr_at(s8, ta[i], kk);
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      if constexpr (BKC)
        bf[j] = __builtin_bit_cast(
            bf16x8_v,
            *reinterpret_cast<const i32x4*>(s8 + fb[kk] + j * kBlkBytes));
      else
        bf[j] = frag_tr_at(s8, tb[j], kk);
    }
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
  // part p of this thread's operand(s): global -> registers (full: a
  // std::bool_constant, see the movers), and registers -> LDS stage st
  auto gload = [&](int k0, int part, auto full) {
    constexpr bool kF = decltype(full)::value;
    if (C::kSplitLoad) {
      if constexpr (AKC)
        mown.template load<kF>(
            va, rs_own, ld_own, k0, Kdim,
            [&](int i) { return mv_a ? blk_a(i) : blk_b(i); }, part);
      else
        mown.template load<kF>(va, rs_own, ld_own, k0, Kdim, mv_a ? m0 : n0,
                               part);
    } else {
      load_one<AKC, kF>(ma, va, rsA, P.lda, k0, part, blk_a, m0, Kdim);
      load_one<BKC, kF>(mb, vb, rsB, P.ldb, k0, part, blk_b, n0, Kdim);
    }
  };
  auto lstore = [&](int st, int part) {
    if (C::kSplitLoad) {
      mown.store(va, smem8 + st * kTileBytes, part);
    } else {
      ma.store(va, smem8 + st * kTileBytes, part);
      mb.store(vb, smem8 + st * kTileBytes, part);
    }
  };
  // 8 waves with different layouts: each wave role gets its own copy of
  // the K-loop, so neither carries the other's mover state
  auto gload_a = [&](int k0, int part, auto full) {
    load_one<AKC, decltype(full)::value>(ma, va, rsA, P.lda, k0, part, blk_a,
                                         m0, Kdim);
  };
  auto lstore_a = [&](int st, int part) {
    ma.store(va, smem8 + st * kTileBytes, part);
  };
  auto gload_b = [&](int k0, int part, auto full) {
    load_one<BKC, decltype(full)::value>(mb, va, rsB, P.ldb, k0, part, blk_b,
                                         n0, Kdim);
  };
  auto lstore_b = [&](int st, int part) {
    mb.store(va, smem8 + st * kTileBytes, part);
  };

  // the iteration that prefetches the last stage when that stage ends
  // inside its tile (the reduction length is not a multiple of BK)
  const int kt_part = ((Kdim - kbeg) % BK != 0) ? nk - 3 : -1;

  // Software pipeline over k-steps of BK.  At iteration kt the mover
  // registers hold stage kt+1 (loaded one iteration earlier) and go to the
  // other LDS buffer in k-slices 0 and 1.  MFMA fragments are
  // double-buffered so the next slice's LDS reads overlap the current
  // slice's MFMAs.  Two schedules, by mover layout:
  //   * K-contiguous movers (each half of a stage has its own registers):
  //     right after half p of stage kt+1 is stored, the same registers are
  //     refilled with half p of stage kt+2, so a load has a whole
  //     iteration to land; the last slice's MFMAs are issued after the
  //     barrier, behind the first LDS reads of the next stage.
  //   * the other schedule (kept selectable): stage kt+2 is loaded in
  //     slices 2 and 3, after both stores, and the barrier follows the
  //     last MFMAs.
  // Both movers keep the halves of a stage in separate registers, so the
  // first schedule serves every layout.
  // Iterations run in pairs with the stage index a compile-time constant
  // (every LDS address an immediate off a per-lane register) and full
  // loads, then singly with a run-time stage and masked loads: the last
  // one when nk is odd, and, when the last stage ends inside the tile,
  // the iteration that prefetches it and those after (run_ksteps).  Loads
  // past K return zeros (masked) or data never read (full), and the one
  // stray store of the last iteration lands in the buffer no one reads
  // any more.
  auto kloop = [&](auto&& gload, auto&& lstore, auto indep_halves) {
    constexpr bool kIndep = decltype(indep_halves)::value;
    constexpr int kMf = BI * BJ;                   // MFMAs per k-slice
    // fragment reads per slice (a transposed fragment takes two), all
    // issued right after the slice's first MFMA: they have the rest of
    // the slice to land while the MFMAs run from registers (3% faster on
    // the Mixtral step than one read after each MFMA)
    constexpr int kRd = BI * (AKC ? 1 : 2) + BJ * (BKC ? 1 : 2);
    constexpr int kMv = C::kSplitLoad ? 4 : 8;     // moves per half stage
    const std::false_type masked{};
    bf16x8_v a0[BI], b0[BJ], a1[BI], b1[BJ];
    if (nk > 0) {
      gload(kbeg, 0, masked);
      gload(kbeg, 1, masked);
      lstore(0, 0);
      lstore(0, 1);
      gload(kbeg + BK, 0, masked);
      gload(kbeg + BK, 1, masked);
      __syncthreads();
      read_frags(0, 0, a0, b0);
    }
    auto step = [&](int kt, int cs, auto full) {
      const int ns = cs ^ 1;
      const int k2 = kbeg + (kt + 2) * BK;
      // slices 0 and 1: MFMAs; reads of the next slice; half p of stage
      // kt+1 to LDS (and, K-contiguous, half p of stage kt+2 loaded)
      read_frags(cs, 1, a1, b1);
      lstore(ns, 0);
      if constexpr (kIndep) gload(k2, 0, full);
      mfmas(a0, b0);
  #pragma unroll
      for (int i = 0; i < kMf; ++i) {
        sched_group(kSgMfma, 1);
        if (i == 0) sched_group(kSgDsRead, kRd);
        if (i < kMv) sched_group(kSgDsWrite, 1);
        if (kIndep && i < kMv) sched_group(kSgVmemRead, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // back to normal priority (raised after the barrier, below)
      __builtin_amdgcn_s_setprio(0);
      read_frags(cs, 2, a0, b0);
      lstore(ns, 1);
      if constexpr (kIndep) gload(k2, 1, full);
      mfmas(a1, b1);
  #pragma unroll
      for (int i = 0; i < kMf; ++i) {
        sched_group(kSgMfma, 1);
        if (i == 0) sched_group(kSgDsRead, kRd);
        if (i < kMv) sched_group(kSgDsWrite, 1);
        if (kIndep && i < kMv) sched_group(kSgVmemRead, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice 2: MFMAs on (a0,b0); reads of slice 3
      read_frags(cs, 3, a1, b1);
      if constexpr (!kIndep) gload(k2, 0, full);
      mfmas(a0, b0);
  #pragma unroll
      for (int i = 0; i < kMf; ++i) {
        sched_group(kSgMfma, 1);
        if (i == 0) sched_group(kSgDsRead, kRd);
        if (!kIndep && i < kMv) sched_group(kSgVmemRead, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kIndep) {
        // slice 3 after the barrier: stage kt+1 is complete, its first
        // fragments are read while slice 3's MFMAs run from registers
        __syncthreads();
        // raised wave priority from the barrier to the end of the next
        // step's slice 0 (1% faster on the Mixtral step; a window of
        // slice 3 alone was 3% slower, and the MX loop got 5% slower)
        __builtin_amdgcn_s_setprio(1);
        read_frags(ns, 0, a0, b0);
        mfmas(a1, b1);
  #pragma unroll
        for (int i = 0; i < kMf; ++i) {
          sched_group(kSgMfma, 1);
          if (i == 0) sched_group(kSgDsRead, kRd);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // slice 3: MFMAs on (a1,b1); second half of stage kt+2
        gload(k2, 1, full);
        mfmas(a1, b1);
  #pragma unroll
        for (int i = 0; i < kMf; ++i) {
          sched_group(kSgMfma, 1);
          if (i < kMv) sched_group(kSgVmemRead, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        read_frags(ns, 0, a0, b0);
      }
    };
    run_ksteps(nk, kt_part, step);
    __builtin_amdgcn_s_setprio(0);
  };

  // MX K-loop: two 64-code k-slices per stage.  The stage's movers work
  // as in the bf16 loop (stores of stage kt+1 in slice 0, loads of stage
  // kt+2 in slice 1); with part 0 each mover thread also moves the scale
  // dword (4 blocks of 32 codes) of its own tile row into the stage's scale
  // area of LDS.  After the barrier each lane reads the dwords of its
  // fragment rows and shifts them by its lane half: lanes 0-31 supply the
  // scale of the slice's first block and lanes 32-63 that of its second,
  // i.e. block 2 kk + fk, which is byte 2 kk of the shifted dword (the
  // MFMA's opsel).  Fragments are
  // read right before the MFMAs that use them; with 8 waves (two a SIMD)
  // only half of the wave's A fragments are held at a time, and each
  // wave's LDS waits are covered by the other wave of its SIMD.
  // role4: this wave moves an E2M1 operand (compile-time, so each role's
  // copy of the loop carries only its own mover)
  auto kloop_mx = [&](auto role4) {
    constexpr bool kRole4 = decltype(role4)::value;
    constexpr int kHalves = (C::kWaves == 4) ? 1 : 2;
    constexpr int kAH = BI / kHalves;             // A fragments held at once
    constexpr int kMfH = kAH * BJ;                // MFMAs per half-slice
    constexpr int kMv = C::kSplitLoad ? 4 : 8;    // moves per part
    const uint32_t srow_a = static_cast<uint32_t>((a_row0 + lt) * P.lds_a);
    const uint32_t srow_b =
        static_cast<uint32_t>((blk_b(lt >> 5) + (lt & 31)) * P.lds_b);
    // scale dwords (4 blocks of 32 codes, one stage) of the thread's tile
    // row for kScaleGroup consecutive stages, loaded together once a
    // group: a 16-byte load per 4 stages instead of four 4-byte ones, each
    // of which touches a cache line of its own for every lane.  A group that runs
    // past the end of the resource reads zeros there (the range check is
    // per dword) and those stages are never stored.
    constexpr int kSg4 = kScaleGroup / 4;    // 16-byte loads a group
    i32x4 vsg[kSg4] = {}, vsgb[kSg4] = {};
    // an E2M1 operand has its own mover (half the bytes a stage)
    Mover4 m4;
    if constexpr (kRole4) m4.init(lt, ld_own, own_tile);
    auto gload_ops = [&](int k0, int part, auto full) {
      if constexpr (kRole4) {
        auto blk = [&](int i) { return mv_a ? blk_a(i) : blk_b(i); };
        m4.template load<decltype(full)::value>(va, rs_own, k0, Kdim, blk,
                                                part);
      } else {
        gload(k0, part, full);
      }
    };
    auto lstore_ops = [&](int st, int part) {
      if constexpr (kRole4)
        m4.store(va, smem8 + st * kTileBytes, part);
      else
        lstore(st, part);
    };
    // qs: the loaded stage's index mod kScaleGroup (its place in its
    // scale group)
    auto gload_mx = [&](int k0, int part, auto full, int qs) {
      gload_ops(k0, part, full);
      if (part == 0 && qs == 0) {
        const bool ok = k0 < Kdim;
#pragma unroll
        for (int g = 0; g < kSg4; ++g) {
          const uint32_t kb =
              static_cast<uint32_t>(k0 >> 4) + 16u * g;      // 32-blocks
          if constexpr (decltype(full)::value) {
            const uint32_t ks = ok ? kb : 16u * g;
            if (C::kSplitLoad) {
              vsg[g] = mv_a ? buf_load16(rsSA, srow_a, ks)
                            : buf_load16(rsSB, srow_b, ks);
            } else {
              vsg[g] = buf_load16(rsSA, srow_a, ks);
              vsgb[g] = buf_load16(rsSB, srow_b, ks);
            }
          } else if (C::kSplitLoad) {
            vsg[g] = mv_a ? buf_load16(rsSA, ok ? srow_a + kb : kOob)
                          : buf_load16(rsSB, ok ? srow_b + kb : kOob);
          } else {
            vsg[g] = buf_load16(rsSA, ok ? srow_a + kb : kOob);
            vsgb[g] = buf_load16(rsSB, ok ? srow_b + kb : kOob);
          }
        }
      }
    };
    // qs: the stored stage's index mod kScaleGroup
    auto lstore_mx = [&](int st, int part, int qs) {
      lstore_ops(st, part);
      if (part == 0) {
        uint32_t* sc = s_scl + st * (2 * BM);
        if (C::kSplitLoad) {
          sc[(mv_a ? 0 : BM) + lt] =
              static_cast<uint32_t>(vsg[qs >> 2][qs & 3]);
        } else {
          sc[lt] = static_cast<uint32_t>(vsg[qs >> 2][qs & 3]);
          sc[BM + lt] = static_cast<uint32_t>(vsgb[qs >> 2][qs & 3]);
        }
      }
    };
    auto read_scales = [&](int st, uint32_t* sa, uint32_t* sb) {
      const uint32_t* sc = s_scl + st * (2 * BM);
#pragma unroll
      for (int i = 0; i < BI; ++i)
        sa[i] = sc[wm * TM + i * 32 + fr] >> (8 * fk);
#pragma unroll
      for (int j = 0; j < BJ; ++j)
        sb[j] = sc[BM + wn * TN + j * 32 + fr] >> (8 * fk);
    };
    // The lane's 32 codes of k-slice kk (codes 64 kk .. 64 kk + 63 of the
    // stage, scale blocks 2 kk and 2 kk + 1) of a tile row.  The block-
    // scaled MFMA takes bytes 0-15 of every lane from the first 32-block
    // (scaled by the byte that lanes 0-31 supply) and bytes 16-31 from the
    // second (scaled by lanes 32-63), so lane half fk holds 16 codes of each
    // block: chunks 4 kk + fk and 4 kk + 2 + fk.
    // Chunks 4 kk + fk and 4 kk + 2 + fk are the bf16 loop's chunk pairs
    // 2 kk and 2 kk + 1 (offsets fa, fb).
    auto frag = [&](int st, const int* fo, int blk, int kk) {
      const uint8_t* p = smem8 + st * kTileBytes + blk * kBlkBytes;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(p + fo[2 * kk]);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(p + fo[2 * kk + 1]);
      return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto read_a = [&](int st, int kk, int h, i32x8* af) {
#pragma unroll
      for (int i = 0; i < kAH; ++i) af[i] = frag(st, fa, h * kAH + i, kk);
    };
    auto read_b = [&](int st, int kk, i32x8* bf) {
#pragma unroll
      for (int j = 0; j < BJ; ++j) bf[j] = frag(st, fb, j, kk);
    };
    i32x8 af[kAH], bf[BJ];
    uint32_t sa[BI], sb[BJ];
    const std::false_type masked{};
    if (nk > 0) {
      gload_mx(kbeg, 0, masked, 0);
      gload_mx(kbeg, 1, masked, 0);
      lstore_mx(0, 0, 0);
      lstore_mx(0, 1, 0);
      gload_mx(kbeg + BK, 0, masked, 1);
      gload_mx(kbeg + BK, 1, masked, 1);
      __syncthreads();
      read_b(0, 0, bf);
      read_a(0, 0, 0, af);
      read_scales(0, sa, sb);
    }
    // q: kt mod kScaleGroup (a compile-time constant in the unrolled
    // groups)
    auto step = [&](int kt, int cs, auto full, int q) {
      const int ns = cs ^ 1;
      const int k2 = kbeg + (kt + 2) * BK;
      const int q1 = (q + 1) & (kScaleGroup - 1);
      const int q2 = (q + 2) & (kScaleGroup - 1);
      // slice 0 (fragments of half 0 already read): stores of stage kt+1
      if constexpr (kHalves == 1) {
        lstore_mx(ns, 0, q1);
        lstore_mx(ns, 1, q1);
        mx_mfmas<0, 0, kAH>(acc, af, bf, sa, sb);
#pragma unroll
        for (int i = 0; i < kMfH; ++i) {
          sched_group(kSgMfma, 1);
          if (i < 2 * kMv + 2) sched_group(kSgDsWrite, 1);
        }
      } else {
        // with 8 waves, half p of stage kt+2 is loaded right after half p
        // of stage kt+1 leaves the same registers for LDS, so the loads
        // have a whole step to land
        lstore_mx(ns, 0, q1);
        gload_mx(k2, 0, full, q2);
        mx_mfmas<0, 0, kAH>(acc, af, bf, sa, sb);
#pragma unroll
        for (int i = 0; i < kMfH; ++i) {
          sched_group(kSgMfma, 1);
          if (i < kMv + 1) sched_group(kSgDsWrite, 1);
          if (i < kMv + 1) sched_group(kSgVmemRead, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        read_a(cs, 0, 1, af);
        lstore_mx(ns, 1, q1);
        gload_mx(k2, 1, full, q2);
        mx_mfmas<0, kAH, kAH>(acc, af, bf, sa, sb);
        sched_group(kSgDsRead, 2 * kAH);
#pragma unroll
        for (int i = 0; i < kMfH; ++i) {
          sched_group(kSgMfma, 1);
          if (i < kMv) sched_group(kSgDsWrite, 1);
          if (i < kMv) sched_group(kSgVmemRead, 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // slice 1 (4 waves: loads of stage kt+2)
      read_b(cs, 1, bf);
      read_a(cs, 1, 0, af);
      if constexpr (kHalves == 1) gload_mx(k2, 0, full, q2);
      mx_mfmas<2, 0, kAH>(acc, af, bf, sa, sb);
      sched_group(kSgDsRead, 2 * (kAH + BJ));
#pragma unroll
      for (int i = 0; i < kMfH; ++i) {
        sched_group(kSgMfma, 1);
        if (kHalves == 1 && i < kMv + 1) sched_group(kSgVmemRead, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kHalves == 2) {
        read_a(cs, 1, 1, af);
        mx_mfmas<2, kAH, kAH>(acc, af, bf, sa, sb);
        sched_group(kSgDsRead, 2 * kAH);
#pragma unroll
        for (int i = 0; i < kMfH; ++i) sched_group(kSgMfma, 1);
      } else {
        gload_mx(k2, 1, full, q2);
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      read_b(ns, 0, bf);
      read_a(ns, 0, 0, af);
      read_scales(ns, sa, sb);
    };
    run_ksteps_g<kScaleGroup>(nk, kt_part, step);
  };

  if constexpr (MX) {
    // with an E2M1 operand the waves that move it run their own loop copy
    const bool own4 =
        (FMT != 0) && (mv_a ? (FMT & 1) != 0 : (FMT & 2) != 0);
    if constexpr (FMT != 0) {
      if (own4) kloop_mx(std::true_type{});
      else kloop_mx(std::false_type{});
    } else {
      kloop_mx(std::false_type{});
    }
  } else if constexpr (C::kSplitLoad && AKC != BKC) {
    if (mv_a) kloop(gload_a, lstore_a, std::bool_constant<kIndepLoop>{});
    else kloop(gload_b, lstore_b, std::bool_constant<kIndepLoop>{});
  } else {
    kloop(gload, lstore, std::bool_constant<kIndepLoop>{});
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
  // Token-axis MX output: each wave's TM = 128 rows are one 128-row unit
  // of the padded layout (four 32-row blocks, two per pass), so a wave
  // writes whole 128-byte code lines and one scale dword per column.
  constexpr bool kTokEpi = MX && (EPI == kSwiglu || EPI == kDSwiglu) &&
                           TM == kMxPad && TN == 64;
  const bool tok = kTokEpi && P.Tc != nullptr;
  int64_t pe = 0;                                  // padded start of e
  const int pad_len = (seg_len + kMxPad - 1) / kMxPad * kMxPad;
  const int wrow0 = m0 + wm * TM;                  // wave's first row in e
  uint32_t tsc[2] = {0u, 0u};                      // scale bytes, 4 blocks
  if (tok) {
    int acc_p = 0;
    for (int i = lane; i < e; i += 64) {
      const int n = P.offsets[i + 1] - P.offsets[i];
      acc_p += (n + kMxPad - 1) / kMxPad * kMxPad;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) acc_p += __shfl_xor(acc_p, m, 64);
    pe = acc_p;
  }
  // kDSwiglu: a lane's rows of a pass are r0 + it * kRowsPerPass.  The AB
  // values of a pass are all read ahead: pass 0's before the barrier below,
  // pass h + 1's right after pass h's accumulators are staged (their
  // registers are free then), so each read has a whole pass to land.  The
  // tile's routing weights go to LDS once (a global read between two dAB
  // stores would wait for them: the compiler cannot tell the two apart).
  constexpr int kDsIt = kEpiRows / kRowsPerPass;
  constexpr int kPre = EPI == kDSwiglu ? kDsIt : 1;
  constexpr int kPasses = TM / kEpiRows;
  uint2 pre_g[kPasses][kPre], pre_u[kPasses][kPre];
  auto load_ab = [&](int h) {
    if constexpr (EPI == kDSwiglu) {
      const int row_base = m0 + wm * TM + h * kEpiRows;
      const bf16_t* AB = P.AB + seg0 * static_cast<int64_t>(2 * f);
      const int col = n0 + wn * TN + (lane % kLanesPerRow) * 4;
#pragma unroll
      for (int it = 0; it < kDsIt; ++it) {
        const int row = row_base + lane / kLanesPerRow + it * kRowsPerPass;
        pre_g[h][it] = make_uint2(0u, 0u);
        pre_u[h][it] = make_uint2(0u, 0u);
        if (row < Mvalid && col < f) {
          const bf16_t* src = AB + static_cast<int64_t>(row) * 2 * f + col;
          pre_g[h][it] = *reinterpret_cast<const uint2*>(src);
          pre_u[h][it] = *reinterpret_cast<const uint2*>(src + f);
        }
      }
    }
  };
  if constexpr (EPI == kDSwiglu) {
    load_ab(0);
    for (int lr = tid; lr < BM; lr += NT)
      s_wrow[lr] = (w && m0 + lr < Mvalid) ? w[m0 + lr] : 1.0f;
    __syncthreads();
  }
  // The passes are expanded at compile time (h indexes the accumulators;
  // the unroller declines bodies this large).
  auto epi_pass = [&](auto h_c) {
    constexpr int h = decltype(h_c)::value;
    const int row_base = m0 + wm * TM + h * kEpiRows;   // absolute row
#pragma unroll
    for (int ii = 0; ii < kEpiRows / 32; ++ii)
#pragma unroll
      for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = ii * 32 + (v >> 2) * 8 + fk * 4 + (v & 3);
          stage[r * LD + j * 32 + fr] = acc[h * (kEpiRows / 32) + ii][j][v];
        }
    wave_lds_sync();
    if (h + 1 < kPasses) load_ab(h + 1);
    if (EPI == kStore || EPI == kStoreF32) {
      const int c4 = (lane % kLanesPerRow) * 4;
      const int col = n0 + wn * TN + c4;
      // unrolled, so the stage reads of all rows are in flight together
#pragma unroll
      for (int it = 0; it < kEpiRows / kRowsPerPass; ++it) {
        const int r = lane / kLanesPerRow + it * kRowsPerPass;
        const int row = row_base + r;
        const f32x4 x = *reinterpret_cast<const f32x4*>(stage + r * LD + c4);
        if (row < Mvalid && col < P.N) {
          const int64_t o = cbase + static_cast<int64_t>(row) * P.ldc + col;
          if (EPI == kStoreF32) {
            *reinterpret_cast<f32x4*>(P.Cf + split * P.plane + o) = x;
          } else {
            uint2 u;
            u.x = pack_bf16x2(x[0], x[1]);
            u.y = pack_bf16x2(x[2], x[3]);
            st_epi<MX>(reinterpret_cast<uint2*>(P.C + o), u);
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
      // routing weights of the pass read up front; rows unrolled so the
      // stage reads overlap
      constexpr int kItG = kEpiRows / kRowsG;
      float pre_wr[kItG];
#pragma unroll
      for (int it = 0; it < kItG; ++it) {
        const int row = row_base + lane / kLanesG + it * kRowsG;
        pre_wr[it] = (w && row < Mvalid && col < f) ? w[row] : 1.0f;
      }
      // Unchecked: every row of the pass and every gate column of the wave
      // is inside the expert, so no lane needs a mask.
      auto sw_iter = [&](int it, auto checked_c) {
        constexpr bool kChecked = decltype(checked_c)::value;
        const int r = lane / kLanesG + it * kRowsG;
        const int row = row_base + r;
        const bool ok = !kChecked || (row < Mvalid && col < f);
        const int64_t ro = static_cast<int64_t>(row);
        const f32x4 g = *reinterpret_cast<const f32x4*>(stage + r * LD + c4);
        const f32x4 u =
            *reinterpret_cast<const f32x4*>(stage + r * LD + TN / 2 + c4);
        const float wr = pre_wr[it];
        float sv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sv[c] = wr * (g[c] * sigmoidf_(g[c]) * u[c]);
        if constexpr (MX) {
          // S along f: one 32-column block per 8 lanes of the row
          uint32_t sbyte;
          const uint32_t q = mx_quant4(sv, ok, &sbyte);
          if (ok) {
            const int64_t qr = (seg0 + ro) * f;
            st_epi<MX>(reinterpret_cast<uint32_t*>(P.Qc + qr + col), q);
            if ((lane & 7) == 0)
              P.Qs[qr / kMxBlock + col / kMxBlock] =
                  static_cast<uint8_t>(sbyte);
          }
        }
        uint2 os;
        os.x = pack_bf16x2(sv[0], sv[1]); os.y = pack_bf16x2(sv[2], sv[3]);
        if (ok) {
          uint2 og, ou;
          og.x = pack_bf16x2(g[0], g[1]); og.y = pack_bf16x2(g[2], g[3]);
          ou.x = pack_bf16x2(u[0], u[1]); ou.y = pack_bf16x2(u[2], u[3]);
          st_epi<MX>(reinterpret_cast<uint2*>(AB + ro * P.ldc + col), og);
          st_epi<MX>(reinterpret_cast<uint2*>(AB + ro * P.ldc + f + col), ou);
          if (P.S) st_epi<MX>(reinterpret_cast<uint2*>(S + ro * f + col), os);
        }
        if constexpr (kTokEpi) {
          // the bf16 S values go back over this row's gate slots for the
          // token-axis pass (zero past the expert's rows)
          if (tok) {
            f32x4 sb;
            sb[0] = ok ? bf_lo(os.x) : 0.0f; sb[1] = ok ? bf_hi(os.x) : 0.0f;
            sb[2] = ok ? bf_lo(os.y) : 0.0f; sb[3] = ok ? bf_hi(os.y) : 0.0f;
            *reinterpret_cast<f32x4*>(stage + r * LD + c4) = sb;
          }
        }
      };
      const bool full = row_base + kEpiRows <= Mvalid &&
                        n0g + wn * (TN / 2) + TN / 2 <= f;
      if (full) {
#pragma unroll
        for (int it = 0; it < kItG; ++it) sw_iter(it, std::false_type{});
      } else {
#pragma unroll
        for (int it = 0; it < kItG; ++it) sw_iter(it, std::true_type{});
      }
      if constexpr (kTokEpi) {
        if (tok) {
          // lane = (32-row block cb of this pass, S column cc of the wave)
          wave_lds_sync();
          const int cb = lane >> 5, cc = lane & 31;
          float v[kMxBlock];
          float amax = 0.0f;
#pragma unroll
          for (int i = 0; i < kMxBlock; ++i) {
            v[i] = stage[(cb * kMxBlock + i) * LD + cc];
            amax = fmaxf(amax, fabsf(v[i]));
          }
          const int ex = mx_scale_exp(amax);
          const float inv = mx_inv_scale(ex);
          i32x4 q[2];
#pragma unroll
          for (int k4 = 0; k4 < 8; ++k4)
            q[k4 >> 2][k4 & 3] = static_cast<int>(
                e4m3_pack4(v[k4 * 4] * inv, v[k4 * 4 + 1] * inv,
                           v[k4 * 4 + 2] * inv, v[k4 * 4 + 3] * inv));
          const int trow = wrow0 + h * kEpiRows + cb * kMxBlock;
          if (trow < pad_len) {
            uint8_t* dst = P.Tc +
                static_cast<int64_t>(n0g + wn * (TN / 2) + cc) * P.ldt + pe +
                trow;
            st_epi<MX>(reinterpret_cast<i32x4*>(dst), q[0]);
            st_epi<MX>(reinterpret_cast<i32x4*>(dst + 16), q[1]);
          }
          tsc[0] |= static_cast<uint32_t>(ex + 127) << (8 * (2 * h + cb));
        }
      }
    } else {  // kDSwiglu
      bf16_t* dAB = P.C + cbase;
      const int c4 = (lane % kLanesPerRow) * 4;
      const int col = n0 + wn * TN + c4;
      // the lane's first row of the pass; row it is rstep elements on
      const int r0 = lane / kLanesPerRow;
      const int64_t rstep = static_cast<int64_t>(kRowsPerPass) * P.ldc;
      bf16_t* drow = dAB + static_cast<int64_t>(row_base + r0) * P.ldc + col;
      const int64_t qstep = static_cast<int64_t>(kRowsPerPass) * (2 * f);
      const int64_t qrow = (seg0 + row_base + r0) * (2 * f);
      // One row of the pass (it) for this lane: dSwiGLU of its 4 columns,
      // the stores, and the row's share of the routing-weight gradient.
      // Unchecked: every row of the pass and every column of the wave is
      // inside the expert, so no lane needs a mask.
      auto ds_iter = [&](int it, auto checked_c) {
        constexpr bool kChecked = decltype(checked_c)::value;
        const int r = r0 + it * kRowsPerPass;
        const int row = row_base + r;
        float part = 0.0f;
        const bool ok = !kChecked || (row < Mvalid && col < f);
        float dg[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float du[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (ok) {
          const f32x4 ds = *reinterpret_cast<const f32x4*>(stage + r * LD + c4);
          const uint2 gb = pre_g[h][it], ub = pre_u[h][it];
          const float g[4] = {bf_lo(gb.x), bf_hi(gb.x), bf_lo(gb.y),
                              bf_hi(gb.y)};
          const float u[4] = {bf_lo(ub.x), bf_hi(ub.x), bf_lo(ub.y),
                              bf_hi(ub.y)};
          const float wr = s_wrow[row - m0];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float sg = sigmoidf_(g[c]);
            const float sl = g[c] * sg;
            part += ds[c] * (sl * u[c]);
            const float dh = wr * ds[c];
            dg[c] = dh * u[c] * sg * (1.0f + g[c] * (1.0f - sg));
            du[c] = dh * sl;
          }
          if (P.C) {
            uint2 og, ou;
            og.x = pack_bf16x2(dg[0], dg[1]); og.y = pack_bf16x2(dg[2], dg[3]);
            ou.x = pack_bf16x2(du[0], du[1]); ou.y = pack_bf16x2(du[2], du[3]);
            bf16_t* dst = drow + it * rstep;
            *reinterpret_cast<uint2*>(dst) = og;
            *reinterpret_cast<uint2*>(dst + f) = ou;
          }
        }
        if constexpr (kTokEpi) {
          // (bf16 dA_g, bf16 dA_u) pairs go back over this row's dS slots
          // for the token-axis pass (zero past the expert's rows)
          if (tok) {
            i32x4 pk;
#pragma unroll
            for (int c = 0; c < 4; ++c)
              pk[c] = static_cast<int>(pack_bf16x2(dg[c], du[c]));
            *reinterpret_cast<i32x4*>(stage + r * LD + c4) = pk;
          }
        }
        if constexpr (MX) {
          // dAB along 2f: gate and up blocks of 32 columns, 8 lanes each
          uint32_t sg_byte, su_byte;
          const uint32_t qg = mx_quant4(dg, ok, &sg_byte);
          const uint32_t qu = mx_quant4(du, ok, &su_byte);
          if (ok) {
            const int64_t qr = qrow + it * qstep;
            *reinterpret_cast<uint32_t*>(P.Qc + qr + col) = qg;
            *reinterpret_cast<uint32_t*>(P.Qc + qr + f + col) = qu;
            if ((lane & 7) == 0) {
              uint8_t* srow = P.Qs + qr / kMxBlock;
              srow[col / kMxBlock] = static_cast<uint8_t>(sg_byte);
              srow[(f + col) / kMxBlock] = static_cast<uint8_t>(su_byte);
            }
          }
        }
        // row sum over the lanes of this row, fixed order
        if constexpr (kLanesPerRow <= 16) {
          part = dpp_group_sum<kLanesPerRow>(part);
        } else {
          part = dpp_group_sum<16>(part);
#pragma unroll
          for (int m = 16; m < kLanesPerRow; m <<= 1)
            part += __shfl_xor(part, m, 64);
        }
        if ((lane % kLanesPerRow) == 0)
          s_dp[wn * BM + wm * TM + h * kEpiRows + r] = part;
      };
      const bool full = row_base + kEpiRows <= Mvalid &&
                        n0 + wn * TN + TN <= f;
      if (full) {
#pragma unroll
        for (int it = 0; it < kDsIt; ++it) ds_iter(it, std::false_type{});
      } else {
#pragma unroll
        for (int it = 0; it < kDsIt; ++it) ds_iter(it, std::true_type{});
      }
      if constexpr (kTokEpi) {
        if (tok) {
          // lane = dS column of the wave; both 32-row blocks of the pass,
          // gate (low half) and up (high half) of the packed pairs.  The
          // codes go out through the wave's LDS region: lane c leaves its
          // column's 64 codes of the pass (four 16-byte chunks, gate at
          // byte 0, up at 4096, chunk k of column c in slot (k + c/4) % 4 of
          // the column's 64 bytes, so that 16 lanes of a write hit 64
          // distinct banks), then four lanes write each column's 64-byte
          // run: 16 runs a store instead of 64 pieces of 16 bytes.
          wave_lds_sync();
          const uint32_t* st32 = reinterpret_cast<const uint32_t*>(stage);
          uint8_t* gb = reinterpret_cast<uint8_t*>(stage);
          auto slot = [](int c, int k) { return ((k + (c >> 2)) & 3) * 16; };
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            uint32_t pk[kMxBlock];
            float ag = 0.0f, au = 0.0f;
#pragma unroll
            for (int i = 0; i < kMxBlock; ++i) {
              pk[i] = st32[(cb * kMxBlock + i) * LD + lane];
              ag = fmaxf(ag, fabsf(bf_lo(pk[i])));
              au = fmaxf(au, fabsf(bf_hi(pk[i])));
            }
            const int eg = mx_scale_exp(ag), eu = mx_scale_exp(au);
            const float ig = mx_inv_scale(eg), iu = mx_inv_scale(eu);
            i32x4 qg[2], qu[2];
#pragma unroll
            for (int k4 = 0; k4 < 8; ++k4) {
              const uint32_t* p4 = pk + k4 * 4;
              qg[k4 >> 2][k4 & 3] = static_cast<int>(e4m3_pack4(
                  bf_lo(p4[0]) * ig, bf_lo(p4[1]) * ig, bf_lo(p4[2]) * ig,
                  bf_lo(p4[3]) * ig));
              qu[k4 >> 2][k4 & 3] = static_cast<int>(e4m3_pack4(
                  bf_hi(p4[0]) * iu, bf_hi(p4[1]) * iu, bf_hi(p4[2]) * iu,
                  bf_hi(p4[3]) * iu));
            }
            // rows 0-31 of the region (block 0's pairs) are read by every
            // lane before block 0's codes overwrite its first 8 KB; block
            // 1 reads rows 32-63, past them
            if (cb == 0) wave_lds_sync();
            uint8_t* gc = gb + lane * 64;
            *reinterpret_cast<i32x4*>(gc + slot(lane, 2 * cb)) = qg[0];
            *reinterpret_cast<i32x4*>(gc + slot(lane, 2 * cb + 1)) = qg[1];
            *reinterpret_cast<i32x4*>(gc + 4096 + slot(lane, 2 * cb)) = qu[0];
            *reinterpret_cast<i32x4*>(gc + 4096 + slot(lane, 2 * cb + 1)) =
                qu[1];
            tsc[0] |= static_cast<uint32_t>(eg + 127) << (8 * (2 * h + cb));
            tsc[1] |= static_cast<uint32_t>(eu + 127) << (8 * (2 * h + cb));
          }
          wave_lds_sync();
          // wrow0 and pad_len are multiples of 128: the pass is all in or
          // all out
          if (wrow0 < pad_len) {
            const int j = lane & 3;
#pragma unroll
            for (int sg = 0; sg < 4; ++sg) {
              const int c = 16 * sg + (lane >> 2);
              const i32x4 vg =
                  *reinterpret_cast<const i32x4*>(gb + c * 64 + slot(c, j));
              const i32x4 vu = *reinterpret_cast<const i32x4*>(
                  gb + 4096 + c * 64 + slot(c, j));
              const int col = n0 + wn * TN + c;
              if (col < f) {
                uint8_t* dg_dst = P.Tc + static_cast<int64_t>(col) * P.ldt +
                                  pe + wrow0 + h * kEpiRows + 16 * j;
                *reinterpret_cast<i32x4*>(dg_dst) = vg;
                *reinterpret_cast<i32x4*>(
                    dg_dst + static_cast<int64_t>(f) * P.ldt) = vu;
              }
            }
          }
        }
      }
    }
    wave_lds_sync();
  };
  static_assert(kPasses == 2, "two epilogue passes of 64 rows");
  epi_pass(std::integral_constant<int, 0>{});
  epi_pass(std::integral_constant<int, 1>{});
  if constexpr (kTokEpi) {
    // one scale dword (the wave's four 32-row blocks) per column
    if (tok && wrow0 < pad_len) {
      const int64_t so = (pe + wrow0) / kMxBlock;
      const int64_t lds_t = P.ldt / kMxBlock;
      if (EPI == kSwiglu) {
        // lanes 0-31 hold blocks 0 and 2, lanes 32-63 blocks 1 and 3
        const uint32_t word = tsc[0] | __shfl(tsc[0], (lane & 31) + 32, 64);
        if (lane < 32) {
          const int col = n0g + wn * (TN / 2) + lane;
          *reinterpret_cast<uint32_t*>(P.Ts + col * lds_t + so) = word;
        }
      } else {
        const int col = n0 + wn * TN + lane;
        if (col < f) {
          *reinterpret_cast<uint32_t*>(P.Ts + col * lds_t + so) = tsc[0];
          *reinterpret_cast<uint32_t*>(P.Ts + (f + col) * lds_t + so) =
              tsc[1];
        }
      }
    }
  }
  if (EPI == kDSwiglu) {
    // the tile's column groups, added in order (wn = 0, 1, ...): the one
    // read of other waves' LDS in the epilogue
    __syncthreads();
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
#ifndef MOE_MX_WAVES
#define MOE_MX_WAVES 8
#endif
using CfgMx = std::conditional_t<MOE_MX_WAVES == 4, Cfg4, Cfg8>;

// Compute units of one XCD of the current device (8 XCDs), read once a
// device.
int xcd_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 32;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess || cus < 8)
      cus = 256;
    cached[dev] = cus / 8;
  }
  return cached[dev];
}

template <class C, int MODE, bool AKC, bool BKC, int EPI, bool MX = false,
          int FMT = 0>
hipError_t launch(Params P, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (P.ksplit != 2) P.ksplit = 1;
  // two pieces a tile: every XCD needs twice its share of ids
  if (P.ksplit == 2) grid = 16 * ((grid + 7) / 8);
  P.xcd_cus = xcd_cus();
  hipLaunchKernelGGL((grouped_gemm_kernel<C, MODE, AKC, BKC, EPI, MX, FMT>),
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
  P.ksplit = out_planes(f); P.plane = Tk * d;
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
  P.ksplit = out_planes(f); P.plane = Tk * d;
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

// ------------------------------------------------------------------ MXFP8
// Operands are E4M3 codes with one E8M0 byte per 32 codes along K; the
// kernel addresses codes in pairs, so leading dimensions and K are halved.

// The token-axis epilogue output needs waves of 128 rows x 64 columns.
constexpr bool kMxTokEpi = CfgMx::TM == kMxPad && CfgMx::TN == 64;

// fc1 forward: AB = Xp . W_gu^T, S = w*silu(g)*u as bf16 (s, optional),
// as MX codes along f (the down GEMM's A) and, optionally, as MX codes
// along each expert's tokens from its bf16 value (the dW2 GEMM's B)
hipError_t gemm_mx_fc1_fwd(const uint8_t* xq, const uint8_t* xs, bool x_fp4,
                           const uint8_t* wq, const uint8_t* ws,
                           const int32_t* offsets, int E, int64_t Tk,
                           int64_t d, int64_t f, const float* w_perm,
                           bf16_t* ab, bf16_t* s, uint8_t* sq, uint8_t* ss,
                           uint8_t* s_tok, uint8_t* s_tok_scales, int64_t ldt,
                           hipStream_t st) {
  if (s_tok && !kMxTokEpi) return hipErrorInvalidValue;
  if (x_fp4 && !CfgMx::kSplitLoad) return hipErrorInvalidValue;
  Params P{};
  // lda in 2-byte units: E4M3 rows of d codes, or E2M1 rows of d/2 bytes
  P.A = reinterpret_cast<const bf16_t*>(xq); P.lda = x_fp4 ? d / 4 : d / 2;
  P.sA = xs; P.lds_a = d / kMxBlock;
  P.B = reinterpret_cast<const bf16_t*>(wq); P.ldb = d / 2;
  P.b_stride = f * d; P.b_rows = 2 * f;
  P.sB = ws; P.lds_b = d / kMxBlock; P.bs_stride = 2 * f * d / kMxBlock;
  P.C = ab; P.ldc = 2 * f;
  P.offsets = offsets; P.E = E; P.Tk = Tk;
  P.N = f; P.K = d / 2; P.f = f;
  P.ntn = static_cast<int>((f + BN / 2 - 1) / (BN / 2));
  P.w = w_perm; P.S = s; P.Qc = sq; P.Qs = ss;
  P.Tc = s_tok; P.Ts = s_tok_scales; P.ldt = ldt;
  if (x_fp4)
    return launch<CfgMx, kSegM, true, true, kSwiglu, true, 1>(
        P, segm_grid(Tk, E, P.ntn), st);
  return launch<CfgMx, kSegM, true, true, kSwiglu, true>(
      P, segm_grid(Tk, E, P.ntn), st);
}

// fc2 forward: O = S . W2^T (fp32 partial planes)
hipError_t gemm_mx_fc2_fwd(const uint8_t* sq, const uint8_t* ss,
                           const uint8_t* wq, const uint8_t* ws,
                           const int32_t* offsets, int E, int64_t Tk,
                           int64_t d, int64_t f, float* o, hipStream_t st) {
  Params P{};
  P.A = reinterpret_cast<const bf16_t*>(sq); P.lda = f / 2;
  P.sA = ss; P.lds_a = f / kMxBlock;
  P.B = reinterpret_cast<const bf16_t*>(wq); P.ldb = f / 2;
  P.b_stride = d * f / 2; P.b_rows = d;
  P.sB = ws; P.lds_b = f / kMxBlock; P.bs_stride = d * f / kMxBlock;
  P.Cf = o; P.ldc = d;
  P.offsets = offsets; P.E = E; P.Tk = Tk;
  P.N = d; P.K = f / 2; P.f = f;
  P.ksplit = out_planes(f); P.plane = Tk * d;
  P.ntn = static_cast<int>((d + BN - 1) / BN);
  return launch<CfgMx, kSegM, true, true, kStoreF32, true>(
      P, segm_grid(Tk, E, P.ntn), st);
}

// fc2 dgrad + dSwiGLU: dS = dO . W2 with W2 quantized along d and stored
// transposed ([f][ldw] codes, expert e in columns [e d, (e+1) d)); dAB as
// bf16 (dab, optional), as MX codes along 2f (the gate_up data gradient's
// A) and, optionally, as MX codes along each expert's tokens from its bf16
// value (the dW_gu GEMM's A)
hipError_t gemm_mx_fc2_dgrad(const uint8_t* doq, const uint8_t* dos,
                             const uint8_t* wtq, const uint8_t* wts,
                             int64_t ldw, const int32_t* offsets, int E,
                             int64_t Tk, int64_t d, int64_t f,
                             const bf16_t* ab, const float* w_perm,
                             bf16_t* dab, uint8_t* dabq, uint8_t* dabs,
                             uint8_t* dab_tok, uint8_t* dab_tok_scales,
                             int64_t ldt, float* dp_part, hipStream_t st) {
  if (dab_tok && !kMxTokEpi) return hipErrorInvalidValue;
  Params P{};
  P.A = reinterpret_cast<const bf16_t*>(doq); P.lda = d / 2;
  P.sA = dos; P.lds_a = d / kMxBlock;
  P.B = reinterpret_cast<const bf16_t*>(wtq); P.ldb = ldw / 2;
  P.b_stride = d / 2; P.b_rows = f;
  P.sB = wts; P.lds_b = ldw / kMxBlock; P.bs_stride = d / kMxBlock;
  P.C = dab; P.ldc = 2 * f;
  P.offsets = offsets; P.E = E; P.Tk = Tk;
  P.N = f; P.K = d / 2; P.f = f;
  P.ntn = gemm_dp_tiles(f);
  P.AB = ab; P.w = w_perm; P.dp_part = dp_part; P.Qc = dabq; P.Qs = dabs;
  P.Tc = dab_tok; P.Ts = dab_tok_scales; P.ldt = ldt;
  return launch<CfgMx, kSegM, true, true, kDSwiglu, true>(
      P, segm_grid(Tk, E, P.ntn), st);
}

// fc1 dgrad: dXp = dAB . W_gu with W_gu quantized along 2f and stored
// transposed ([d][ldw] codes, expert e in columns [2 e f, 2 (e+1) f))
hipError_t gemm_mx_fc1_dgrad(const uint8_t* dabq, const uint8_t* dabs,
                             const uint8_t* wtq, const uint8_t* wts,
                             int64_t ldw, const int32_t* offsets, int E,
                             int64_t Tk, int64_t d, int64_t f, float* dxp,
                             hipStream_t st) {
  Params P{};
  P.A = reinterpret_cast<const bf16_t*>(dabq); P.lda = f;
  P.sA = dabs; P.lds_a = 2 * f / kMxBlock;
  P.B = reinterpret_cast<const bf16_t*>(wtq); P.ldb = ldw / 2;
  P.b_stride = f; P.b_rows = d;
  P.sB = wts; P.lds_b = ldw / kMxBlock; P.bs_stride = 2 * f / kMxBlock;
  P.Cf = dxp; P.ldc = d;
  P.offsets = offsets; P.E = E; P.Tk = Tk;
  P.N = d; P.K = f; P.f = f;
  P.ksplit = out_planes(f); P.plane = Tk * d;
  P.ntn = static_cast<int>((d + BN - 1) / BN);
  return launch<CfgMx, kSegM, true, true, kStoreF32, true>(
      P, segm_grid(Tk, E, P.ntn), st);
}

// wgrad: C[e] (M x N) = sum over the expert's padded token range of
// A[m][t] B[n][t], both operands quantized along tokens and transposed
// ([rows][ldt] codes, [rows][ldt / 32] scales)
hipError_t gemm_mx_wgrad(const uint8_t* aq, const uint8_t* as,
                         const uint8_t* bq, const uint8_t* bs, bool b_fp4,
                         int64_t ldt, const int32_t* offsets, int E,
                         int64_t M, int64_t N, bf16_t* c, hipStream_t st) {
  if (b_fp4 && !CfgMx::kSplitLoad) return hipErrorInvalidValue;
  Params P{};
  P.A = reinterpret_cast<const bf16_t*>(aq); P.lda = ldt / 2;
  P.sA = as; P.lds_a = ldt / kMxBlock;
  // B: E4M3 rows of ldt codes, or E2M1 rows of ldt/2 bytes (2-byte units)
  P.B = reinterpret_cast<const bf16_t*>(bq); P.ldb = b_fp4 ? ldt / 4 : ldt / 2;
  P.sB = bs; P.lds_b = ldt / kMxBlock;
  P.C = c; P.ldc = N; P.c_stride = M * N;
  P.offsets = offsets; P.E = E;
  P.M = static_cast<int>(M); P.N = static_cast<int>(N);
  P.ntn = static_cast<int>((N + BN - 1) / BN);
  const int64_t mtiles = (M + BM - 1) / BM;
  const int grid = static_cast<int>(E * mtiles * P.ntn);
  if (b_fp4)
    return launch<CfgMx, kSegKT, true, true, kStore, true, 2>(P, grid, st);
  return launch<CfgMx, kSegKT, true, true, kStore, true>(P, grid, st);
}

}  // namespace moe
