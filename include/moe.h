/*
 * moe.h -- C-ABI of libmoe.so: the mixture-of-experts expert-MLP hot path
 * (top-k routing, permutation by expert, grouped GEMM with fused SwiGLU and
 * routing-weight scaling, optional MXFP8 block quantization, un-permute
 * combine; forward and backward) as hand-written HIP kernels for gfx950.
 *
 * Sources, cited by page title and section:
 *  [P1] "Efficient MoE Training for Biological Foundation Models" (NVIDIA
 *       Developer Blog): Challenge 1 (per-expert loop; GroupedLinear takes
 *       per-expert token counts, split_sizes, gate_up has out_features =
 *       2 * intermediate_size, bias=False), Challenge 2 (MXFP8: one scaling
 *       factor per block of 32 consecutive values), Challenge 3
 *       (GroupedLinear(gate_up) -> ScaledSwiGLU -> GroupedLinear(down), the
 *       routing probabilities are the SwiGLU's scales; a matching fused
 *       backward; quantization folded into the fused path).
 *  [P4] "How MoE Architecture Cuts Costs and Boosts Efficiency: Efficient
 *       Training of Biological Foundation Models", section "Why Biology Is
 *       Especially Well-Suited for MoE" (top-K router over per-expert
 *       scores) and "Engineering Challenges of Efficient Training" (load
 *       balance).
 *  [P5] the hgpu.org abstract of an MXFP4 MoE training recipe on Hopper
 *       (block-quantized activations converted from row blocks to column
 *       blocks with their scales, without a round trip through bf16).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; the
 *    library never allocates or frees memory.  Scratch memory is the
 *    caller's `workspace` (size from moe_workspace_bytes); it need not be
 *    zeroed.  The one exception, moe_permute_noalloc, uses a fixed
 *    per-GPU scratch array of the library instead (see there).
 *  - Row-major layouts.  bf16 tensors are passed as `void*` holding IEEE
 *    bfloat16 bit patterns.  Every tensor pointer must be 16-byte aligned.
 *  - Work is enqueued on `stream` and the call returns without waiting.
 *    Counts and offsets stay on the device (no host synchronisation).
 *  - Errors: arguments are validated on the host before anything is
 *    launched.  On a validation failure the call returns a non-zero
 *    moe_status, launches nothing and leaves every output untouched;
 *    moe_last_error() then describes the failure (thread-local).  A failed
 *    kernel launch returns MOE_ERR_HIP.  No exception crosses the ABI.
 *  - Limits: 1 <= k <= E <= 1024, k <= 32, T >= 1, T*k < 2^31, d and
 *    f >= 8 and multiples of 8 (bf16) or of 32 (MXFP8).  Sizes are bound
 *    per buffer resource, not per tensor: one expert's weight, and for the
 *    weight gradients T*k rows of 2f (bf16) values, or a token-axis MX
 *    operand, must each stay within 4 GiB - 256 B; x and the router weight
 *    within 2 GiB.  (The Mixtral shape, d = 4096 and f = 14336, runs up to about
 *    T*k = 74,000 rows a call.)
 *  - Deterministic: identical inputs give bitwise identical outputs (no
 *    floating-point atomics; all reductions run in a fixed order).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment      */
  MOE_ERR_UNSUPPORTED = 2,  /* valid request outside the supported set  */
  MOE_ERR_WORKSPACE = 3,    /* workspace smaller than moe_workspace_bytes */
  MOE_ERR_HIP = 4           /* a HIP launch failed                       */
} moe_status;

typedef enum moe_prec {
  MOE_BF16 = 0,   /* bf16 operands, fp32 accumulation                    */
  MOE_MXFP8 = 1,  /* E4M3 codes + one E8M0 scale byte per 32 values       */
  MOE_MXFP4 = 2   /* MXFP8 GEMMs with MXFP4 activations ([P5]): the       */
                  /* dispatched x and the saved fc1 input are E2M1 codes  */
                  /* (two a byte) + one E8M0 scale byte per 32 values     */
} moe_prec;

/* Entry ids for moe_workspace_bytes. */
typedef enum moe_entry {
  MOE_ENTRY_PERMUTE = 0,
  MOE_ENTRY_MLP_FWD = 1,
  MOE_ENTRY_MLP_BWD = 2,
  MOE_ENTRY_ROUTER_BWD = 3
} moe_entry;

/* Short name of a status code (static string). */
const char* moe_status_str(moe_status s);

/* Description of the last failure of a call made by this thread. */
const char* moe_last_error(void);

/* Version string of the library build. */
const char* moe_version(void);

/*
 * moe_router_logits -- router scores, [P4] (the router emits one score per
 * expert):  logits[t][e] = sum_i x[t][i] * w_g[e][i] (+ bias[e]).
 *   x       [T][d]  bf16        w_g   [E][d] bf16
 *   bias    [E]     fp32 or NULL
 *   logits  [T][E]  fp32 out    (fp32 accumulation on bf16 MFMA)
 */
moe_status moe_router_logits(const void* x, const void* w_g, const float* bias,
                             int64_t T, int64_t d, int32_t E, float* logits,
                             hipStream_t stream);

/*
 * moe_route -- top-k expert choice and routing weights, [P4] (only the K
 * best-scoring experts run) and [P1] Challenge 1 (routing weights scale the
 * expert outputs).  Per token: experts ordered by descending score, equal
 * scores by ascending id (+0.0 and -0.0 are equal); the first k are kept in
 * that order.  renorm != 0: weights are the softmax over the k chosen
 * scores (softmax then renormalisation over the chosen k); renorm == 0:
 * the softmax over all E scores, taken at the chosen experts.
 *   logits   [T][E] fp32 (finite)
 *   topk_idx [T][k] int32 out,  topk_w [T][k] fp32 out
 */
moe_status moe_route(const float* logits, int64_t T, int32_t E, int32_t k,
                     int32_t renorm, int32_t* topk_idx, float* topk_w,
                     hipStream_t stream);

/*
 * moe_router_backward -- gradient of the router, and the load-balancing
 * term, [P4] "Engineering Challenges of Efficient Training" (a router that
 * keeps favouring a few experts is counteracted by a balancing term; the
 * pages give no formula, the one below is the common one).  With the
 * choices topk_idx held fixed (the top-k selection is piecewise constant):
 *   s = sum_j p_j dp_j over the token's k slots, and
 *   renorm != 0: dlogits[t][idx_j] = p_j (dp_j - s), 0 at unchosen experts;
 *   renorm == 0: dlogits[t][e] = P_e (g_e - s), P = softmax over all E,
 *                g_e = dp_j where e = idx_j, else 0.
 * With counts (the dispatch plan's [E]) the balancing term
 *   aux = aux_coef * E * sum_e f_e * mean_t P[t][e],  f_e = counts[e]/(T k)
 * (f held constant) adds aux_coef * E / T * P_e (f_e - sum_e' f_e' P_e')
 * to dlogits and its value goes to aux_loss[0] (when not NULL).  Then
 *   dw_g [E][d] fp32 = dlogits^T x,  db [E] fp32 = sum_t dlogits[t]
 *   dx_out [T][d] bf16 = dx_in + dlogits . w_g   (fp32 sum, one rounding)
 * topk_w are the forward's routing weights p; dp [T][k] fp32 comes from
 * moe_grouped_mlp_bwd.  dw_g, db, dx_in, dx_out, aux_loss and counts may be
 * NULL (the matching output is skipped; dx_in NULL means zero).  x (bf16
 * [T][d]) is read only for dw_g, w_g (bf16 [E][d]) only for dx_out; d must
 * then be a positive multiple of 8.  All sums run in a fixed order
 * (deterministic).  Errors: MOE_ERR_INVALID_ARG for a missing pointer, bad
 * T/E/k/d or aux_loss without counts; MOE_ERR_WORKSPACE for a short
 * workspace.  All pointers are device memory owned by the caller.
 * Workspace: MOE_ENTRY_ROUTER_BWD.
 */
moe_status moe_router_backward(const float* logits, const int32_t* topk_idx,
                               const float* topk_w, const float* dp,
                               const int32_t* counts, float aux_coef,
                               int64_t T, int32_t E, int32_t k,
                               int32_t renorm, const void* x, const void* w_g,
                               int64_t d, float* dlogits, float* dw_g,
                               float* db, const float* dx_in, void* dx_out,
                               float* aux_loss, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * moe_permute -- dispatch plan and token permutation, [P1] Challenge 1
 * (each expert gathers its tokens; split_sizes are the per-expert counts).
 *   counts[e]   = number of (t, j) with topk_idx[t][j] == e       [E]
 *   offsets[e]  = sum of counts[e'] for e' < e; offsets[E] = T*k   [E+1]
 *   pos[t][j]   = offsets[e] + #{t' < t : e in topk_idx[t']}      [T][k]
 *                 (rows of an expert follow ascending token id)
 *   src[r]      = token of permuted row r                          [T*k]
 *   w_perm[r]   = topk_w of the slot that maps to row r            [T*k]
 *   x_perm[r]   = x[src[r]]                                        [T*k][d]
 * prec == MOE_BF16: x and x_perm are bf16, x_scales/x_perm_scales unused.
 * prec == MOE_MXFP8: x/x_perm are E4M3 codes (uint8 [.][d]) with E8M0
 *   scales x_scales/x_perm_scales (uint8 [.][d/32]) moved along.
 * topk_w may be NULL (then w_perm may be NULL too).  Integer outputs are
 * exact and deterministic.  Workspace: MOE_ENTRY_PERMUTE.
 */
moe_status moe_permute(moe_prec prec, const int32_t* topk_idx,
                       const float* topk_w, int64_t T, int32_t E, int32_t k,
                       const void* x, const uint8_t* x_scales, int64_t d,
                       int32_t* counts, int32_t* offsets, int32_t* pos,
                       int32_t* src, float* w_perm, void* x_perm,
                       uint8_t* x_perm_scales, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * moe_permute_noalloc -- moe_permute without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments (minus workspace), outputs and errors as moe_permute.  Its
 * scratch (the plan's per-chunk counts) is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES in device memory, one copy per GPU, held until
 * the process ends; the call allocates and frees nothing.  The plan uses
 * at most 512 chunks, so every valid (T*k, E) fits (at most 512 * E * 4
 * bytes); a plan needing more than the limit would be rejected with
 * MOE_ERR_UNSUPPORTED before any launch.  The
 * kernels write every scratch word they read, so nothing is cleared
 * between calls.  Every call on one GPU shares that GPU's scratch: calls
 * that overlap on one GPU (concurrent streams, or threads) race and give
 * undefined results; calls ordered on one stream are safe.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (2u << 20)
moe_status moe_permute_noalloc(moe_prec prec, const int32_t* topk_idx,
                               const float* topk_w, int64_t T, int32_t E,
                               int32_t k, const void* x,
                               const uint8_t* x_scales, int64_t d,
                               int32_t* counts, int32_t* offsets,
                               int32_t* pos, int32_t* src, float* w_perm,
                               void* x_perm, uint8_t* x_perm_scales,
                               hipStream_t stream);

/*
 * moe_permute_rows -- row permutation with an existing plan (used for the
 * upstream gradient in the backward pass): x_perm[pos[t][j]] = x[t].
 * Same dtype rules as moe_permute.
 */
moe_status moe_permute_rows(moe_prec prec, const int32_t* pos, int64_t T,
                            int32_t k, const void* x, const uint8_t* x_scales,
                            int64_t d, void* x_perm, uint8_t* x_perm_scales,
                            hipStream_t stream);

/*
 * moe_grouped_mlp_fwd -- all experts' SwiGLU MLPs as grouped GEMMs over the
 * permuted rows, [P1] Challenge 1 (one grouped submission, per-expert
 * weights) and Challenge 3 (gate_up -> ScaledSwiGLU -> down, fused).  For
 * every expert e and row r in [offsets[e], offsets[e+1]):
 *   AB[r]  = x_perm[r] . w_gu[e]^T                 (gate: first f columns)
 *   S[r]   = w_perm[r] * silu(AB[r][:f]) * AB[r][f:]
 *   O[r]   = S[r] . w2[e]^T
 *   w_gu [E][2f][d], w2 [E][d][f]; ab_saved [T*k][2f] bf16 out,
 *   s_saved [T*k][f] bf16 out; out_perm [P][T*k][d] fp32 out, P =
 *   moe_row_planes(f): O as P partial sums over consecutive ranges of the
 *   reduction (kept in fp32 and summed, in plane order, by moe_unpermute,
 *   so that each output is rounded once).
 * prec == MOE_MXFP8 ([P1] Challenge 2: blocks of 32 along each GEMM's
 *   reduction axis, E4M3 codes with E8M0 scales): x_perm is codes + scales
 *   along d (from moe_permute), w_gu/w2 are codes with scales along their
 *   last axis (from moe_mxfp8_quantize, axis 0); S is quantized along f
 *   inside the gate_up epilogue, from its fp32 value, for the down GEMM
 *   (held in the workspace); ab_saved/s_saved stay bf16, out_perm fp32.
 *   d and f must be multiples of 128.
 *   With s_tok / s_tok_scales (MXFP8 only; [P5]'s conversion from row blocks
 *   to column blocks, done inside the kernel that produces S) the same epilogue also
 *   writes S quantized along each expert's tokens from its bf16 value --
 *   bit for bit what moe_mxfp8_quantize axis 1 (seg_offsets = offsets,
 *   rows_pad = ldt) makes of s_saved -- for the dW2 GEMM of the backward:
 *   codes [f][ldt], scales [f][ldt/32], ldt a multiple of 128 and at
 *   least moe_mxfp8_padded_rows(Tk, E).  Every expert's padded rows are
 *   written (zero codes past its last row); columns past the last
 *   expert's padded rows are not.  s_saved may then be NULL.  For bf16
 *   s_tok must be NULL and s_saved is required.
 * prec == MOE_MXFP4 ([P5]: FP8 GEMMs with MXFP4 activations): as
 *   MOE_MXFP8 except that x_perm is the MXFP4 payload from moe_permute --
 *   E2M1 codes [T*k][d/2] (two a byte, from moe_mxfp4_quantize axis 0)
 *   with scales [T*k][d/32] -- which the gate_up GEMM widens to E4M3 codes
 *   on their way to LDS (every E2M1 value is an E4M3 value; the scales are
 *   kept), so the GEMM runs on the FP8 MFMA.
 * w_perm may be NULL (weight 1).  Workspace: MOE_ENTRY_MLP_FWD (none for
 * bf16).
 */
moe_status moe_grouped_mlp_fwd(moe_prec prec, const void* x_perm,
                               const uint8_t* x_perm_scales,
                               const int32_t* offsets, int32_t E, int64_t Tk,
                               int64_t d, int64_t f, const void* w_gu,
                               const uint8_t* w_gu_scales, const void* w2,
                               const uint8_t* w2_scales, const float* w_perm,
                               void* ab_saved, void* s_saved, void* out_perm,
                               uint8_t* s_tok, uint8_t* s_tok_scales,
                               int64_t ldt, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_mlp_bwd -- backward of moe_grouped_mlp_fwd ([P1] Challenge 3
 * names a matching fused backward).  With dO = dout_perm (rows permuted
 * like x_perm) and H = silu(A_g) * A_u recomputed from ab_saved:
 *   dW2[e]   = dO_e^T . S_e            (K = rows of e; zero if none)
 *   dS       = dO . w2[e]
 *   dp[t][j] = <dS[r], H[r]>, r = pos[t][j]      (fp32, fixed-order sums)
 *   dA_g     = w*dS * A_u * sig(A_g) * (1 + A_g*(1 - sig(A_g)))
 *   dA_u     = w*dS * silu(A_g)
 *   dW_gu[e] = dAB_e^T . x_perm_e
 *   dx_perm  = dAB . w_gu[e]
 *   dout_perm [T*k][d] bf16, x_perm [T*k][d] bf16, ab_saved, s_saved as
 *   written by the forward; dx_perm [P][T*k][d] fp32 out (P partial-sum
 *   planes as out_perm); dw_gu [E][2f][d], dw2 [E][d][f] bf16 out;
 *   dp [T][k] fp32 out (needs pos).
 * prec == MOE_MXFP8: inputs and outputs stay bf16; every GEMM operand is
 *   quantized inside the call along that GEMM's reduction axis: dO along
 *   d, w2 along d and w_gu along 2f (per expert), dAB along 2f (in the
 *   epilogue that produces it, from fp32), and for the weight gradients
 *   dO, s_saved, dAB (its bf16 value) and x_perm along the rows of each
 *   expert, blocks restarting at the expert's first row.  d and f must be
 *   multiples of 128.  dAB's token-axis codes come out of the epilogue
 *   that produces dAB (no bf16 dAB is stored).  With s_tok/s_tok_scales
 *   from the forward (ldt = moe_mxfp8_padded_rows(T*k, E)) S is not
 *   quantized again and s_saved may be NULL; for bf16 s_tok must be NULL.
 *   x_perm_scales is unused (NULL) for bf16 and MXFP8.  The weights' codes
 *   along their columns may come in ready-made: w_gu_col_codes [d][E*2f]
 *   with w_gu_col_scales [d][E*2f/32], and w2_col_codes [f][E*d] with
 *   w2_col_scales [f][E*d/32], the col outputs of moe_mxfp8_quantize_weight
 *   over w_gu viewed as [E*2f][d] and w2 viewed as [E*d][f] (as a training
 *   forward makes them); the call then skips those two quantizations.
 *   Each pair is given whole or NULL; all four are NULL for bf16.
 * prec == MOE_MXFP4: as MOE_MXFP8 except that x_perm is the forward's
 *   MXFP4 payload (codes [T*k][d/2], x_perm_scales [T*k][d/32]); the dW_gu
 *   GEMM reads it converted to MXFP4 blocks along each expert's tokens
 *   (moe_mxfp4_quantize axis 1 from MXFP4 rows), widened to E4M3 as
 *   above, so no bf16 copy of x is needed.
 * Workspace: MOE_ENTRY_MLP_BWD.
 */
moe_status moe_grouped_mlp_bwd(moe_prec prec, const void* dout_perm,
                               const void* x_perm,
                               const uint8_t* x_perm_scales,
                               const int32_t* offsets,
                               const int32_t* pos, int64_t T, int32_t k,
                               int32_t E, int64_t d, int64_t f,
                               const void* w_gu, const void* w2,
                               const void* ab_saved, const void* s_saved,
                               const uint8_t* s_tok,
                               const uint8_t* s_tok_scales, int64_t ldt,
                               const uint8_t* w_gu_col_codes,
                               const uint8_t* w_gu_col_scales,
                               const uint8_t* w2_col_codes,
                               const uint8_t* w2_col_scales,
                               const float* w_perm, void* dx_perm,
                               void* dw_gu, void* dw2, float* dp,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * Stage entry points: the single grouped GEMMs that moe_grouped_mlp_fwd and
 * moe_grouped_mlp_bwd are made of ([P1] Challenge 1: GroupedLinear as one
 * grouped submission per projection; Challenge 3: ScaledSwiGLU fused into
 * the gate_up projection and a matching backward).  Each launches exactly
 * one kernel, so callers can time, overlap or reorder the pieces.  Shapes
 * and dtypes are those of the fused entry points.
 *
 * moe_gate_up_swiglu_fwd: ab_saved = x_perm . w_gu[e]^T (bf16) and
 *   s_saved = w_perm * silu(gate) * up (bf16).
 * moe_down_fwd: out_perm = s_saved . w2[e]^T (fp32, P planes).
 * moe_down_swiglu_bwd: dS = dout_perm . w2[e]; writes dab [T*k][2f] bf16
 *   (dA_g, dA_u as in moe_grouped_mlp_bwd) and dp_part [T*k][ntiles] fp32,
 *   the per-tile sums of dS * H, ntiles = moe_dp_tiles(f).
 * moe_gate_up_dgrad: dx_perm = dab . w_gu[e] (fp32, P planes).
 * moe_grouped_wgrad: for each expert e, c[e] (M x N, bf16) = sum over the
 *   expert's rows r of a[r][m] * b[r][n]; a [T*k][lda], b [T*k][ldb]
 *   row-major; experts without rows get exact zeros.  (dW2: a = dout_perm,
 *   b = s_saved, M = d, N = f; dW_gu: a = dab, b = x_perm, M = 2f, N = d.)
 * moe_dp_reduce: dp[t][j] = sum over tiles, in order, of
 *   dp_part[pos[t][j]][tile].
 */
int32_t moe_dp_tiles(int64_t f);

moe_status moe_gate_up_swiglu_fwd(const void* x_perm, const int32_t* offsets,
                                  int32_t E, int64_t Tk, int64_t d, int64_t f,
                                  const void* w_gu, const float* w_perm,
                                  void* ab_saved, void* s_saved,
                                  hipStream_t stream);

moe_status moe_down_fwd(const void* s_saved, const int32_t* offsets,
                        int32_t E, int64_t Tk, int64_t d, int64_t f,
                        const void* w2, float* out_perm, hipStream_t stream);

moe_status moe_down_swiglu_bwd(const void* dout_perm, const int32_t* offsets,
                               int32_t E, int64_t Tk, int64_t d, int64_t f,
                               const void* w2, const void* ab_saved,
                               const float* w_perm, void* dab, float* dp_part,
                               hipStream_t stream);

moe_status moe_gate_up_dgrad(const void* dab, const int32_t* offsets,
                             int32_t E, int64_t Tk, int64_t d, int64_t f,
                             const void* w_gu, float* dx_perm,
                             hipStream_t stream);

moe_status moe_grouped_wgrad(const void* a, int64_t lda, const void* b,
                             int64_t ldb, const int32_t* offsets, int32_t E,
                             int64_t Tk, int64_t M, int64_t N, void* c,
                             hipStream_t stream);

moe_status moe_dp_reduce(const float* dp_part, int32_t ntiles,
                         const int32_t* pos, int64_t T, int32_t k, float* dp,
                         hipStream_t stream);

/*
 * MXFP8 stage entry points ([P1] Challenge 2): the block-scaled versions
 * of the stage GEMMs above, one kernel each, on E4M3 codes (uint8) with
 * one E8M0 scale byte per 32 codes along the reduction axis.  d and f must
 * be multiples of 128; outputs as in the bf16 stages.
 *
 * moe_mx_gate_up_swiglu_fwd: xq [T*k][d], xs [T*k][d/32] (x_fp4 != 0:
 *   E2M1 codes xq [T*k][d/2], two a byte); wq [E][2f][d],
 *   ws [E][2f][d/32]; writes ab_saved, s_saved (bf16, may be NULL) and S
 *   quantized along f from its fp32 value: sq [T*k][f], ss [T*k][f/32];
 *   with s_tok/s_tok_scales also S along each expert's tokens (as in
 *   moe_grouped_mlp_fwd; NULL to skip).
 * moe_mx_down_fwd: sq/ss as written above; wq [E][d][f], ws [E][d][f/32];
 *   out_perm [P][T*k][d] fp32.
 * moe_mx_down_swiglu_bwd: doq [T*k][d], dos [T*k][d/32] (dout_perm along
 *   d); w2tq [f][E*d], w2ts [f][E*d/32] (w2 viewed as [E*d][f] quantized
 *   with moe_mxfp8_quantize axis 1, one segment, rows_pad E*d: expert e
 *   in columns [e*d, (e+1)*d)); writes dab (bf16, may be NULL), dAB
 *   quantized along 2f from fp32 (dabq [T*k][2f], dabs [T*k][2f/32]),
 *   dp_part and, with dab_tok/dab_tok_scales, dAB along each expert's
 *   tokens from its bf16 value (codes [2f][ldt], scales [2f][ldt/32],
 *   bit for bit moe_mxfp8_quantize axis 1 of the bf16 dab; NULL to skip).
 * moe_mx_gate_up_dgrad: dabq/dabs as written above; wgutq [d][E*2f],
 *   wguts [d][E*2f/32] (w_gu viewed as [E*2f][d], axis 1, one segment,
 *   rows_pad E*2f); dx_perm [P][T*k][d] fp32.
 * moe_mx_grouped_wgrad: c[e] (M x N, bf16) = sum over expert e's padded
 *   token range of a[m][t] * b[n][t], where aq [M][ldt], as [M][ldt/32],
 *   bq [N][ldt], bs [N][ldt/32] come from moe_mxfp8_quantize axis 1 with
 *   seg_offsets = offsets (nseg = E) and rows_pad = ldt (a multiple of 128,
 *   at least moe_mxfp8_padded_rows(T*k, E)).  Experts without rows get
 *   exact zeros.  b_fp4 != 0: b is E2M1, codes bq [N][ldt/2] (two a byte)
 *   from moe_mxfp4_quantize axis 1.
 */
moe_status moe_mx_gate_up_swiglu_fwd(
    const uint8_t* xq, const uint8_t* xs, int32_t x_fp4,
    const int32_t* offsets, int32_t E,
    int64_t Tk, int64_t d, int64_t f, const uint8_t* wq, const uint8_t* ws,
    const float* w_perm, void* ab_saved, void* s_saved, uint8_t* sq,
    uint8_t* ss, uint8_t* s_tok, uint8_t* s_tok_scales, int64_t ldt,
    hipStream_t stream);

moe_status moe_mx_down_fwd(const uint8_t* sq, const uint8_t* ss,
                           const int32_t* offsets, int32_t E, int64_t Tk,
                           int64_t d, int64_t f, const uint8_t* wq,
                           const uint8_t* ws, float* out_perm,
                           hipStream_t stream);

moe_status moe_mx_down_swiglu_bwd(
    const uint8_t* doq, const uint8_t* dos, const int32_t* offsets,
    int32_t E, int64_t Tk, int64_t d, int64_t f, const uint8_t* w2tq,
    const uint8_t* w2ts, const void* ab_saved, const float* w_perm,
    void* dab, uint8_t* dabq, uint8_t* dabs, uint8_t* dab_tok,
    uint8_t* dab_tok_scales, int64_t ldt, float* dp_part,
    hipStream_t stream);

moe_status moe_mx_gate_up_dgrad(const uint8_t* dabq, const uint8_t* dabs,
                                const int32_t* offsets, int32_t E, int64_t Tk,
                                int64_t d, int64_t f, const uint8_t* wgutq,
                                const uint8_t* wguts, float* dx_perm,
                                hipStream_t stream);

moe_status moe_mx_grouped_wgrad(const uint8_t* aq, const uint8_t* as,
                                const uint8_t* bq, const uint8_t* bs,
                                int32_t b_fp4, int64_t ldt,
                                const int32_t* offsets,
                                int32_t E, int64_t Tk, int64_t M, int64_t N,
                                void* c, hipStream_t stream);

/*
 * moe_unpermute -- combine, [P1] Challenge 1 (the loop index-adds each
 * expert's rows back into the token's output).  Gather form, no atomics:
 *   y[t] = sum over j, in ascending expert id, of wt * o_perm[pos[t][j]]
 * with wt = w[t][j] (or 1 when w is NULL); fp32 accumulation, one final
 * rounding.  o_perm [o_planes][T*k][d] fp32 (o_fp32 != 0; a row is the
 * sum of its planes, added in plane order) or [T*k][d] bf16 (o_fp32 == 0,
 * o_planes must be 1); y [T][d] bf16 (y_fp32 == 0) or fp32 (y_fp32 != 0).
 * With dlogits (fp32 [T][E], the router score gradients moe_router_backward
 * returns) the router's share of the input gradient is added before the
 * rounding: y[t] += sum over e, in order, of dlogits[t][e] * w_g[e]
 * (w_g bf16 [E][d], 1 <= E <= 1024), the same arithmetic as that entry's
 * dx_in/dx_out, so the backward's dX leaves in one pass; dlogits NULL
 * ignores w_g and E.
 */
moe_status moe_unpermute(const void* o_perm, int32_t o_fp32,
                         int32_t o_planes, const int32_t* pos, const float* w,
                         int64_t T, int32_t k, int64_t d, int32_t y_fp32,
                         void* y, const float* dlogits, const void* w_g,
                         int32_t E, hipStream_t stream);

/* Number of partial-sum planes P in out_perm and dx_perm for intermediate
 * width f: 2 when f >= 4096 (fc2's reduction over f and fc1's data-gradient
 * reduction over 2f are each cut in two), else 1; 0 when f < 1. */
int32_t moe_row_planes(int64_t f);

/*
 * moe_mxfp8_quantize -- MX block quantization, [P1] Challenge 2 (8-bit
 * values, one scale per block of 32 consecutive values).  Per block:
 * amax = max|v|; e = clamp(floor(log2 amax) - 8, -127, 127) (e = -127 for
 * an all-zero block); scale byte = e + 127; code = E4M3(v / 2^e), rounded
 * to nearest with ties to even mantissa and saturated to +-448, sign kept.
 *   src [rows][cols] bf16.
 *   axis == 0: blocks of 32 consecutive columns (cols % 32 == 0);
 *     codes [rows][cols], scales [rows][cols/32].
 *   axis == 1: blocks of 32 consecutive rows that restart at every segment
 *     start seg_offsets[s] (nseg segments, seg_offsets [nseg+1] on the
 *     device, seg_offsets[0] == 0, seg_offsets[nseg] == rows; NULL means
 *     one segment); the last block of a segment covers the rows left.
 *     Output is transposed so that each block is contiguous: codes
 *     [cols][rows_pad], scales [cols][rows_pad/32]; row r of segment s
 *     lands at column pad_off[s] + (r - seg_offsets[s]) where pad_off[s]
 *     is the sum of the previous segments' lengths, each rounded up to 128
 *     (so every segment starts on a multiple of 128).  Padding holds code
 *     0 with scale byte 0.  rows_pad: a multiple of 128, at least
 *     moe_mxfp8_padded_rows(rows, nseg).
 * Inputs are finite.  Codes and scales are exact (bit-identical to the
 * definition above).
 */
moe_status moe_mxfp8_quantize(const void* src, int64_t rows, int64_t cols,
                              int32_t axis, const int32_t* seg_offsets,
                              int32_t nseg, uint8_t* codes, uint8_t* scales,
                              int64_t rows_pad, hipStream_t stream);

/*
 * moe_mxfp8_quantize_weight -- both MX layouts of one weight matrix from a
 * single read of it ([P1] Challenge 3: the weights are quantized for the
 * forward GEMM, along their rows, and for the data-gradient GEMM, along
 * their columns).  src [rows][cols] bf16; writes
 *   row_codes [rows][cols], row_scales [rows][cols/32]: bit for bit
 *     moe_mxfp8_quantize axis 0;
 *   col_codes [cols][rows], col_scales [cols][rows/32]: bit for bit
 *     moe_mxfp8_quantize axis 1 with one segment and rows_pad = rows.
 * rows a multiple of 128, cols a multiple of 64.  Errors:
 * MOE_ERR_INVALID_ARG for a missing pointer or bad sizes.  All pointers are
 * device memory owned by the caller.  No workspace.
 */
moe_status moe_mxfp8_quantize_weight(const void* src, int64_t rows,
                                     int64_t cols, uint8_t* row_codes,
                                     uint8_t* row_scales, uint8_t* col_codes,
                                     uint8_t* col_scales,
                                     hipStream_t stream);

/*
 * moe_mxfp4_quantize -- MXFP4 block quantization ([P5]: MXFP4 activations
 * and dispatch payloads under FP8 GEMMs; row-blocked FP4 turned into column
 * blocks with new scales).  E2M1 codes (0, 0.5, 1, 1.5, 2, 3, 4, 6 and
 * negatives; sign in bit 3), two a byte with the lower index in the low
 * nibble, and one E8M0 scale byte per 32 values: scale exponent
 * e = clamp(floor(log2 amax) - 2, -127, 127) (-127 for an all-zero block),
 * byte e + 127, codes rounded to nearest with ties to the even code and
 * saturated at +-6.
 *   src_fmt 0: src is bf16 [rows][cols].
 *   src_fmt 1: src is MXFP4 rows, codes [rows][cols/2] with src_scales
 *     [rows][cols/32]; every value is decoded exactly first (axis 1 only:
 *     the row-to-column conversion).
 *   axis 0: codes [rows][cols/2], scales [rows][cols/32] (src_fmt 0).
 *   axis 1: blocks of 32 rows restarting at each segment start
 *     (seg_offsets [nseg+1] on the device, or NULL for one segment),
 *     transposed and 128-padded as moe_mxfp8_quantize axis 1: codes
 *     [cols][rows_pad/2], scales [cols][rows_pad/32]; every byte up to
 *     rows_pad is written (padding: code 0, scale byte 0).
 * cols must be a multiple of 32.  Bit-exact and deterministic.
 */
moe_status moe_mxfp4_quantize(const void* src, int32_t src_fmt,
                              const uint8_t* src_scales, int64_t rows,
                              int64_t cols, int32_t axis,
                              const int32_t* seg_offsets, int32_t nseg,
                              uint8_t* codes, uint8_t* scales,
                              int64_t rows_pad, hipStream_t stream);

/* Host-side bound on rows_pad for axis == 1 quantization: the padded
 * segment lengths sum to a multiple of 128 that is at most rows + 127 *
 * nseg, so the bound is that number rounded down to a multiple of 128
 * (exact for one segment). */
int64_t moe_mxfp8_padded_rows(int64_t rows, int32_t nseg);

/*
 * moe_workspace_bytes -- workspace size an entry point needs for the given
 * problem (0 when none).  Returns 0 for invalid arguments.
 */
size_t moe_workspace_bytes(moe_entry entry, moe_prec prec, int64_t T,
                           int32_t E, int32_t k, int64_t d, int64_t f);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
