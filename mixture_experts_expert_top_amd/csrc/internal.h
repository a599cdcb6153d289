// Launchers shared between the kernel translation units and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
// Buffer resources address their range with 32-bit byte offsets, and a
// load at an offset at or past the range returns zero (tile masking).
// kOob is the offset the kernels give a masked load; every resource range
// is at most kOob bytes, so a masked load never reads memory.
constexpr uint32_t kOob = 0xffffff00u;
constexpr int64_t kMaxResourceBytes = kOob;
// Partial-sum planes of the fp32 row outputs (fc2's O and fc1's data
// gradient dXp), laid out [planes][T*k][d]; the combine adds them in plane
// order.  Their reductions (over f and 2f) are cut in two when f is at
// least kSplitF, which pays while each half still spans many k-steps
// (measured at f = 14336).  With a narrower f one plane keeps the tiles
// long and halves the combine's reads (measured at f = 1408).
constexpr int64_t kSplitF = 4096;
inline int out_planes(int64_t f) { return f >= kSplitF ? 2 : 1; }
// MXFP8 along tokens: every expert segment is padded to a multiple of this
// many rows so that each starts on a whole k-step of the MX GEMMs.
constexpr int kMxPad = 128;

// routing (route.hip)
hipError_t launch_router_logits(const bf16_t* x, const bf16_t* w_g,
                                const float* bias, int64_t T, int64_t d, int E,
                                float* logits, hipStream_t s);
hipError_t launch_route(const float* logits, int64_t T, int E, int k,
                        int renorm, int32_t* idx, float* w, hipStream_t s);

// dispatch plan and row movement (permute.hip)
size_t plan_workspace_bytes(int64_t Tk, int E);
hipError_t launch_plan(const int32_t* idx, int64_t T, int E, int k,
                       int32_t* counts, int32_t* offsets, int32_t* pos,
                       void* ws, hipStream_t s);
// pos/src/w_perm from the plan + the rows of x (row_bytes each) and an
// optional side array of side_bytes per row (MX scales).
hipError_t launch_scatter(const int32_t* idx, const float* topk_w, int64_t T,
                          int E, int k, const int32_t* offsets, int32_t* pos,
                          int32_t* src, float* w_perm, const void* x,
                          int64_t row_bytes, void* x_perm,
                          const void* side, int64_t side_bytes, void* side_perm,
                          const void* ws, hipStream_t s);
hipError_t launch_permute_rows(const int32_t* pos, int64_t T, int k,
                               const void* x, int64_t row_bytes, void* x_perm,
                               const void* side, int64_t side_bytes,
                               void* side_perm, hipStream_t s);
hipError_t launch_unpermute(const void* o, int o_fp32, int o_planes,
                            const int32_t* pos, const float* w, int64_t T,
                            int k, int64_t d, int y_fp32, void* y,
                            const float* dl, const bf16_t* wg, int E,
                            hipStream_t s);
hipError_t launch_dp_reduce(const float* dp_part, int ntn, const int32_t* pos,
                            int64_t T, int k, float* dp, hipStream_t s);

// MXFP8 quantization (mxfp8.hip)
hipError_t launch_mx_quant_rows(const bf16_t* src, int64_t rows, int64_t cols,
                                uint8_t* codes, uint8_t* scales,
                                hipStream_t s);
// token-axis blocks; logical row r is src row gather[r] (gather may be null)
hipError_t launch_mx_quant_tokens(const bf16_t* src, const int32_t* gather,
                                  int64_t rows, int64_t cols,
                                  const int32_t* seg, int nseg,
                                  uint8_t* codes, uint8_t* scales,
                                  int64_t rows_pad, hipStream_t s);
// Both layouts of one bf16 matrix from a single read: quant_rows' codes and
// the one-segment token-axis (transposed) codes; rows % 128 == 0.
hipError_t launch_mx_quant_both(const bf16_t* src, int64_t rows,
                                int64_t cols, uint8_t* row_codes,
                                uint8_t* row_scales, uint8_t* col_codes,
                                uint8_t* col_scales, hipStream_t s);

// MXFP4 (E2M1 codes two a byte, E8M0 scale per 32): rows of a bf16 tensor,
// and blocks along the rows (token axis, 128-padded segments, transposed)
// from bf16 (src_scales == nullptr) or from MXFP4 rows (codes [rows][cols/2]
// with src_scales [rows][cols/32]).
hipError_t launch_mx4_quant_rows(const bf16_t* src, int64_t rows,
                                 int64_t cols, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s);
hipError_t launch_mx4_quant_tokens(const void* src,
                                   const uint8_t* src_scales, int64_t rows,
                                   int64_t cols, const int32_t* seg, int nseg,
                                   uint8_t* codes, uint8_t* scales,
                                   int64_t rows_pad, hipStream_t s);

// router backward (route.hip)
size_t router_backward_workspace(int64_t T, int E, int64_t d);
hipError_t launch_router_backward(const float* logits, const int32_t* idx,
                                  const float* p, const float* dp,
                                  const int32_t* counts, float alpha,
                                  int64_t T, int E, int k, int renorm,
                                  const bf16_t* x, const bf16_t* w_g,
                                  int64_t d, float* dlogits, float* dw_g,
                                  float* db, const float* dx_in,
                                  bf16_t* dx_out, float* aux_loss, void* ws,
                                  hipStream_t s);

// grouped GEMMs (gemm.hip)
int gemm_dp_tiles(int64_t f);
hipError_t gemm_fc1_fwd(const bf16_t* xp, const bf16_t* w_gu,
                        const int32_t* offsets, int E, int64_t Tk, int64_t d,
                        int64_t f, const float* w_perm, bf16_t* ab, bf16_t* s,
                        hipStream_t st);
hipError_t gemm_fc2_fwd(const bf16_t* s, const bf16_t* w2,
                        const int32_t* offsets, int E, int64_t Tk, int64_t d,
                        int64_t f, float* o, hipStream_t st);
hipError_t gemm_fc2_dgrad(const bf16_t* dO, const bf16_t* w2,
                          const int32_t* offsets, int E, int64_t Tk,
                          int64_t d, int64_t f, const bf16_t* ab,
                          const float* w_perm, bf16_t* dab, float* dp_part,
                          hipStream_t st);
hipError_t gemm_fc1_dgrad(const bf16_t* dab, const bf16_t* w_gu,
                          const int32_t* offsets, int E, int64_t Tk,
                          int64_t d, int64_t f, float* dxp, hipStream_t st);
hipError_t gemm_wgrad(const bf16_t* a, int64_t lda, const bf16_t* b,
                      int64_t ldb, const int32_t* offsets, int E, int64_t Tk,
                      int64_t M, int64_t N, bf16_t* c, hipStream_t st);

// MXFP8 grouped GEMMs (gemm.hip): codes + scale bytes, see the definitions
hipError_t gemm_mx_fc1_fwd(const uint8_t* xq, const uint8_t* xs, bool x_fp4,
                           const uint8_t* wq, const uint8_t* ws,
                           const int32_t* offsets, int E, int64_t Tk,
                           int64_t d, int64_t f, const float* w_perm,
                           bf16_t* ab, bf16_t* s, uint8_t* sq, uint8_t* ss,
                           uint8_t* s_tok, uint8_t* s_tok_scales, int64_t ldt,
                           hipStream_t st);
hipError_t gemm_mx_fc2_fwd(const uint8_t* sq, const uint8_t* ss,
                           const uint8_t* wq, const uint8_t* ws,
                           const int32_t* offsets, int E, int64_t Tk,
                           int64_t d, int64_t f, float* o, hipStream_t st);
hipError_t gemm_mx_fc2_dgrad(const uint8_t* doq, const uint8_t* dos,
                             const uint8_t* wtq, const uint8_t* wts,
                             int64_t ldw, const int32_t* offsets, int E,
                             int64_t Tk, int64_t d, int64_t f,
                             const bf16_t* ab, const float* w_perm,
                             bf16_t* dab, uint8_t* dabq, uint8_t* dabs,
                             uint8_t* dab_tok, uint8_t* dab_tok_scales,
                             int64_t ldt, float* dp_part, hipStream_t st);
hipError_t gemm_mx_fc1_dgrad(const uint8_t* dabq, const uint8_t* dabs,
                             const uint8_t* wtq, const uint8_t* wts,
                             int64_t ldw, const int32_t* offsets, int E,
                             int64_t Tk, int64_t d, int64_t f, float* dxp,
                             hipStream_t st);
hipError_t gemm_mx_wgrad(const uint8_t* aq, const uint8_t* as,
                         const uint8_t* bq, const uint8_t* bs, bool b_fp4,
                         int64_t ldt, const int32_t* offsets, int E,
                         int64_t M, int64_t N, bf16_t* c, hipStream_t st);

}  // namespace moe
