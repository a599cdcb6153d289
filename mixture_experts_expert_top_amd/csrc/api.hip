// C-ABI of libmoe: argument validation, workspace layout and launch order.
// Semantics of every entry point are documented in include/moe.h.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "internal.h"

using moe::bf16_t;

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe_status ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxBytes = (int64_t{1} << 31) - 1;
// Largest byte range of one buffer resource: just under 4 GiB, so that the
// kernels' masked-load offset lies past every range.  The grouped GEMMs
// bound each resource by what one workgroup touches: the rows of one tile
// (row-segmented GEMMs), one expert's weight, one expert's rows of a
// weight-gradient operand, or one token-axis MX operand.
constexpr int64_t kMaxRange = moe::kMaxResourceBytes;

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

#define REQUIRE(cond, st, ...)               \
  do {                                       \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p)                                                      \
  do {                                                                      \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, #p " is NULL");    \
    if (!aligned16(p))                                                      \
      return fail(MOE_ERR_INVALID_ARG, #p " is not 16-byte aligned");       \
  } while (0)

#define REQUIRE_OPT_PTR(p)                                                  \
  do {                                                                      \
    if ((p) != nullptr && !aligned16(p))                                    \
      return fail(MOE_ERR_INVALID_ARG, #p " is not 16-byte aligned");       \
  } while (0)

moe_status check_route_dims(int64_t T, int32_t E, int32_t k) {
  REQUIRE(T >= 1, MOE_ERR_INVALID_ARG, "T must be >= 1 (got %lld)",
          static_cast<long long>(T));
  REQUIRE(T <= (int64_t{1} << 30), MOE_ERR_UNSUPPORTED, "T too large");
  REQUIRE(E >= 1 && E <= moe::kMaxExperts, MOE_ERR_INVALID_ARG,
          "E must be in [1, %d] (got %d)", moe::kMaxExperts, E);
  REQUIRE(k >= 1 && k <= E, MOE_ERR_INVALID_ARG,
          "k must be in [1, E] (got k=%d, E=%d)", k, E);
  REQUIRE(k <= moe::kMaxTopK, MOE_ERR_UNSUPPORTED, "k must be <= %d",
          moe::kMaxTopK);
  REQUIRE(T * k <= (int64_t{1} << 31) - 1, MOE_ERR_UNSUPPORTED,
          "T*k too large");
  return MOE_OK;
}

moe_status check_prec(moe_prec prec) {
  REQUIRE(prec == MOE_BF16 || prec == MOE_MXFP8 || prec == MOE_MXFP4,
          MOE_ERR_INVALID_ARG, "unknown precision %d",
          static_cast<int>(prec));
  return MOE_OK;
}

// MX GEMM operands (MXFP8, or MXFP8 with MXFP4 activations)
bool is_mx(moe_prec prec) {
  return prec == MOE_MXFP8 || prec == MOE_MXFP4;
}

// Bytes of one row of d activation values as moved by the permutations:
// bf16, E4M3 codes, or E2M1 codes two a byte.
int64_t act_row_bytes(moe_prec prec, int64_t d) {
  return prec == MOE_BF16 ? d * 2 : (prec == MOE_MXFP8 ? d : d / 2);
}

moe_status check_feature(const char* name, int64_t v, moe_prec prec) {
  const int64_t q = is_mx(prec) ? 32 : 8;
  REQUIRE(v >= q && v % q == 0, MOE_ERR_INVALID_ARG,
          "%s must be a positive multiple of %lld (got %lld)", name,
          static_cast<long long>(q), static_cast<long long>(v));
  return MOE_OK;
}

moe_status check_mlp_dims(int32_t E, int64_t Tk, int64_t d, int64_t f,
                          moe_prec prec) {
  REQUIRE(E >= 1 && E <= moe::kMaxExperts, MOE_ERR_INVALID_ARG,
          "E must be in [1, %d]", moe::kMaxExperts);
  REQUIRE(Tk >= 1, MOE_ERR_INVALID_ARG, "Tk must be >= 1");
  if (moe_status st = check_feature("d", d, prec)) return st;
  if (moe_status st = check_feature("f", f, prec)) return st;
  REQUIRE(2 * f * d * 2 <= kMaxRange, MOE_ERR_UNSUPPORTED,
          "one expert's weight is larger than 4 GiB");
  return MOE_OK;
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// The MX GEMMs read one scale dword (4 blocks of 32) per row and stage of
// 128 codes: every reduction length and scale row must be a multiple of
// 128 codes.
moe_status check_mx_dims(int64_t d, int64_t f) {
  REQUIRE(d % moe::kMxPad == 0 && f % moe::kMxPad == 0, MOE_ERR_INVALID_ARG,
          "MXFP8 grouped MLP needs d and f multiples of %d (got %lld, %lld)",
          moe::kMxPad, static_cast<long long>(d), static_cast<long long>(f));
  return MOE_OK;
}

int64_t padded_tokens(int64_t Tk, int32_t E) {
  const int64_t p = moe::kMxPad;
  return (Tk + (p - 1) * static_cast<int64_t>(E)) / p * p;
}

// Forward MX workspace: S as codes [Tk][f] and scales [Tk][f/32].
struct MxFwdWorkspace {
  size_t sq = 0, ss = 0, total = 0;
};

MxFwdWorkspace mx_fwd_layout(int64_t Tk, int64_t f) {
  MxFwdWorkspace w;
  size_t off = 0;
  w.sq = off; off += align256(static_cast<size_t>(Tk * f));
  w.ss = off; off += align256(static_cast<size_t>(Tk * f / 32));
  w.total = off;
  return w;
}

// Backward MX workspace: every backward GEMM operand in MX form.
//   doq/dos   dO rows along d           [Tk][d], [Tk][d/32]
//   w2t*      W2 along d, transposed    [f][E d], [f][E d/32]
//   wgut*     W_gu along 2f, transposed [d][E 2f], [d][E 2f/32]
//   dabq/dabs dAB rows along 2f         [Tk][2f], [Tk][2f/32]
//   *t        token-axis operands of the weight gradients, transposed
//             [cols][Tk_pad] codes and [cols][Tk_pad/32] scales
struct MxBwdWorkspace {
  size_t doq, dos, w2tq, w2ts, wgutq, wguts, dabq, dabs;
  size_t dot, dots, st, sts, dabt, dabts, xpt, xpts;
  size_t total;
  int64_t tk_pad;
};

MxBwdWorkspace mx_bwd_layout(int64_t Tk, int32_t E, int64_t d, int64_t f,
                             size_t base) {
  MxBwdWorkspace w;
  size_t off = base;
  auto take = [&](int64_t bytes) {
    const size_t o = off;
    off += align256(static_cast<size_t>(bytes));
    return o;
  };
  const int64_t tp = padded_tokens(Tk, E);
  w.tk_pad = tp;
  w.doq = take(Tk * d);            w.dos = take(Tk * d / 32);
  w.w2tq = take(E * d * f);        w.w2ts = take(E * d * f / 32);
  w.wgutq = take(E * 2 * f * d);   w.wguts = take(E * 2 * f * d / 32);
  w.dabq = take(Tk * 2 * f);       w.dabs = take(Tk * 2 * f / 32);
  w.dot = take(d * tp);            w.dots = take(d * tp / 32);
  w.st = take(f * tp);             w.sts = take(f * tp / 32);
  w.dabt = take(2 * f * tp);       w.dabts = take(2 * f * tp / 32);
  w.xpt = take(d * tp);            w.xpts = take(d * tp / 32);
  w.total = off;
  return w;
}

struct BwdWorkspace {
  size_t dab = 0, dp_part = 0, total = 0;
};

// The MX backward keeps no bf16 dAB (its epilogue writes both MX forms):
// its workspace starts with dp_part alone.
size_t mx_bwd_base(int64_t Tk, int64_t f) {
  return align256(static_cast<size_t>(Tk * moe::gemm_dp_tiles(f) * 4));
}

// Optional token-axis MX output (codes [cols][ldt], scales [cols][ldt/32]):
// both pointers or neither; ldt a multiple of 128 holding every expert's
// padded rows.
moe_status check_tok_out(const char* what, const void* codes,
                         const void* scales, int64_t ldt, int64_t Tk,
                         int32_t E, int64_t cols) {
  if (!codes && !scales) return MOE_OK;
  REQUIRE(codes && scales, MOE_ERR_INVALID_ARG,
          "%s: token-axis codes and scales go together", what);
  REQUIRE(aligned16(codes) && aligned16(scales), MOE_ERR_INVALID_ARG,
          "%s: token-axis outputs must be 16-byte aligned", what);
  REQUIRE(ldt % 128 == 0 && ldt >= padded_tokens(Tk, E), MOE_ERR_INVALID_ARG,
          "%s: ldt must be a multiple of 128 and >= %lld (got %lld)", what,
          static_cast<long long>(padded_tokens(Tk, E)),
          static_cast<long long>(ldt));
  REQUIRE(cols * ldt <= (int64_t{1} << 40), MOE_ERR_UNSUPPORTED,
          "%s: token-axis output too large", what);
  return MOE_OK;
}

BwdWorkspace bwd_layout(int64_t Tk, int64_t f) {
  BwdWorkspace w;
  w.dab = 0;
  size_t off = align256(static_cast<size_t>(Tk * 2 * f * 2));
  w.dp_part = off;
  off += align256(static_cast<size_t>(Tk * moe::gemm_dp_tiles(f) * 4));
  w.total = off;
  return w;
}

}  // namespace

namespace {

// Validation shared by the two permutation entries (everything but the
// workspace); the launch order of both.
moe_status permute_check(moe_prec prec, const int32_t* topk_idx,
                         const float* topk_w, int64_t T, int32_t E, int32_t k,
                         const void* x, const uint8_t* x_scales, int64_t d,
                         int32_t* counts, int32_t* offsets, int32_t* pos,
                         int32_t* src, float* w_perm, void* x_perm,
                         uint8_t* x_perm_scales) {
  if (moe_status st = check_prec(prec)) return st;
  REQUIRE_PTR(topk_idx);
  REQUIRE_OPT_PTR(topk_w);
  REQUIRE_PTR(x);
  REQUIRE_PTR(counts);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(pos);
  REQUIRE_PTR(src);
  REQUIRE_OPT_PTR(w_perm);
  REQUIRE_PTR(x_perm);
  REQUIRE(!(w_perm && !topk_w), MOE_ERR_INVALID_ARG,
          "w_perm given without topk_w");
  if (moe_status st = check_route_dims(T, E, k)) return st;
  if (moe_status st = check_feature("d", d, prec)) return st;
  const int64_t row_bytes = act_row_bytes(prec, d);
  REQUIRE(T * k * row_bytes <= kMaxBytes * 4, MOE_ERR_UNSUPPORTED,
          "permuted tensor too large");
  if (is_mx(prec)) {
    REQUIRE_PTR(x_scales);
    REQUIRE_PTR(x_perm_scales);
  }
  return MOE_OK;
}

moe_status permute_launch(moe_prec prec, const int32_t* topk_idx,
                          const float* topk_w, int64_t T, int32_t E,
                          int32_t k, const void* x, const uint8_t* x_scales,
                          int64_t d, int32_t* counts, int32_t* offsets,
                          int32_t* pos, int32_t* src, float* w_perm,
                          void* x_perm, uint8_t* x_perm_scales, void* ws,
                          hipStream_t stream) {
  const int64_t row_bytes = act_row_bytes(prec, d);
  hipError_t e = moe::launch_plan(topk_idx, T, E, k, counts, offsets, pos,
                                  ws, stream);
  if (e != hipSuccess) return hip_status(e, "moe_permute/plan");
  const bool mx = is_mx(prec);
  e = moe::launch_scatter(topk_idx, topk_w, T, E, k, offsets, pos, src,
                          topk_w ? w_perm : nullptr, x, row_bytes, x_perm,
                          mx ? x_scales : nullptr, mx ? d / 32 : 0,
                          mx ? x_perm_scales : nullptr, ws, stream);
  return hip_status(e, "moe_permute/scatter");
}

}  // namespace

// ------------------------------------------------------- allocation-free
// Scratch of moe_permute_noalloc: a fixed array in device memory, one copy
// on every GPU the library runs on, held until the process ends.  On the
// host the array's name is only a stand-in; kernels get the device address
// that hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current GPU's scratch (looked up on its first use,
// with that device current).
moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "moe_permute_noalloc/hipGetDevice");
  REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_ERR_UNSUPPORTED,
          "device index %d is beyond the %d the library tracks", dev,
          kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
      return hip_status(e, "moe_permute_noalloc/hipGetSymbolAddress");
    REQUIRE(p != nullptr, MOE_ERR_HIP,
            "moe_permute_noalloc: no device address for the scratch array");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

const char* moe_version(void) { return "libmoe 0.1 gfx950"; }

size_t moe_workspace_bytes(moe_entry entry, moe_prec prec, int64_t T,
                           int32_t E, int32_t k, int64_t d, int64_t f) {
  if (T < 1 || E < 1 || E > moe::kMaxExperts || k < 1 || k > E) return 0;
  if (prec != MOE_BF16 && !is_mx(prec)) return 0;
  const int64_t Tk = T * k;
  switch (entry) {
    case MOE_ENTRY_PERMUTE:
      return moe::plan_workspace_bytes(Tk, E);
    case MOE_ENTRY_MLP_FWD:
      if (prec == MOE_BF16 || f < 1) return 0;
      return mx_fwd_layout(Tk, f).total;
    case MOE_ENTRY_ROUTER_BWD:
      return moe::router_backward_workspace(T, E, d < 1 ? 1 : d);
    case MOE_ENTRY_MLP_BWD:
      if (f < 1 || d < 1) return 0;
      if (prec == MOE_BF16) return bwd_layout(Tk, f).total;
      return mx_bwd_layout(Tk, E, d, f, mx_bwd_base(Tk, f)).total;
  }
  return 0;
}

moe_status moe_router_logits(const void* x, const void* w_g, const float* bias,
                             int64_t T, int64_t d, int32_t E, float* logits,
                             hipStream_t stream) {
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_g);
  REQUIRE_OPT_PTR(bias);
  REQUIRE_PTR(logits);
  REQUIRE(T >= 1, MOE_ERR_INVALID_ARG, "T must be >= 1");
  REQUIRE(E >= 1 && E <= moe::kMaxExperts, MOE_ERR_INVALID_ARG,
          "E must be in [1, %d]", moe::kMaxExperts);
  if (moe_status st = check_feature("d", d, MOE_BF16)) return st;
  REQUIRE(T * d * 2 <= kMaxBytes && E * d * 2 <= kMaxBytes,
          MOE_ERR_UNSUPPORTED, "tensor larger than 2 GiB");
  return hip_status(moe::launch_router_logits(static_cast<const bf16_t*>(x),
                                              static_cast<const bf16_t*>(w_g),
                                              bias, T, d, E, logits, stream),
                    "moe_router_logits");
}

moe_status moe_route(const float* logits, int64_t T, int32_t E, int32_t k,
                     int32_t renorm, int32_t* topk_idx, float* topk_w,
                     hipStream_t stream) {
  REQUIRE_PTR(logits);
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(topk_w);
  if (moe_status st = check_route_dims(T, E, k)) return st;
  return hip_status(
      moe::launch_route(logits, T, E, k, renorm ? 1 : 0, topk_idx, topk_w,
                        stream),
      "moe_route");
}

moe_status moe_router_backward(const float* logits, const int32_t* topk_idx,
                               const float* topk_w, const float* dp,
                               const int32_t* counts, float aux_coef,
                               int64_t T, int32_t E, int32_t k,
                               int32_t renorm, const void* x, const void* w_g,
                               int64_t d, float* dlogits, float* dw_g,
                               float* db, const float* dx_in, void* dx_out,
                               float* aux_loss, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  REQUIRE_PTR(logits);
  REQUIRE_PTR(topk_idx);
  REQUIRE_PTR(topk_w);
  REQUIRE_PTR(dp);
  REQUIRE_OPT_PTR(counts);
  REQUIRE_PTR(dlogits);
  REQUIRE_OPT_PTR(dw_g);
  REQUIRE_OPT_PTR(db);
  REQUIRE_OPT_PTR(dx_in);
  REQUIRE_OPT_PTR(dx_out);
  REQUIRE_OPT_PTR(aux_loss);
  if (moe_status st = check_route_dims(T, E, k)) return st;
  const bool need_x = dw_g != nullptr;
  const bool need_w = dx_out != nullptr;
  if (need_x) REQUIRE_PTR(x);
  if (need_w) REQUIRE_PTR(w_g);
  if (need_x || need_w) {
    if (moe_status st = check_feature("d", d, MOE_BF16)) return st;
    REQUIRE(T * d * 4 <= kMaxBytes * 2, MOE_ERR_UNSUPPORTED,
            "T x d too large");
  }
  REQUIRE(!(aux_loss && !counts), MOE_ERR_INVALID_ARG,
          "aux_loss needs counts");
  const size_t need = moe::router_backward_workspace(T, E, d > 0 ? d : 1);
  REQUIRE(workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  REQUIRE_PTR(workspace);
  return hip_status(
      moe::launch_router_backward(
          logits, topk_idx, topk_w, dp, counts, aux_coef, T, E, k, renorm,
          static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(w_g), d,
          dlogits, dw_g, db, dx_in, static_cast<bf16_t*>(dx_out), aux_loss,
          workspace, stream),
      "moe_router_backward");
}

moe_status moe_permute(moe_prec prec, const int32_t* topk_idx,
                       const float* topk_w, int64_t T, int32_t E, int32_t k,
                       const void* x, const uint8_t* x_scales, int64_t d,
                       int32_t* counts, int32_t* offsets, int32_t* pos,
                       int32_t* src, float* w_perm, void* x_perm,
                       uint8_t* x_perm_scales, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (moe_status st = permute_check(prec, topk_idx, topk_w, T, E, k, x,
                                    x_scales, d, counts, offsets, pos, src,
                                    w_perm, x_perm, x_perm_scales))
    return st;
  const size_t need = moe::plan_workspace_bytes(T * k, E);
  REQUIRE(workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  REQUIRE_PTR(workspace);
  return permute_launch(prec, topk_idx, topk_w, T, E, k, x, x_scales, d,
                        counts, offsets, pos, src, w_perm, x_perm,
                        x_perm_scales, workspace, stream);
}

moe_status moe_permute_noalloc(moe_prec prec, const int32_t* topk_idx,
                               const float* topk_w, int64_t T, int32_t E,
                               int32_t k, const void* x,
                               const uint8_t* x_scales, int64_t d,
                               int32_t* counts, int32_t* offsets,
                               int32_t* pos, int32_t* src, float* w_perm,
                               void* x_perm, uint8_t* x_perm_scales,
                               hipStream_t stream) {
  if (moe_status st = permute_check(prec, topk_idx, topk_w, T, E, k, x,
                                    x_scales, d, counts, offsets, pos, src,
                                    w_perm, x_perm, x_perm_scales))
    return st;
  const size_t need = moe::plan_workspace_bytes(T * k, E);
  REQUIRE(need <= MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_UNSUPPORTED,
          "moe_permute_noalloc: the plan of T*k = %lld slots over E = %d "
          "experts needs %zu bytes of scratch, above its %zu-byte limit "
          "(use moe_permute with a workspace)",
          static_cast<long long>(T) * k, E, need,
          static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (moe_status st = scratch_of_current_device(&ws)) return st;
  return permute_launch(prec, topk_idx, topk_w, T, E, k, x, x_scales, d,
                        counts, offsets, pos, src, w_perm, x_perm,
                        x_perm_scales, ws, stream);
}

moe_status moe_permute_rows(moe_prec prec, const int32_t* pos, int64_t T,
                            int32_t k, const void* x, const uint8_t* x_scales,
                            int64_t d, void* x_perm, uint8_t* x_perm_scales,
                            hipStream_t stream) {
  if (moe_status st = check_prec(prec)) return st;
  REQUIRE_PTR(pos);
  REQUIRE_PTR(x);
  REQUIRE_PTR(x_perm);
  REQUIRE(T >= 1, MOE_ERR_INVALID_ARG, "T must be >= 1");
  REQUIRE(k >= 1 && k <= moe::kMaxTopK, MOE_ERR_INVALID_ARG,
          "k must be in [1, %d]", moe::kMaxTopK);
  if (moe_status st = check_feature("d", d, prec)) return st;
  const bool mx = is_mx(prec);
  if (mx) {
    REQUIRE_PTR(x_scales);
    REQUIRE_PTR(x_perm_scales);
  }
  const int64_t row_bytes = act_row_bytes(prec, d);
  return hip_status(
      moe::launch_permute_rows(pos, T, k, x, row_bytes, x_perm,
                               mx ? x_scales : nullptr, mx ? d / 32 : 0,
                               mx ? x_perm_scales : nullptr, stream),
      "moe_permute_rows");
}

moe_status moe_grouped_mlp_fwd(moe_prec prec, const void* x_perm,
                               const uint8_t* x_perm_scales,
                               const int32_t* offsets, int32_t E, int64_t Tk,
                               int64_t d, int64_t f, const void* w_gu,
                               const uint8_t* w_gu_scales, const void* w2,
                               const uint8_t* w2_scales, const float* w_perm,
                               void* ab_saved, void* s_saved, void* out_perm,
                               uint8_t* s_tok, uint8_t* s_tok_scales,
                               int64_t ldt, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  if (moe_status st = check_prec(prec)) return st;
  REQUIRE_PTR(x_perm);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w_gu);
  REQUIRE_PTR(w2);
  REQUIRE_OPT_PTR(w_perm);
  REQUIRE_PTR(ab_saved);
  REQUIRE_OPT_PTR(s_saved);
  REQUIRE_PTR(out_perm);
  REQUIRE(is_mx(prec) || (!s_tok && !s_tok_scales), MOE_ERR_INVALID_ARG,
          "token-axis S codes are an MX output");
  REQUIRE(s_saved || (is_mx(prec) && s_tok), MOE_ERR_INVALID_ARG,
          "s_saved is NULL (it may be only with MX token-axis S codes)");
  REQUIRE(E >= 1 && E <= moe::kMaxExperts, MOE_ERR_INVALID_ARG,
          "E must be in [1, %d]", moe::kMaxExperts);
  REQUIRE(Tk >= 1, MOE_ERR_INVALID_ARG, "Tk must be >= 1");
  if (moe_status st = check_feature("d", d, prec)) return st;
  if (moe_status st = check_feature("f", f, prec)) return st;
  REQUIRE(2 * f * d * 2 <= kMaxRange, MOE_ERR_UNSUPPORTED,
          "one expert's weight is larger than 4 GiB");
  if (is_mx(prec)) {
    if (moe_status st = check_mx_dims(d, f)) return st;
    REQUIRE_PTR(x_perm_scales);
    REQUIRE_PTR(w_gu_scales);
    REQUIRE_PTR(w2_scales);
    if (moe_status st = check_tok_out("moe_grouped_mlp_fwd", s_tok,
                                      s_tok_scales, ldt, Tk, E, f))
      return st;
    const MxFwdWorkspace L = mx_fwd_layout(Tk, f);
    REQUIRE(workspace_bytes >= L.total, MOE_ERR_WORKSPACE,
            "workspace too small: %zu < %zu bytes", workspace_bytes, L.total);
    REQUIRE_PTR(workspace);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    hipError_t e = moe::gemm_mx_fc1_fwd(
        static_cast<const uint8_t*>(x_perm), x_perm_scales,
        prec == MOE_MXFP4, static_cast<const uint8_t*>(w_gu), w_gu_scales,
        offsets, E, Tk, d, f,
        w_perm, static_cast<bf16_t*>(ab_saved), static_cast<bf16_t*>(s_saved),
        ws + L.sq, ws + L.ss, s_tok, s_tok_scales, ldt, stream);
    if (e != hipSuccess) return hip_status(e, "moe_grouped_mlp_fwd/mx_fc1");
    e = moe::gemm_mx_fc2_fwd(ws + L.sq, ws + L.ss,
                             static_cast<const uint8_t*>(w2), w2_scales,
                             offsets, E, Tk, d, f,
                             static_cast<float*>(out_perm), stream);
    return hip_status(e, "moe_grouped_mlp_fwd/mx_fc2");
  }
  hipError_t e = moe::gemm_fc1_fwd(
      static_cast<const bf16_t*>(x_perm), static_cast<const bf16_t*>(w_gu),
      offsets, E, Tk, d, f, w_perm, static_cast<bf16_t*>(ab_saved),
      static_cast<bf16_t*>(s_saved), stream);
  if (e != hipSuccess) return hip_status(e, "moe_grouped_mlp_fwd/fc1");
  e = moe::gemm_fc2_fwd(static_cast<const bf16_t*>(s_saved),
                        static_cast<const bf16_t*>(w2), offsets, E, Tk, d, f,
                        static_cast<float*>(out_perm), stream);
  return hip_status(e, "moe_grouped_mlp_fwd/fc2");
}

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
                               hipStream_t stream) {
  if (moe_status st = check_prec(prec)) return st;
  REQUIRE_OPT_PTR(w_gu_col_codes);
  REQUIRE_OPT_PTR(w_gu_col_scales);
  REQUIRE_OPT_PTR(w2_col_codes);
  REQUIRE_OPT_PTR(w2_col_scales);
  REQUIRE(!w_gu_col_codes == !w_gu_col_scales &&
              !w2_col_codes == !w2_col_scales,
          MOE_ERR_INVALID_ARG,
          "column codes and their scales come together or not at all");
  REQUIRE(is_mx(prec) || (!w_gu_col_codes && !w2_col_codes),
          MOE_ERR_INVALID_ARG, "column weight codes are an MX input");
  REQUIRE_PTR(dout_perm);
  REQUIRE_PTR(x_perm);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(pos);
  REQUIRE_PTR(w_gu);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(ab_saved);
  REQUIRE_OPT_PTR(s_saved);
  REQUIRE_OPT_PTR(w_perm);
  REQUIRE_PTR(dx_perm);
  REQUIRE(is_mx(prec) || (!s_tok && !s_tok_scales), MOE_ERR_INVALID_ARG,
          "token-axis S codes are an MX input");
  REQUIRE(s_saved || (is_mx(prec) && s_tok), MOE_ERR_INVALID_ARG,
          "s_saved is NULL (it may be only with MX token-axis S codes)");
  if (prec == MOE_MXFP4) REQUIRE_PTR(x_perm_scales);
  REQUIRE_PTR(dw_gu);
  REQUIRE_PTR(dw2);
  REQUIRE_PTR(dp);
  if (moe_status st = check_route_dims(T, E, k)) return st;
  if (moe_status st = check_feature("d", d, prec)) return st;
  if (moe_status st = check_feature("f", f, prec)) return st;
  const int64_t Tk = T * k;
  // the weight gradients read each expert's rows of dAB (2f wide) and of
  // the permuted x / dO (d wide) through one resource; an expert may hold
  // every row
  REQUIRE(2 * f * d * 2 <= kMaxRange && Tk * 2 * f * 2 <= kMaxRange &&
              Tk * d * 2 <= kMaxRange,
          MOE_ERR_UNSUPPORTED,
          "T*k rows of 2f bf16 values, or one expert's weight, exceed 4 GiB");
  const BwdWorkspace L = bwd_layout(Tk, f);
  if (is_mx(prec)) {
    if (moe_status st = check_mx_dims(d, f)) return st;
    if (moe_status st = check_tok_out("moe_grouped_mlp_bwd", s_tok,
                                      s_tok_scales, ldt, Tk, E, f))
      return st;
    REQUIRE(!s_tok || ldt == padded_tokens(Tk, E), MOE_ERR_INVALID_ARG,
            "ldt must be moe_mxfp8_padded_rows(T*k, E) = %lld (got %lld)",
            static_cast<long long>(padded_tokens(Tk, E)),
            static_cast<long long>(ldt));
    const MxBwdWorkspace X = mx_bwd_layout(Tk, E, d, f, mx_bwd_base(Tk, f));
    REQUIRE(2 * f * X.tk_pad <= kMaxRange && E * 2 * f * d <= kMaxRange,
            MOE_ERR_UNSUPPORTED, "MX operand larger than 4 GiB");
    REQUIRE(workspace_bytes >= X.total, MOE_ERR_WORKSPACE,
            "workspace too small: %zu < %zu bytes", workspace_bytes, X.total);
    REQUIRE_PTR(workspace);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* dp_part = reinterpret_cast<float*>(ws);
    const bf16_t* dO = static_cast<const bf16_t*>(dout_perm);
    const int64_t tp = X.tk_pad;
    hipError_t e;
#define MX_STEP(call, what)                                           \
    e = (call);                                                       \
    if (e != hipSuccess) return hip_status(e, "moe_grouped_mlp_bwd/" what)
    // operands of the data gradients: the weights' column codes come in
    // ready-made or are made here
    MX_STEP(moe::launch_mx_quant_rows(dO, Tk, d, ws + X.doq, ws + X.dos,
                                      stream), "quant_dO");
    const uint8_t* w2tq = w2_col_codes ? w2_col_codes : ws + X.w2tq;
    const uint8_t* w2ts = w2_col_scales ? w2_col_scales : ws + X.w2ts;
    const uint8_t* wgutq = w_gu_col_codes ? w_gu_col_codes : ws + X.wgutq;
    const uint8_t* wguts = w_gu_col_scales ? w_gu_col_scales : ws + X.wguts;
    if (!w2_col_codes)
      MX_STEP(moe::launch_mx_quant_tokens(static_cast<const bf16_t*>(w2),
                                          nullptr, E * d, f, nullptr, 1,
                                          ws + X.w2tq, ws + X.w2ts, E * d,
                                          stream), "quant_W2");
    if (!w_gu_col_codes)
      MX_STEP(moe::launch_mx_quant_tokens(static_cast<const bf16_t*>(w_gu),
                                          nullptr, E * 2 * f, d, nullptr, 1,
                                          ws + X.wgutq, ws + X.wguts,
                                          E * 2 * f, stream), "quant_W_gu");
    MX_STEP(moe::gemm_mx_fc2_dgrad(ws + X.doq, ws + X.dos, w2tq,
                                   w2ts, E * d, offsets, E, Tk, d, f,
                                   static_cast<const bf16_t*>(ab_saved),
                                   w_perm, nullptr, ws + X.dabq, ws + X.dabs,
                                   ws + X.dabt, ws + X.dabts, tp, dp_part,
                                   stream), "mx_fc2_dgrad");
    MX_STEP(moe::launch_dp_reduce(dp_part, moe::gemm_dp_tiles(f), pos, T, k,
                                  dp, stream), "dp");
    MX_STEP(moe::gemm_mx_fc1_dgrad(ws + X.dabq, ws + X.dabs, wgutq,
                                   wguts, E * 2 * f, offsets, E, Tk, d,
                                   f, static_cast<float*>(dx_perm), stream),
            "mx_fc1_dgrad");
    // token-axis operands of the weight gradients
    MX_STEP(moe::launch_mx_quant_tokens(dO, nullptr, Tk, d, offsets, E,
                                        ws + X.dot, ws + X.dots, tp, stream),
            "quant_dO_tokens");
    const uint8_t* st_c = s_tok;
    const uint8_t* st_s = s_tok_scales;
    if (!s_tok) {
      MX_STEP(moe::launch_mx_quant_tokens(
                  static_cast<const bf16_t*>(s_saved), nullptr, Tk, f,
                  offsets, E, ws + X.st, ws + X.sts, tp, stream),
              "quant_S_tokens");
      st_c = ws + X.st;
      st_s = ws + X.sts;
    }
    MX_STEP(moe::gemm_mx_wgrad(ws + X.dot, ws + X.dots, st_c, st_s, false,
                               tp, offsets, E, d, f,
                               static_cast<bf16_t*>(dw2), stream),
            "mx_dw2");
    // the dW_gu GEMM's Xp along tokens: E4M3 from the bf16 rows, or (MXFP4
    // activations) E2M1 converted from the MXFP4 payload rows
    const bool act4 = prec == MOE_MXFP4;
    if (act4) {
      MX_STEP(moe::launch_mx4_quant_tokens(x_perm, x_perm_scales, Tk, d,
                                           offsets, E, ws + X.xpt,
                                           ws + X.xpts, tp, stream),
              "convert_Xp_tokens");
    } else {
      MX_STEP(moe::launch_mx_quant_tokens(static_cast<const bf16_t*>(x_perm),
                                          nullptr, Tk, d, offsets, E,
                                          ws + X.xpt, ws + X.xpts, tp,
                                          stream),
              "quant_Xp_tokens");
    }
    MX_STEP(moe::gemm_mx_wgrad(ws + X.dabt, ws + X.dabts, ws + X.xpt,
                               ws + X.xpts, act4, tp, offsets, E, 2 * f, d,
                               static_cast<bf16_t*>(dw_gu), stream),
            "mx_dw_gu");
#undef MX_STEP
    return ok();
  }
  REQUIRE(workspace_bytes >= L.total, MOE_ERR_WORKSPACE,
          "workspace too small: %zu < %zu bytes", workspace_bytes, L.total);
  REQUIRE_PTR(workspace);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  bf16_t* dab = reinterpret_cast<bf16_t*>(ws + L.dab);
  float* dp_part = reinterpret_cast<float*>(ws + L.dp_part);
  const bf16_t* dO = static_cast<const bf16_t*>(dout_perm);
  const bf16_t* xp = static_cast<const bf16_t*>(x_perm);
  hipError_t e = moe::gemm_fc2_dgrad(
      dO, static_cast<const bf16_t*>(w2), offsets, E, Tk, d, f,
      static_cast<const bf16_t*>(ab_saved), w_perm, dab, dp_part, stream);
  if (e != hipSuccess) return hip_status(e, "moe_grouped_mlp_bwd/fc2_dgrad");
  e = moe::launch_dp_reduce(dp_part, moe::gemm_dp_tiles(f), pos, T, k, dp,
                            stream);
  if (e != hipSuccess) return hip_status(e, "moe_grouped_mlp_bwd/dp");
  e = moe::gemm_wgrad(dO, d, static_cast<const bf16_t*>(s_saved), f, offsets,
                      E, Tk, d, f, static_cast<bf16_t*>(dw2), stream);
  if (e != hipSuccess) return hip_status(e, "moe_grouped_mlp_bwd/dw2");
  e = moe::gemm_fc1_dgrad(dab, static_cast<const bf16_t*>(w_gu), offsets, E,
                          Tk, d, f, static_cast<float*>(dx_perm), stream);
  if (e != hipSuccess) return hip_status(e, "moe_grouped_mlp_bwd/fc1_dgrad");
  e = moe::gemm_wgrad(dab, 2 * f, xp, d, offsets, E, Tk, 2 * f, d,
                      static_cast<bf16_t*>(dw_gu), stream);
  return hip_status(e, "moe_grouped_mlp_bwd/dw_gu");
}

int32_t moe_row_planes(int64_t f) { return f >= 1 ? moe::out_planes(f) : 0; }

moe_status moe_unpermute(const void* o_perm, int32_t o_fp32,
                         int32_t o_planes, const int32_t* pos, const float* w,
                         int64_t T, int32_t k, int64_t d, int32_t y_fp32,
                         void* y, const float* dlogits, const void* w_g,
                         int32_t E, hipStream_t stream) {
  REQUIRE_PTR(o_perm);
  REQUIRE_PTR(pos);
  REQUIRE_OPT_PTR(w);
  REQUIRE_PTR(y);
  REQUIRE_OPT_PTR(dlogits);
  if (dlogits) {
    REQUIRE_PTR(w_g);
    REQUIRE(E >= 1 && E <= moe::kMaxExperts, MOE_ERR_INVALID_ARG,
            "E must be in [1, %d] with dlogits", moe::kMaxExperts);
    REQUIRE(E * d * 2 <= kMaxBytes, MOE_ERR_UNSUPPORTED,
            "router weight larger than 2 GiB");
  }
  REQUIRE(T >= 1, MOE_ERR_INVALID_ARG, "T must be >= 1");
  REQUIRE(k >= 1 && k <= moe::kMaxTopK, MOE_ERR_INVALID_ARG,
          "k must be in [1, %d]", moe::kMaxTopK);
  if (moe_status st = check_feature("d", d, MOE_BF16)) return st;
  REQUIRE(o_planes >= 1 && o_planes <= 8 && (o_fp32 || o_planes == 1),
          MOE_ERR_INVALID_ARG,
          "o_planes must be in [1, 8] (1 for bf16 rows), got %d", o_planes);
  REQUIRE(T * k * d * 4 <= kMaxBytes * 2, MOE_ERR_UNSUPPORTED,
          "plane larger than 4 GiB");
  return hip_status(
      moe::launch_unpermute(o_perm, o_fp32 ? 1 : 0, o_planes, pos, w, T, k, d,
                            y_fp32 ? 1 : 0, y, dlogits,
                            static_cast<const bf16_t*>(w_g),
                            dlogits ? E : 0, stream),
      "moe_unpermute");
}

int32_t moe_dp_tiles(int64_t f) {
  return f >= 1 ? moe::gemm_dp_tiles(f) : 0;
}

moe_status moe_gate_up_swiglu_fwd(const void* x_perm, const int32_t* offsets,
                                  int32_t E, int64_t Tk, int64_t d, int64_t f,
                                  const void* w_gu, const float* w_perm,
                                  void* ab_saved, void* s_saved,
                                  hipStream_t stream) {
  REQUIRE_PTR(x_perm);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w_gu);
  REQUIRE_OPT_PTR(w_perm);
  REQUIRE_PTR(ab_saved);
  REQUIRE_PTR(s_saved);
  if (moe_status st = check_mlp_dims(E, Tk, d, f, MOE_BF16)) return st;
  return hip_status(
      moe::gemm_fc1_fwd(static_cast<const bf16_t*>(x_perm),
                        static_cast<const bf16_t*>(w_gu), offsets, E, Tk, d, f,
                        w_perm, static_cast<bf16_t*>(ab_saved),
                        static_cast<bf16_t*>(s_saved), stream),
      "moe_gate_up_swiglu_fwd");
}

moe_status moe_down_fwd(const void* s_saved, const int32_t* offsets,
                        int32_t E, int64_t Tk, int64_t d, int64_t f,
                        const void* w2, float* out_perm, hipStream_t stream) {
  REQUIRE_PTR(s_saved);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(out_perm);
  if (moe_status st = check_mlp_dims(E, Tk, d, f, MOE_BF16)) return st;
  return hip_status(
      moe::gemm_fc2_fwd(static_cast<const bf16_t*>(s_saved),
                        static_cast<const bf16_t*>(w2), offsets, E, Tk, d, f,
                        out_perm, stream),
      "moe_down_fwd");
}

moe_status moe_down_swiglu_bwd(const void* dout_perm, const int32_t* offsets,
                               int32_t E, int64_t Tk, int64_t d, int64_t f,
                               const void* w2, const void* ab_saved,
                               const float* w_perm, void* dab, float* dp_part,
                               hipStream_t stream) {
  REQUIRE_PTR(dout_perm);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w2);
  REQUIRE_PTR(ab_saved);
  REQUIRE_OPT_PTR(w_perm);
  REQUIRE_PTR(dab);
  REQUIRE_PTR(dp_part);
  if (moe_status st = check_mlp_dims(E, Tk, d, f, MOE_BF16)) return st;
  return hip_status(
      moe::gemm_fc2_dgrad(static_cast<const bf16_t*>(dout_perm),
                          static_cast<const bf16_t*>(w2), offsets, E, Tk, d, f,
                          static_cast<const bf16_t*>(ab_saved), w_perm,
                          static_cast<bf16_t*>(dab), dp_part, stream),
      "moe_down_swiglu_bwd");
}

moe_status moe_gate_up_dgrad(const void* dab, const int32_t* offsets,
                             int32_t E, int64_t Tk, int64_t d, int64_t f,
                             const void* w_gu, float* dx_perm,
                             hipStream_t stream) {
  REQUIRE_PTR(dab);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w_gu);
  REQUIRE_PTR(dx_perm);
  if (moe_status st = check_mlp_dims(E, Tk, d, f, MOE_BF16)) return st;
  return hip_status(
      moe::gemm_fc1_dgrad(static_cast<const bf16_t*>(dab),
                          static_cast<const bf16_t*>(w_gu), offsets, E, Tk, d,
                          f, dx_perm, stream),
      "moe_gate_up_dgrad");
}

moe_status moe_grouped_wgrad(const void* a, int64_t lda, const void* b,
                             int64_t ldb, const int32_t* offsets, int32_t E,
                             int64_t Tk, int64_t M, int64_t N, void* c,
                             hipStream_t stream) {
  REQUIRE_PTR(a);
  REQUIRE_PTR(b);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(c);
  REQUIRE(E >= 1 && E <= moe::kMaxExperts, MOE_ERR_INVALID_ARG,
          "E must be in [1, %d]", moe::kMaxExperts);
  REQUIRE(Tk >= 1, MOE_ERR_INVALID_ARG, "Tk must be >= 1");
  if (moe_status st = check_feature("M", M, MOE_BF16)) return st;
  if (moe_status st = check_feature("N", N, MOE_BF16)) return st;
  REQUIRE(lda >= M && lda % 8 == 0 && ldb >= N && ldb % 8 == 0,
          MOE_ERR_INVALID_ARG, "need lda >= M, ldb >= N, both multiples of 8");
  REQUIRE(Tk * lda * 2 <= kMaxRange && Tk * ldb * 2 <= kMaxRange &&
              M * N * 2 * static_cast<int64_t>(E) <= kMaxBytes * 8,
          MOE_ERR_UNSUPPORTED, "operand rows of one expert exceed 4 GiB");
  return hip_status(
      moe::gemm_wgrad(static_cast<const bf16_t*>(a), lda,
                      static_cast<const bf16_t*>(b), ldb, offsets, E, Tk, M, N,
                      static_cast<bf16_t*>(c), stream),
      "moe_grouped_wgrad");
}

moe_status moe_dp_reduce(const float* dp_part, int32_t ntiles,
                         const int32_t* pos, int64_t T, int32_t k, float* dp,
                         hipStream_t stream) {
  REQUIRE_PTR(dp_part);
  REQUIRE_PTR(pos);
  REQUIRE_PTR(dp);
  REQUIRE(T >= 1 && k >= 1 && ntiles >= 1, MOE_ERR_INVALID_ARG,
          "T, k and ntiles must be >= 1");
  return hip_status(moe::launch_dp_reduce(dp_part, ntiles, pos, T, k, dp,
                                          stream),
                    "moe_dp_reduce");
}

// ------------------------------------------------------------ MX stages

moe_status moe_mx_gate_up_swiglu_fwd(
    const uint8_t* xq, const uint8_t* xs, int32_t x_fp4,
    const int32_t* offsets, int32_t E,
    int64_t Tk, int64_t d, int64_t f, const uint8_t* wq, const uint8_t* ws,
    const float* w_perm, void* ab_saved, void* s_saved, uint8_t* sq,
    uint8_t* ss, uint8_t* s_tok, uint8_t* s_tok_scales, int64_t ldt,
    hipStream_t stream) {
  REQUIRE_PTR(xq); REQUIRE_PTR(xs); REQUIRE_PTR(offsets);
  REQUIRE_PTR(wq); REQUIRE_PTR(ws); REQUIRE_OPT_PTR(w_perm);
  REQUIRE_PTR(ab_saved); REQUIRE_OPT_PTR(s_saved); REQUIRE_PTR(sq);
  REQUIRE_PTR(ss);
  if (moe_status st = check_mlp_dims(E, Tk, d, f, MOE_MXFP8)) return st;
  if (moe_status st = check_mx_dims(d, f)) return st;
  if (moe_status st = check_tok_out("moe_mx_gate_up_swiglu_fwd", s_tok,
                                    s_tok_scales, ldt, Tk, E, f))
    return st;
  return hip_status(
      moe::gemm_mx_fc1_fwd(xq, xs, x_fp4 != 0, wq, ws, offsets, E, Tk, d, f,
                           w_perm,
                           static_cast<bf16_t*>(ab_saved),
                           static_cast<bf16_t*>(s_saved), sq, ss, s_tok,
                           s_tok_scales, ldt, stream),
      "moe_mx_gate_up_swiglu_fwd");
}

moe_status moe_mx_down_fwd(const uint8_t* sq, const uint8_t* ss,
                           const int32_t* offsets, int32_t E, int64_t Tk,
                           int64_t d, int64_t f, const uint8_t* wq,
                           const uint8_t* ws, float* out_perm,
                           hipStream_t stream) {
  REQUIRE_PTR(sq); REQUIRE_PTR(ss); REQUIRE_PTR(offsets);
  REQUIRE_PTR(wq); REQUIRE_PTR(ws); REQUIRE_PTR(out_perm);
  if (moe_status st = check_mlp_dims(E, Tk, d, f, MOE_MXFP8)) return st;
  if (moe_status st = check_mx_dims(d, f)) return st;
  return hip_status(moe::gemm_mx_fc2_fwd(sq, ss, wq, ws, offsets, E, Tk, d,
                                         f, out_perm, stream),
                    "moe_mx_down_fwd");
}

moe_status moe_mx_down_swiglu_bwd(
    const uint8_t* doq, const uint8_t* dos, const int32_t* offsets,
    int32_t E, int64_t Tk, int64_t d, int64_t f, const uint8_t* w2tq,
    const uint8_t* w2ts, const void* ab_saved, const float* w_perm,
    void* dab, uint8_t* dabq, uint8_t* dabs, uint8_t* dab_tok,
    uint8_t* dab_tok_scales, int64_t ldt, float* dp_part,
    hipStream_t stream) {
  REQUIRE_PTR(doq); REQUIRE_PTR(dos); REQUIRE_PTR(offsets);
  REQUIRE_PTR(w2tq); REQUIRE_PTR(w2ts); REQUIRE_PTR(ab_saved);
  REQUIRE_OPT_PTR(w_perm); REQUIRE_OPT_PTR(dab); REQUIRE_PTR(dabq);
  REQUIRE_PTR(dabs); REQUIRE_PTR(dp_part);
  if (moe_status st = check_mlp_dims(E, Tk, d, f, MOE_MXFP8)) return st;
  if (moe_status st = check_mx_dims(d, f)) return st;
  if (moe_status st = check_tok_out("moe_mx_down_swiglu_bwd", dab_tok,
                                    dab_tok_scales, ldt, Tk, E, 2 * f))
    return st;
  return hip_status(
      moe::gemm_mx_fc2_dgrad(doq, dos, w2tq, w2ts, E * d, offsets, E, Tk, d,
                             f, static_cast<const bf16_t*>(ab_saved), w_perm,
                             static_cast<bf16_t*>(dab), dabq, dabs, dab_tok,
                             dab_tok_scales, ldt, dp_part, stream),
      "moe_mx_down_swiglu_bwd");
}

moe_status moe_mx_gate_up_dgrad(const uint8_t* dabq, const uint8_t* dabs,
                                const int32_t* offsets, int32_t E, int64_t Tk,
                                int64_t d, int64_t f, const uint8_t* wgutq,
                                const uint8_t* wguts, float* dx_perm,
                                hipStream_t stream) {
  REQUIRE_PTR(dabq); REQUIRE_PTR(dabs); REQUIRE_PTR(offsets);
  REQUIRE_PTR(wgutq); REQUIRE_PTR(wguts); REQUIRE_PTR(dx_perm);
  if (moe_status st = check_mlp_dims(E, Tk, d, f, MOE_MXFP8)) return st;
  if (moe_status st = check_mx_dims(d, f)) return st;
  return hip_status(
      moe::gemm_mx_fc1_dgrad(dabq, dabs, wgutq, wguts, E * 2 * f, offsets, E,
                             Tk, d, f, dx_perm, stream),
      "moe_mx_gate_up_dgrad");
}

moe_status moe_mx_grouped_wgrad(const uint8_t* aq, const uint8_t* as,
                                const uint8_t* bq, const uint8_t* bs,
                                int32_t b_fp4, int64_t ldt,
                                const int32_t* offsets,
                                int32_t E, int64_t Tk, int64_t M, int64_t N,
                                void* c, hipStream_t stream) {
  REQUIRE_PTR(aq); REQUIRE_PTR(as); REQUIRE_PTR(bq); REQUIRE_PTR(bs);
  REQUIRE_PTR(offsets); REQUIRE_PTR(c);
  REQUIRE(E >= 1 && E <= moe::kMaxExperts, MOE_ERR_INVALID_ARG,
          "E must be in [1, %d]", moe::kMaxExperts);
  REQUIRE(Tk >= 1, MOE_ERR_INVALID_ARG, "Tk must be >= 1");
  if (moe_status st = check_feature("M", M, MOE_BF16)) return st;
  if (moe_status st = check_feature("N", N, MOE_BF16)) return st;
  REQUIRE(ldt % moe::kMxPad == 0 && ldt >= padded_tokens(Tk, E),
          MOE_ERR_INVALID_ARG,
          "ldt must be a multiple of %d and >= moe_mxfp8_padded_rows(Tk, E)",
          moe::kMxPad);
  REQUIRE(M * ldt <= kMaxRange && N * ldt <= kMaxRange &&
              M * N * 2 * static_cast<int64_t>(E) <= kMaxBytes * 8,
          MOE_ERR_UNSUPPORTED, "token-axis operand larger than 4 GiB");
  return hip_status(moe::gemm_mx_wgrad(aq, as, bq, bs, b_fp4 != 0, ldt,
                                       offsets, E, M, N,
                                       static_cast<bf16_t*>(c), stream),
                    "moe_mx_grouped_wgrad");
}

int64_t moe_mxfp8_padded_rows(int64_t rows, int32_t nseg) {
  if (rows < 0 || nseg < 1) return 0;
  const int64_t p = moe::kMxPad;
  return (rows + (p - 1) * static_cast<int64_t>(nseg)) / p * p;
}

moe_status moe_mxfp8_quantize(const void* src, int64_t rows, int64_t cols,
                              int32_t axis, const int32_t* seg_offsets,
                              int32_t nseg, uint8_t* codes, uint8_t* scales,
                              int64_t rows_pad, hipStream_t stream) {
  REQUIRE_PTR(src);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  REQUIRE(rows >= 1 && cols >= 1, MOE_ERR_INVALID_ARG,
          "rows and cols must be >= 1");
  REQUIRE(rows * cols * 2 <= kMaxBytes * 2, MOE_ERR_UNSUPPORTED,
          "source larger than 4 GiB");
  const bf16_t* s = static_cast<const bf16_t*>(src);
  if (axis == 0) {
    REQUIRE(cols % 32 == 0, MOE_ERR_INVALID_ARG,
            "axis 0 needs cols %% 32 == 0 (got %lld)",
            static_cast<long long>(cols));
    return hip_status(moe::launch_mx_quant_rows(s, rows, cols, codes, scales,
                                                stream),
                      "moe_mxfp8_quantize/rows");
  }
  REQUIRE(axis == 1, MOE_ERR_INVALID_ARG, "axis must be 0 or 1");
  REQUIRE(nseg >= 1 && nseg <= moe::kMaxExperts, MOE_ERR_INVALID_ARG,
          "nseg must be in [1, %d]", moe::kMaxExperts);
  REQUIRE(seg_offsets != nullptr || nseg == 1, MOE_ERR_INVALID_ARG,
          "seg_offsets may be NULL only for one segment");
  REQUIRE_OPT_PTR(seg_offsets);
  REQUIRE(cols % 8 == 0, MOE_ERR_INVALID_ARG, "axis 1 needs cols %% 8 == 0");
  REQUIRE(rows_pad >= moe_mxfp8_padded_rows(rows, nseg) &&
              rows_pad % moe::kMxPad == 0,
          MOE_ERR_INVALID_ARG,
          "rows_pad must be a multiple of %d and >= moe_mxfp8_padded_rows",
          moe::kMxPad);
  REQUIRE(cols * rows_pad <= kMaxBytes * 2, MOE_ERR_UNSUPPORTED,
          "output larger than 4 GiB");
  return hip_status(moe::launch_mx_quant_tokens(s, nullptr, rows, cols,
                                                seg_offsets, nseg, codes,
                                                scales, rows_pad, stream),
                    "moe_mxfp8_quantize/tokens");
}

moe_status moe_mxfp8_quantize_weight(const void* src, int64_t rows,
                                     int64_t cols, uint8_t* row_codes,
                                     uint8_t* row_scales, uint8_t* col_codes,
                                     uint8_t* col_scales,
                                     hipStream_t stream) {
  REQUIRE_PTR(src);
  REQUIRE_PTR(row_codes);
  REQUIRE_PTR(row_scales);
  REQUIRE_PTR(col_codes);
  REQUIRE_PTR(col_scales);
  REQUIRE(rows >= 1 && cols >= 1, MOE_ERR_INVALID_ARG,
          "rows and cols must be >= 1");
  REQUIRE(rows % moe::kMxPad == 0 && cols % 64 == 0, MOE_ERR_INVALID_ARG,
          "rows must be a multiple of %d and cols of 64 (got %lld, %lld)",
          moe::kMxPad, static_cast<long long>(rows),
          static_cast<long long>(cols));
  REQUIRE(rows * cols * 2 <= kMaxBytes * 2, MOE_ERR_UNSUPPORTED,
          "source larger than 4 GiB");
  return hip_status(
      moe::launch_mx_quant_both(static_cast<const bf16_t*>(src), rows, cols,
                                row_codes, row_scales, col_codes, col_scales,
                                stream),
      "moe_mxfp8_quantize_weight");
}

moe_status moe_mxfp4_quantize(const void* src, int32_t src_fmt,
                              const uint8_t* src_scales, int64_t rows,
                              int64_t cols, int32_t axis,
                              const int32_t* seg_offsets, int32_t nseg,
                              uint8_t* codes, uint8_t* scales,
                              int64_t rows_pad, hipStream_t stream) {
  REQUIRE_PTR(src);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  REQUIRE(src_fmt == 0 || src_fmt == 1, MOE_ERR_INVALID_ARG,
          "src_fmt must be 0 (bf16) or 1 (MXFP4 rows)");
  if (src_fmt == 1) REQUIRE_PTR(src_scales);
  REQUIRE(rows >= 1 && cols >= 1, MOE_ERR_INVALID_ARG,
          "rows and cols must be >= 1");
  REQUIRE(cols % 32 == 0, MOE_ERR_INVALID_ARG,
          "cols must be a multiple of 32 (got %lld)",
          static_cast<long long>(cols));
  REQUIRE(rows * cols * 2 <= kMaxBytes * 2, MOE_ERR_UNSUPPORTED,
          "source larger than 4 GiB");
  if (axis == 0) {
    REQUIRE(src_fmt == 0, MOE_ERR_INVALID_ARG,
            "axis 0 quantizes bf16 rows (src_fmt 0)");
    return hip_status(
        moe::launch_mx4_quant_rows(static_cast<const bf16_t*>(src), rows,
                                   cols, codes, scales, stream),
        "moe_mxfp4_quantize/rows");
  }
  REQUIRE(axis == 1, MOE_ERR_INVALID_ARG, "axis must be 0 or 1");
  REQUIRE(nseg >= 1 && nseg <= moe::kMaxExperts, MOE_ERR_INVALID_ARG,
          "nseg must be in [1, %d]", moe::kMaxExperts);
  REQUIRE(seg_offsets != nullptr || nseg == 1, MOE_ERR_INVALID_ARG,
          "seg_offsets may be NULL only for one segment");
  REQUIRE_OPT_PTR(seg_offsets);
  REQUIRE(rows_pad >= moe_mxfp8_padded_rows(rows, nseg) &&
              rows_pad % moe::kMxPad == 0,
          MOE_ERR_INVALID_ARG,
          "rows_pad must be a multiple of %d and >= moe_mxfp8_padded_rows",
          moe::kMxPad);
  REQUIRE(cols * rows_pad <= kMaxBytes * 4, MOE_ERR_UNSUPPORTED,
          "output larger than 4 GiB");
  return hip_status(
      moe::launch_mx4_quant_tokens(src, src_fmt == 1 ? src_scales : nullptr,
                                   rows, cols, seg_offsets, nseg, codes,
                                   scales, rows_pad, stream),
      "moe_mxfp4_quantize/tokens");
}

}  // extern "C"
