"""Python binding of libmoe.so (see include/moe.h for the semantics).

Argument marshalling only: each function checks that the torch tensors have
the dtype, device and contiguity the C-ABI expects, passes their device
pointers and the current HIP stream, and raises MoeError on a non-zero
status.  All compute happens in the library's kernels.  Importing this
module fails loudly when libmoe.so has not been built.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_BF16 = 0
MOE_MXFP8 = 1
MOE_MXFP4 = 2
MOE_ENTRY_PERMUTE = 0
MOE_ENTRY_MLP_FWD = 1
MOE_ENTRY_MLP_BWD = 2
MOE_ENTRY_ROUTER_BWD = 3

EXPORTED = [
    "moe_status_str", "moe_last_error", "moe_version", "moe_router_logits",
    "moe_route", "moe_permute", "moe_permute_rows", "moe_grouped_mlp_fwd",
    "moe_grouped_mlp_bwd", "moe_unpermute", "moe_mxfp8_quantize",
    "moe_mxfp8_quantize_weight",
    "moe_mxfp8_padded_rows", "moe_workspace_bytes", "moe_dp_tiles",
    "moe_gate_up_swiglu_fwd", "moe_down_fwd", "moe_down_swiglu_bwd",
    "moe_gate_up_dgrad", "moe_grouped_wgrad", "moe_dp_reduce",
    "moe_row_planes", "moe_mx_gate_up_swiglu_fwd", "moe_mx_down_fwd",
    "moe_mx_down_swiglu_bwd", "moe_mx_gate_up_dgrad", "moe_mx_grouped_wgrad",
    "moe_router_backward", "moe_mxfp4_quantize", "moe_permute_noalloc",
]
# fixed per-GPU scratch of moe_permute_noalloc (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 2 << 20


class MoeError(RuntimeError):
    def __init__(self, name, status, status_str, message):
        super().__init__(f"{name} failed: {status_str}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m mixture_experts_expert_top_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                       ctypes.c_size_t)
    sig = {
        "moe_status_str": (ctypes.c_char_p, [I32]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_version": (ctypes.c_char_p, []),
        "moe_router_logits": (I32, [P, P, P, I64, I64, I32, P, P]),
        "moe_route": (I32, [P, I64, I32, I32, I32, P, P, P]),
        "moe_permute": (I32, [I32, P, P, I64, I32, I32, P, P, I64, P, P, P,
                              P, P, P, P, P, SZ, P]),
        "moe_permute_noalloc": (I32, [I32, P, P, I64, I32, I32, P, P, I64,
                                      P, P, P, P, P, P, P, P]),
        "moe_permute_rows": (I32, [I32, P, I64, I32, P, P, I64, P, P, P]),
        "moe_grouped_mlp_fwd": (I32, [I32, P, P, P, I32, I64, I64, I64, P, P,
                                      P, P, P, P, P, P, P, P, I64, P, SZ,
                                      P]),
        "moe_grouped_mlp_bwd": (I32, [I32, P, P, P, P, P, I64, I32, I32,
                                      I64, I64, P, P, P, P, P, P, I64, P, P,
                                      P, P, P, P, P, P, P, P, SZ, P]),
        "moe_unpermute": (I32, [P, I32, I32, P, P, I64, I32, I64, I32, P,
                                P, P, I32, P]),
        "moe_row_planes": (I32, [I64]),
        "moe_mxfp8_quantize": (I32, [P, I64, I64, I32, P, I32, P, P, I64, P]),
        "moe_mxfp8_quantize_weight": (I32, [P, I64, I64, P, P, P, P, P]),
        "moe_mxfp8_padded_rows": (I64, [I64, I32]),
        "moe_mxfp4_quantize": (I32, [P, I32, P, I64, I64, I32, P, I32, P, P,
                                     I64, P]),
        "moe_workspace_bytes": (SZ, [I32, I32, I64, I32, I32, I64, I64]),
        "moe_dp_tiles": (I32, [I64]),
        "moe_gate_up_swiglu_fwd": (I32, [P, P, I32, I64, I64, I64, P, P, P,
                                         P, P]),
        "moe_down_fwd": (I32, [P, P, I32, I64, I64, I64, P, P, P]),
        "moe_down_swiglu_bwd": (I32, [P, P, I32, I64, I64, I64, P, P, P, P,
                                      P, P]),
        "moe_gate_up_dgrad": (I32, [P, P, I32, I64, I64, I64, P, P, P]),
        "moe_grouped_wgrad": (I32, [P, I64, P, I64, P, I32, I64, I64, I64, P,
                                    P]),
        "moe_dp_reduce": (I32, [P, I32, P, I64, I32, P, P]),
        "moe_mx_gate_up_swiglu_fwd": (I32, [P, P, I32, P, I32, I64, I64, I64,
                                            P, P, P, P, P, P, P, P, P, I64,
                                            P]),
        "moe_mx_down_fwd": (I32, [P, P, P, I32, I64, I64, I64, P, P, P, P]),
        "moe_mx_down_swiglu_bwd": (I32, [P, P, P, I32, I64, I64, I64, P, P,
                                         P, P, P, P, P, P, P, I64, P, P]),
        "moe_mx_gate_up_dgrad": (I32, [P, P, P, I32, I64, I64, I64, P, P, P,
                                       P]),
        "moe_mx_grouped_wgrad": (I32, [P, P, P, P, I32, I64, P, I32, I64,
                                       I64, I64, P, P]),
        "moe_router_backward": (I32, [P, P, P, P, P, ctypes.c_float, I64,
                                      I32, I32, I32, P, P, I64, P, P, P, P,
                                      P, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _p(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(name, status):
    if status != 0:
        raise MoeError(name, status, lib.moe_status_str(status).decode(),
                       lib.moe_last_error().decode())


def _want(t, name, dtype, shape=None, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, "
                         f"got {tuple(t.shape)}")


def version():
    return lib.moe_version().decode()




def row_planes(f):
    """Partial-sum planes of out_perm / dx_perm for intermediate width f."""
    return int(lib.moe_row_planes(int(f)))


def moe_workspace_bytes(entry, prec, T, E, k, d, f):
    return int(lib.moe_workspace_bytes(entry, prec, T, E, k, d, f))


def moe_router_logits(x, w_g, bias, logits, stream=None):
    T, d = x.shape
    E = w_g.shape[0]
    _want(x, "x", torch.bfloat16)
    _want(w_g, "w_g", torch.bfloat16, (E, d))
    _want(bias, "bias", torch.float32, (E,), allow_none=True)
    _want(logits, "logits", torch.float32, (T, E))
    _check("moe_router_logits", lib.moe_router_logits(
        _p(x), _p(w_g), _p(bias), T, d, E, _p(logits), _stream(stream)))


def moe_route(logits, k, renorm, topk_idx, topk_w, stream=None):
    T, E = logits.shape
    _want(logits, "logits", torch.float32)
    _want(topk_idx, "topk_idx", torch.int32, (T, k))
    _want(topk_w, "topk_w", torch.float32, (T, k))
    _check("moe_route", lib.moe_route(_p(logits), T, E, k, int(renorm),
                                      _p(topk_idx), _p(topk_w),
                                      _stream(stream)))


def moe_router_backward(logits, topk_idx, topk_w, dp, counts, aux_coef,
                        renorm, x, w_g, dlogits, dw_g, db, dx_in, dx_out,
                        aux_loss, workspace, stream=None):
    T, E = logits.shape
    k = topk_idx.shape[1]
    d = (x if x is not None else w_g).shape[1] if (
        x is not None or w_g is not None) else 0
    _want(logits, "logits", torch.float32)
    _want(topk_idx, "topk_idx", torch.int32, (T, k))
    _want(topk_w, "topk_w", torch.float32, (T, k))
    _want(dp, "dp", torch.float32, (T, k))
    _want(counts, "counts", torch.int32, (E,), allow_none=True)
    _want(x, "x", torch.bfloat16, (T, d), allow_none=True)
    _want(w_g, "w_g", torch.bfloat16, (E, d), allow_none=True)
    _want(dlogits, "dlogits", torch.float32, (T, E))
    _want(dw_g, "dw_g", torch.float32, (E, d), allow_none=True)
    _want(db, "db", torch.float32, (E,), allow_none=True)
    _want(dx_in, "dx_in", torch.float32, (T, d), allow_none=True)
    _want(dx_out, "dx_out", torch.bfloat16, (T, d), allow_none=True)
    _want(aux_loss, "aux_loss", torch.float32, (1,), allow_none=True)
    nbytes = workspace.numel() * workspace.element_size() if workspace \
        is not None else 0
    _check("moe_router_backward", lib.moe_router_backward(
        _p(logits), _p(topk_idx), _p(topk_w), _p(dp), _p(counts),
        float(aux_coef), T, E, k, int(renorm), _p(x), _p(w_g), d,
        _p(dlogits), _p(dw_g), _p(db), _p(dx_in), _p(dx_out), _p(aux_loss),
        _p(workspace), nbytes, _stream(stream)))


def _permute_args(prec, topk_idx, topk_w, E, x, x_scales, counts, offsets,
                  pos, src, w_perm, x_perm, x_perm_scales):
    T, k = topk_idx.shape
    xdt, per = _act(prec, x, "x")
    w = x.shape[1]
    d = w * per
    _want(topk_idx, "topk_idx", torch.int32)
    _want(topk_w, "topk_w", torch.float32, (T, k), allow_none=True)
    _want(x, "x", xdt, (T, w))
    _want(x_perm, "x_perm", xdt, (T * k, w))
    if prec != MOE_BF16:
        _want(x_scales, "x_scales", torch.uint8, (T, d // 32))
        _want(x_perm_scales, "x_perm_scales", torch.uint8, (T * k, d // 32))
    for n, t, shp in (("counts", counts, (E,)), ("offsets", offsets, (E + 1,)),
                      ("pos", pos, (T, k)), ("src", src, (T * k,))):
        _want(t, n, torch.int32, shp)
    _want(w_perm, "w_perm", torch.float32, (T * k,), allow_none=True)
    return (prec, _p(topk_idx), _p(topk_w), T, E, k, _p(x), _p(x_scales), d,
            _p(counts), _p(offsets), _p(pos), _p(src), _p(w_perm), _p(x_perm),
            _p(x_perm_scales))


def moe_permute(prec, topk_idx, topk_w, E, x, x_scales, counts, offsets, pos,
                src, w_perm, x_perm, x_perm_scales, workspace, stream=None):
    args = _permute_args(prec, topk_idx, topk_w, E, x, x_scales, counts,
                         offsets, pos, src, w_perm, x_perm, x_perm_scales)
    nbytes = workspace.numel() * workspace.element_size() if workspace \
        is not None else 0
    _check("moe_permute", lib.moe_permute(*args, _p(workspace), nbytes,
                                          _stream(stream)))


def moe_permute_noalloc(prec, topk_idx, topk_w, E, x, x_scales, counts,
                        offsets, pos, src, w_perm, x_perm, x_perm_scales,
                        stream=None):
    args = _permute_args(prec, topk_idx, topk_w, E, x, x_scales, counts,
                         offsets, pos, src, w_perm, x_perm, x_perm_scales)
    _check("moe_permute_noalloc", lib.moe_permute_noalloc(*args,
                                                          _stream(stream)))


def moe_permute_rows(prec, pos, x, x_scales, x_perm, x_perm_scales,
                     stream=None):
    T, k = pos.shape
    xdt, per = _act(prec, x, "x")
    w = x.shape[1]
    d = w * per
    _want(pos, "pos", torch.int32)
    _want(x, "x", xdt, (T, w))
    _want(x_perm, "x_perm", xdt, (T * k, w))
    _check("moe_permute_rows", lib.moe_permute_rows(
        prec, _p(pos), T, k, _p(x), _p(x_scales), d, _p(x_perm),
        _p(x_perm_scales), _stream(stream)))


def _act(prec, x, what):
    """(dtype, values per stored element) of an activation tensor: bf16,
    E4M3 codes, or E2M1 codes two a byte."""
    if prec == MOE_BF16:
        return torch.bfloat16, 1
    return torch.uint8, (2 if prec == MOE_MXFP4 else 1)


def _tok_out(name, codes, scales, cols):
    """(ldt, codes, scales) of an optional token-axis MX tensor
    ([cols][ldt] codes, [cols][ldt/32] scales)."""
    if codes is None and scales is None:
        return 0
    ldt = codes.shape[1]
    _want(codes, name, torch.uint8, (cols, ldt))
    _want(scales, name + "_scales", torch.uint8, (cols, ldt // 32))
    return ldt


def moe_grouped_mlp_fwd(prec, x_perm, x_perm_scales, offsets, w_gu,
                        w_gu_scales, w2, w2_scales, w_perm, ab_saved, s_saved,
                        out_perm, workspace=None, stream=None, s_tok=None,
                        s_tok_scales=None):
    Tk = x_perm.shape[0]
    E, two_f, d = w_gu.shape
    f = two_f // 2
    _want(offsets, "offsets", torch.int32, (E + 1,))
    xdt, per = _act(prec, x_perm, "x_perm")
    _want(x_perm, "x_perm", xdt, (Tk, d // per))
    if prec == MOE_BF16:
        _want(x_perm, "x_perm", torch.bfloat16)
        _want(w_gu, "w_gu", torch.bfloat16, (E, 2 * f, d))
        _want(w2, "w2", torch.bfloat16, (E, d, f))
    _want(w_perm, "w_perm", torch.float32, (Tk,), allow_none=True)
    _want(ab_saved, "ab_saved", torch.bfloat16, (Tk, 2 * f))
    _want(s_saved, "s_saved", torch.bfloat16, (Tk, f), allow_none=True)
    _want(out_perm, "out_perm", torch.float32, (row_planes(f), Tk, d))
    ldt = _tok_out("s_tok", s_tok, s_tok_scales, f)
    nbytes = workspace.numel() * workspace.element_size() if workspace \
        is not None else 0
    _check("moe_grouped_mlp_fwd", lib.moe_grouped_mlp_fwd(
        prec, _p(x_perm), _p(x_perm_scales), _p(offsets), E, Tk, d, f,
        _p(w_gu), _p(w_gu_scales), _p(w2), _p(w2_scales), _p(w_perm),
        _p(ab_saved), _p(s_saved), _p(out_perm), _p(s_tok), _p(s_tok_scales),
        ldt, _p(workspace), nbytes, _stream(stream)))


def moe_grouped_mlp_bwd(prec, dout_perm, x_perm, offsets, pos, w_gu, w2,
                        ab_saved, s_saved, w_perm, dx_perm, dw_gu, dw2, dp,
                        workspace, stream=None, s_tok=None, s_tok_scales=None,
                        x_perm_scales=None, w_gu_col=None, w2_col=None):
    """x_perm: bf16 rows (bf16 and MXFP8), or for MXFP4 the forward's
    payload, E2M1 codes [T*k, d/2] with x_perm_scales [T*k, d/32].
    w_gu_col / w2_col (MX): (codes, scales) of the weights along their
    columns as moe_mxfp8_quantize_weight makes them, codes [d, E*2f] /
    [f, E*d], scales [d, E*2f/32] / [f, E*d/32]; None to quantize inside
    the call."""
    Tk, d = dout_perm.shape
    T, k = pos.shape
    E, two_f, _ = w_gu.shape
    f = two_f // 2
    if prec == MOE_MXFP4:
        _want(x_perm, "x_perm", torch.uint8, (Tk, d // 2))
        _want(x_perm_scales, "x_perm_scales", torch.uint8, (Tk, d // 32))
    else:
        _want(x_perm, "x_perm", torch.bfloat16, (Tk, d))
    for n, t, shp in (("dout_perm", dout_perm, (Tk, d)),
                      ("w_gu", w_gu, (E, 2 * f, d)), ("w2", w2, (E, d, f)),
                      ("ab_saved", ab_saved, (Tk, 2 * f)),
                      ("dw_gu", dw_gu, (E, 2 * f, d)), ("dw2", dw2, (E, d, f))):
        _want(t, n, torch.bfloat16, shp)
    _want(s_saved, "s_saved", torch.bfloat16, (Tk, f), allow_none=True)
    ldt = _tok_out("s_tok", s_tok, s_tok_scales, f)
    _want(dx_perm, "dx_perm", torch.float32, (row_planes(f), Tk, d))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    _want(pos, "pos", torch.int32)
    _want(w_perm, "w_perm", torch.float32, (Tk,), allow_none=True)
    _want(dp, "dp", torch.float32, (T, k))
    cols = {}
    for n, pair, rows, width in (("w_gu_col", w_gu_col, d, E * 2 * f),
                                 ("w2_col", w2_col, f, E * d)):
        if pair is None:
            cols[n] = (None, None)
            continue
        codes, scales = pair
        _want(codes, n + " codes", torch.uint8, (rows, width))
        _want(scales, n + " scales", torch.uint8, (rows, width // 32))
        cols[n] = (codes, scales)
    nbytes = workspace.numel() * workspace.element_size() if workspace \
        is not None else 0
    _check("moe_grouped_mlp_bwd", lib.moe_grouped_mlp_bwd(
        prec, _p(dout_perm), _p(x_perm), _p(x_perm_scales), _p(offsets),
        _p(pos), T, k, E, d, f,
        _p(w_gu), _p(w2), _p(ab_saved), _p(s_saved), _p(s_tok),
        _p(s_tok_scales), ldt, _p(cols["w_gu_col"][0]),
        _p(cols["w_gu_col"][1]), _p(cols["w2_col"][0]),
        _p(cols["w2_col"][1]), _p(w_perm), _p(dx_perm), _p(dw_gu), _p(dw2),
        _p(dp), _p(workspace), nbytes, _stream(stream)))


def moe_unpermute(o_perm, pos, w, y, stream=None, dlogits=None, w_g=None):
    """o_perm: bf16 [T*k, d] rows, or fp32 [T*k, d] / [planes, T*k, d].
    dlogits (fp32 [T, E]) with w_g (bf16 [E, d]): add the router's share
    of the input gradient before the rounding."""
    T, k = pos.shape
    d = o_perm.shape[-1]
    if o_perm.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("o_perm must be bfloat16 or float32")
    planes = o_perm.shape[0] if o_perm.dim() == 3 else 1
    _want(o_perm, "o_perm", o_perm.dtype,
          (planes, T * k, d) if o_perm.dim() == 3 else (T * k, d))
    _want(pos, "pos", torch.int32)
    _want(w, "w", torch.float32, (T, k), allow_none=True)
    if y.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("y must be bfloat16 or float32")
    _want(y, "y", y.dtype, (T, d))
    E = 0
    if dlogits is not None:
        E = dlogits.shape[1]
        _want(dlogits, "dlogits", torch.float32, (T, E))
        _want(w_g, "w_g", torch.bfloat16, (E, d))
    _check("moe_unpermute", lib.moe_unpermute(
        _p(o_perm), 1 if o_perm.dtype == torch.float32 else 0, planes,
        _p(pos), _p(w), T, k, d,
        1 if y.dtype == torch.float32 else 0, _p(y), _p(dlogits),
        _p(w_g) if dlogits is not None else None, E, _stream(stream)))


def moe_mxfp8_padded_rows(rows, nseg):
    return int(lib.moe_mxfp8_padded_rows(rows, nseg))


def moe_mxfp8_quantize(src, axis, seg_offsets, codes, scales, rows_pad=0,
                       stream=None):
    rows, cols = src.shape
    _want(src, "src", torch.bfloat16)
    _want(codes, "codes", torch.uint8)
    _want(scales, "scales", torch.uint8)
    nseg = 1 if seg_offsets is None else seg_offsets.numel() - 1
    if seg_offsets is not None:
        _want(seg_offsets, "seg_offsets", torch.int32)
    _check("moe_mxfp8_quantize", lib.moe_mxfp8_quantize(
        _p(src), rows, cols, axis, _p(seg_offsets), nseg, _p(codes),
        _p(scales), rows_pad, _stream(stream)))


def moe_mxfp8_quantize_weight(src, row_codes, row_scales, col_codes,
                              col_scales, stream=None):
    """Both MX layouts of a bf16 [rows, cols] weight from one read:
    row_codes [rows, cols] / row_scales [rows, cols/32] (axis 0) and
    col_codes [cols, rows] / col_scales [cols, rows/32] (axis 1, one
    segment)."""
    rows, cols = src.shape
    _want(src, "src", torch.bfloat16)
    _want(row_codes, "row_codes", torch.uint8, (rows, cols))
    _want(row_scales, "row_scales", torch.uint8, (rows, cols // 32))
    _want(col_codes, "col_codes", torch.uint8, (cols, rows))
    _want(col_scales, "col_scales", torch.uint8, (cols, rows // 32))
    _check("moe_mxfp8_quantize_weight", lib.moe_mxfp8_quantize_weight(
        _p(src), rows, cols, _p(row_codes), _p(row_scales), _p(col_codes),
        _p(col_scales), _stream(stream)))


def moe_mxfp4_quantize(src, axis, seg_offsets, codes, scales, rows_pad=0,
                       src_scales=None, cols=None, stream=None):
    """src: bf16 [rows, cols], or (with src_scales) MXFP4 rows as uint8
    codes [rows, cols/2] with scales [rows, cols/32].  Codes are two a
    byte: axis 0 gives [rows, cols/2], axis 1 [cols, rows_pad/2]."""
    rows = src.shape[0]
    if src_scales is None:
        _want(src, "src", torch.bfloat16)
        cols = src.shape[1]
        fmt = 0
    else:
        cols = 2 * src.shape[1]
        _want(src, "src", torch.uint8)
        _want(src_scales, "src_scales", torch.uint8, (rows, cols // 32))
        fmt = 1
    _want(codes, "codes", torch.uint8)
    _want(scales, "scales", torch.uint8)
    nseg = 1 if seg_offsets is None else seg_offsets.numel() - 1
    if seg_offsets is not None:
        _want(seg_offsets, "seg_offsets", torch.int32)
    _check("moe_mxfp4_quantize", lib.moe_mxfp4_quantize(
        _p(src), fmt, _p(src_scales), rows, cols, axis, _p(seg_offsets),
        nseg, _p(codes), _p(scales), rows_pad, _stream(stream)))


# ---------------------------------------------------------------- stages

def moe_dp_tiles(f):
    return int(lib.moe_dp_tiles(f))


def _mlp_dims(x_perm, w_gu):
    Tk, d = x_perm.shape
    E, two_f, _ = w_gu.shape
    return Tk, d, E, two_f // 2


def moe_gate_up_swiglu_fwd(x_perm, offsets, w_gu, w_perm, ab_saved, s_saved,
                           stream=None):
    Tk, d, E, f = _mlp_dims(x_perm, w_gu)
    _want(x_perm, "x_perm", torch.bfloat16)
    _want(w_gu, "w_gu", torch.bfloat16, (E, 2 * f, d))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    _want(w_perm, "w_perm", torch.float32, (Tk,), allow_none=True)
    _want(ab_saved, "ab_saved", torch.bfloat16, (Tk, 2 * f))
    _want(s_saved, "s_saved", torch.bfloat16, (Tk, f))
    _check("moe_gate_up_swiglu_fwd", lib.moe_gate_up_swiglu_fwd(
        _p(x_perm), _p(offsets), E, Tk, d, f, _p(w_gu), _p(w_perm),
        _p(ab_saved), _p(s_saved), _stream(stream)))


def moe_down_fwd(s_saved, offsets, w2, out_perm, stream=None):
    Tk, f = s_saved.shape
    E, d, _ = w2.shape
    _want(s_saved, "s_saved", torch.bfloat16)
    _want(w2, "w2", torch.bfloat16, (E, d, f))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    _want(out_perm, "out_perm", torch.float32, (row_planes(f), Tk, d))
    _check("moe_down_fwd", lib.moe_down_fwd(
        _p(s_saved), _p(offsets), E, Tk, d, f, _p(w2), _p(out_perm),
        _stream(stream)))


def moe_down_swiglu_bwd(dout_perm, offsets, w2, ab_saved, w_perm, dab,
                        dp_part, stream=None):
    Tk, d = dout_perm.shape
    E, _, f = w2.shape
    _want(dout_perm, "dout_perm", torch.bfloat16)
    _want(w2, "w2", torch.bfloat16, (E, d, f))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    _want(ab_saved, "ab_saved", torch.bfloat16, (Tk, 2 * f))
    _want(w_perm, "w_perm", torch.float32, (Tk,), allow_none=True)
    _want(dab, "dab", torch.bfloat16, (Tk, 2 * f))
    _want(dp_part, "dp_part", torch.float32, (Tk, moe_dp_tiles(f)))
    _check("moe_down_swiglu_bwd", lib.moe_down_swiglu_bwd(
        _p(dout_perm), _p(offsets), E, Tk, d, f, _p(w2), _p(ab_saved),
        _p(w_perm), _p(dab), _p(dp_part), _stream(stream)))


def moe_gate_up_dgrad(dab, offsets, w_gu, dx_perm, stream=None):
    Tk, two_f = dab.shape
    E, _, d = w_gu.shape
    f = two_f // 2
    _want(dab, "dab", torch.bfloat16)
    _want(w_gu, "w_gu", torch.bfloat16, (E, 2 * f, d))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    _want(dx_perm, "dx_perm", torch.float32, (row_planes(f), Tk, d))
    _check("moe_gate_up_dgrad", lib.moe_gate_up_dgrad(
        _p(dab), _p(offsets), E, Tk, d, f, _p(w_gu), _p(dx_perm),
        _stream(stream)))


def moe_grouped_wgrad(a, b, offsets, c, stream=None):
    Tk, M = a.shape
    _, N = b.shape
    E = offsets.numel() - 1
    _want(a, "a", torch.bfloat16)
    _want(b, "b", torch.bfloat16, (Tk, N))
    _want(offsets, "offsets", torch.int32)
    _want(c, "c", torch.bfloat16, (E, M, N))
    _check("moe_grouped_wgrad", lib.moe_grouped_wgrad(
        _p(a), M, _p(b), N, _p(offsets), E, Tk, M, N, _p(c),
        _stream(stream)))


def moe_dp_reduce(dp_part, pos, dp, stream=None):
    T, k = pos.shape
    _want(dp_part, "dp_part", torch.float32)
    _want(pos, "pos", torch.int32)
    _want(dp, "dp", torch.float32, (T, k))
    _check("moe_dp_reduce", lib.moe_dp_reduce(
        _p(dp_part), dp_part.shape[1], _p(pos), T, k, _p(dp),
        _stream(stream)))


# ------------------------------------------------------------- MX stages
# Codes are uint8 tensors, scales uint8 tensors with one byte per 32 codes
# along the reduction axis (layouts in include/moe.h).

def moe_mx_gate_up_swiglu_fwd(xq, xs, offsets, wq, ws, w_perm, ab_saved,
                              s_saved, sq, ss, s_tok=None, s_tok_scales=None,
                              stream=None, x_fp4=False):
    """xq: E4M3 codes [T*k, d], or (x_fp4) E2M1 codes [T*k, d/2]."""
    Tk = xq.shape[0]
    E, two_f, d = wq.shape
    f = two_f // 2
    _want(xq, "xq", torch.uint8, (Tk, d // 2 if x_fp4 else d))
    _want(xs, "xs", torch.uint8, (Tk, d // 32))
    _want(wq, "wq", torch.uint8, (E, 2 * f, d))
    _want(ws, "ws", torch.uint8, (E, 2 * f, d // 32))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    _want(w_perm, "w_perm", torch.float32, (Tk,), allow_none=True)
    _want(ab_saved, "ab_saved", torch.bfloat16, (Tk, 2 * f))
    _want(s_saved, "s_saved", torch.bfloat16, (Tk, f), allow_none=True)
    _want(sq, "sq", torch.uint8, (Tk, f))
    _want(ss, "ss", torch.uint8, (Tk, f // 32))
    ldt = _tok_out("s_tok", s_tok, s_tok_scales, f)
    _check("moe_mx_gate_up_swiglu_fwd", lib.moe_mx_gate_up_swiglu_fwd(
        _p(xq), _p(xs), int(bool(x_fp4)), _p(offsets), E, Tk, d, f, _p(wq),
        _p(ws),
        _p(w_perm), _p(ab_saved), _p(s_saved), _p(sq), _p(ss), _p(s_tok),
        _p(s_tok_scales), ldt, _stream(stream)))


def moe_mx_down_fwd(sq, ss, offsets, wq, ws, out_perm, stream=None):
    Tk, f = sq.shape
    E, d, _ = wq.shape
    _want(sq, "sq", torch.uint8)
    _want(ss, "ss", torch.uint8, (Tk, f // 32))
    _want(wq, "wq", torch.uint8, (E, d, f))
    _want(ws, "ws", torch.uint8, (E, d, f // 32))
    _want(offsets, "offsets", torch.int32, (E + 1,))
    _want(out_perm, "out_perm", torch.float32, (row_planes(f), Tk, d))
    _check("moe_mx_down_fwd", lib.moe_mx_down_fwd(
        _p(sq), _p(ss), _p(offsets), E, Tk, d, f, _p(wq), _p(ws),
        _p(out_perm), _stream(stream)))


def moe_mx_down_swiglu_bwd(doq, dos, offsets, w2tq, w2ts, ab_saved, w_perm,
                           dab, dabq, dabs, dp_part, dab_tok=None,
                           dab_tok_scales=None, stream=None):
    Tk, d = doq.shape
    f, Ed = w2tq.shape
    E = offsets.numel() - 1
    _want(doq, "doq", torch.uint8)
    _want(dos, "dos", torch.uint8, (Tk, d // 32))
    _want(w2tq, "w2tq", torch.uint8, (f, E * d))
    _want(w2ts, "w2ts", torch.uint8, (f, E * d // 32))
    _want(offsets, "offsets", torch.int32)
    _want(ab_saved, "ab_saved", torch.bfloat16, (Tk, 2 * f))
    _want(w_perm, "w_perm", torch.float32, (Tk,), allow_none=True)
    _want(dab, "dab", torch.bfloat16, (Tk, 2 * f), allow_none=True)
    _want(dabq, "dabq", torch.uint8, (Tk, 2 * f))
    _want(dabs, "dabs", torch.uint8, (Tk, 2 * f // 32))
    _want(dp_part, "dp_part", torch.float32, (Tk, moe_dp_tiles(f)))
    ldt = _tok_out("dab_tok", dab_tok, dab_tok_scales, 2 * f)
    _check("moe_mx_down_swiglu_bwd", lib.moe_mx_down_swiglu_bwd(
        _p(doq), _p(dos), _p(offsets), E, Tk, d, f, _p(w2tq), _p(w2ts),
        _p(ab_saved), _p(w_perm), _p(dab), _p(dabq), _p(dabs), _p(dab_tok),
        _p(dab_tok_scales), ldt, _p(dp_part), _stream(stream)))


def moe_mx_gate_up_dgrad(dabq, dabs, offsets, wgutq, wguts, dx_perm,
                         stream=None):
    Tk, two_f = dabq.shape
    f = two_f // 2
    d = wgutq.shape[0]
    E = offsets.numel() - 1
    _want(dabq, "dabq", torch.uint8)
    _want(dabs, "dabs", torch.uint8, (Tk, two_f // 32))
    _want(wgutq, "wgutq", torch.uint8, (d, E * two_f))
    _want(wguts, "wguts", torch.uint8, (d, E * two_f // 32))
    _want(offsets, "offsets", torch.int32)
    _want(dx_perm, "dx_perm", torch.float32, (row_planes(f), Tk, d))
    _check("moe_mx_gate_up_dgrad", lib.moe_mx_gate_up_dgrad(
        _p(dabq), _p(dabs), _p(offsets), E, Tk, d, f, _p(wgutq), _p(wguts),
        _p(dx_perm), _stream(stream)))


def moe_mx_grouped_wgrad(aq, as_, bq, bs, offsets, Tk, c, stream=None,
                         b_fp4=False):
    """aq [M, ldt] E4M3 codes; bq [N, ldt] E4M3, or (b_fp4) E2M1 codes
    [N, ldt/2]."""
    M, ldt = aq.shape
    N = bq.shape[0]
    E = offsets.numel() - 1
    _want(aq, "aq", torch.uint8)
    _want(as_, "as", torch.uint8, (M, ldt // 32))
    _want(bq, "bq", torch.uint8, (N, ldt // 2 if b_fp4 else ldt))
    _want(bs, "bs", torch.uint8, (N, ldt // 32))
    _want(offsets, "offsets", torch.int32)
    _want(c, "c", torch.bfloat16, (E, M, N))
    _check("moe_mx_grouped_wgrad", lib.moe_mx_grouped_wgrad(
        _p(aq), _p(as_), _p(bq), _p(bs), int(bool(b_fp4)), ldt,
        _p(offsets), E, Tk, M, N, _p(c), _stream(stream)))
