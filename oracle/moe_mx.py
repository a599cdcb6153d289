"""The MoE expert-MLP layer with MXFP8 GEMM operands, forward and backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Efficient MoE Training for Biological Foundation Models", Challenge 2
(MXFP8 keeps 8-bit values with one scale per block of 32 consecutive
values) and Challenge 3 (the BF16 activations and weights are quantized
before the low-precision GEMMs, and the fused operators emit their outputs
already quantized).  The pages do not list the quantization points; the
reading taken here is that every GEMM operand is MX-coded in blocks of 32
along that GEMM's reduction axis, that a value is quantized from the
highest precision the producer holds, and that everything outside the GEMMs
(SwiGLU, its gradient, the routing weights, the combines) stays as in the
bf16 path:

  forward   x              along d         (before the permutation)
            W_gu           along d         (per row of [E, 2f, d])
            W2             along f         (per row of [E, d, f])
            S              along f         (from the unrounded S)
  backward  dY             along d         (before the permutation)
            W2             along d         (column-wise, per expert)
            dAB            along 2f        (from the unrounded dAB)
            W_gu           along 2f        (column-wise, per expert)
            dO, S, dAB, Xp along tokens    (blocks restart at each expert's
                                            first row; from the bf16 copies)

Stored activations are bfloat16 as in the bf16 path (AB and S for the
backward, dAB for the weight gradients).

The MXFP4-activation variant (``act4=True``; the hgpu.org abstract of the
MXFP4 MoE training recipe: FP8 GEMMs, MXFP4 activations and expert-parallel
payloads, FP4 row blocks converted to column blocks with new scales)
changes two points and nothing else:

  forward   x              MXFP4 along d   (the dispatched payload)
  backward  Xp             MXFP4 along tokens, from the dequantized MXFP4
                           payload (no bf16 copy of x is used)  Arithmetic between quantization
points is float64.  Each function is the plain composition of the float64
step functions of ``moe_ref`` and the codec of ``mx_ref``; nothing is
blocked or fused.

Pinned by tests/test_oracle_mx_layer_pins.py: a dense masked formulation
(every expert on every token, no dispatch plan) whose quantizer is torch's
float8_e4m3fn cast with independently computed block scales; exactness on
inputs that are MX-representable along the documented axis only; the
reduction to the plain layer when no block loses precision; the size of
the MX error against the exact layer; and the sampled single-output
helpers against the full layer.
"""

import numpy as np

from . import moe_ref as R
from . import mx4_ref as M4
from . import mx_ref as M


def mx_rows(a):
    """Quantize-dequantize along the last axis (blocks of 32 columns)."""
    a = np.asarray(a, dtype=np.float64)
    shape = a.shape
    c, s = M.quantize_rows(a.reshape(-1, shape[-1]))
    return M.dequantize_rows(c, s).reshape(shape)


def mx_cols(w):
    """Quantize-dequantize each expert's [R, C] matrix along R (blocks of
    32 consecutive rows of one column)."""
    w = np.asarray(w, dtype=np.float64)
    return np.stack([mx_rows(w[e].T).T for e in range(w.shape[0])])


def mx_tokens(a, offsets):
    """Quantize-dequantize along rows of a [Tk, C] permuted tensor, blocks
    of 32 rows restarting at every expert segment start."""
    c, blocks = M.quantize_segments(a, offsets)
    return M.dequantize_segments(c, blocks)


def mx4_rows(a):
    """MXFP4 quantize-dequantize along the last axis."""
    a = np.asarray(a, dtype=np.float64)
    shape = a.shape
    c, s = M4.quantize_rows4(a.reshape(-1, shape[-1]))
    return M4.dequantize_rows4(c, s).reshape(shape)


def mx4_tokens(a, offsets):
    """MXFP4 quantize-dequantize along the rows of a [Tk, C] permuted
    tensor, blocks restarting at every expert segment start."""
    c, blocks = M4.quantize_segments4(a, offsets)
    return M4.dequantize_segments4(c, blocks)


def _payload(x, act4):
    """x as the fc1 GEMM reads it: MX along d, MXFP4 or MXFP8."""
    return mx4_rows(x) if act4 else mx_rows(x)


def experts_forward_mx(x, idx, p, w_gu, w2, act4=False):
    """Forward with routing given.  Returns the bf16 path's dict plus the
    dequantized GEMM operands (xq, w_gu_q, w2_q, s_q)."""
    x = np.asarray(x, dtype=np.float64)
    w_gu = np.asarray(w_gu, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    E = w_gu.shape[0]
    f = w_gu.shape[1] // 2
    d = x.shape[1]
    counts, offsets, pos, src = R.dispatch_plan(idx, E)
    xq = _payload(x, act4)
    w_gu_q = mx_rows(w_gu)
    w2_q = mx_rows(w2)
    xp_q = R.permute_rows(xq, src)
    w_perm = R.permuted_weights(p, pos)
    Tk = xp_q.shape[0]
    ab = np.zeros((Tk, 2 * f))
    s = np.zeros((Tk, f))
    s_q = np.zeros((Tk, f))
    o = np.zeros((Tk, d))
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        ab_e = R.gate_up(xp_q[r0:r1], w_gu_q[e])
        s_e = R.scaled_swiglu(ab_e, w_perm[r0:r1])
        s_q[r0:r1] = mx_rows(s_e)
        o[r0:r1] = R.down(s_q[r0:r1], w2_q[e])
        ab[r0:r1] = R.bf16_round(ab_e)
        s[r0:r1] = R.bf16_round(s_e)
    y = R.combine(o, pos, idx)
    return dict(idx=np.asarray(idx), p=np.asarray(p, dtype=np.float64),
                counts=counts, offsets=offsets, pos=pos, src=src,
                xp=R.permute_rows(x, src), xp_q=xp_q, xq=xq,
                w_gu_q=w_gu_q, w2_q=w2_q, w_perm=w_perm,
                ab=ab, s=s, s_q=s_q, o=o, y=y, act4=act4)


def moe_forward_mx(x, logits, w_gu, w2, k, renorm=True, act4=False):
    """Route on the given scores, then the MX forward."""
    idx, p = R.topk_route(logits, k, renorm)
    return experts_forward_mx(x, idx, p, w_gu, w2, act4)


def moe_backward_mx(fwd, dy, w_gu, w2):
    """Backward of ``experts_forward_mx`` for the upstream gradient dy.

    Routing is held fixed.  Returns dict(dx, dw_gu, dw2, dp, dab) plus the
    dequantized operands of every backward GEMM."""
    dy = np.asarray(dy, dtype=np.float64)
    w_gu = np.asarray(w_gu, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    E, two_f, d = w_gu.shape
    offsets, pos, src = fwd["offsets"], fwd["pos"], fwd["src"]
    ab, s, xp, w_perm = fwd["ab"], fwd["s"], fwd["xp"], fwd["w_perm"]
    Tk = xp.shape[0]
    do = R.permute_rows(dy, src)               # bf16 values of dY rows
    do_q = R.permute_rows(mx_rows(dy), src)    # along d, before permuting
    w2_c = mx_cols(w2)                         # along d
    w_gu_c = mx_cols(w_gu)                     # along 2f
    do_t = mx_tokens(do, offsets)
    s_t = mx_tokens(s, offsets)
    # the weight gradient's Xp: MXFP8 along tokens from the bf16 rows, or
    # (act4) MXFP4 along tokens from the dequantized MXFP4 payload
    xp_t = (mx4_tokens(fwd["xp_q"], offsets) if fwd.get("act4")
            else mx_tokens(xp, offsets))
    dab = np.zeros((Tk, two_f))
    dab_q = np.zeros((Tk, two_f))
    dxp = np.zeros((Tk, d))
    dw_gu = np.zeros_like(w_gu)
    dw2 = np.zeros_like(w2)
    dp_perm = np.zeros(Tk)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        dw2[e] = R.wgrad(do_t[r0:r1], s_t[r0:r1])
        dab_e, dp_perm[r0:r1] = R.down_backward(do_q[r0:r1], ab[r0:r1],
                                                w_perm[r0:r1], w2_c[e])
        dab_q[r0:r1] = mx_rows(dab_e)
        dab[r0:r1] = R.bf16_round(dab_e)
        dxp[r0:r1] = R.gate_up_dgrad(dab_q[r0:r1], w_gu_c[e])
    dab_t = mx_tokens(dab, offsets)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            dw_gu[e] = R.wgrad(dab_t[r0:r1], xp_t[r0:r1])
    T, k = pos.shape
    dx = np.zeros((T, d))
    dp = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            dx[t] += dxp[pos[t, j]]
            dp[t, j] = dp_perm[pos[t, j]]
    return dict(dx=dx, dw_gu=dw_gu, dw2=dw2, dp=dp, dab=dab, dab_q=dab_q,
                do=do, do_q=do_q, do_t=do_t, s_t=s_t, xp_t=xp_t,
                dab_t=dab_t, w2_c=w2_c, w_gu_c=w_gu_c, dxp=dxp)


# --------------------------------------------------------------------------
# Sampled evaluation for full-size parity checks: the same definition for
# single outputs.  Row-wise blocks of a row depend on that row alone and
# token-axis blocks on one column alone, so each helper quantizes only the
# rows or columns it needs.
# --------------------------------------------------------------------------

def expert_weights_mx(w_gu_e=None, w2_e=None, backward=False):
    """Dequantized MX forms of one expert's weights: forward w_gu along d
    ("gu_q") and w2 along f ("w2_q"); with ``backward`` also w2 along d
    ("w2_c") and w_gu along 2f ("gu_c")."""
    out = {}
    if w_gu_e is not None:
        w_gu_e = np.asarray(w_gu_e, dtype=np.float64)
        out["gu_q"] = mx_rows(w_gu_e)
        if backward:
            out["gu_c"] = mx_rows(w_gu_e.T).T
    if w2_e is not None:
        w2_e = np.asarray(w2_e, dtype=np.float64)
        out["w2_q"] = mx_rows(w2_e)
        if backward:
            out["w2_c"] = mx_rows(w2_e.T).T
    return out


def token_forward_mx(x_t, idx_t, p_t, W, act4=False):
    """y[t] for one token: its experts' MX forward rows summed in ascending
    expert id.  W[e] holds expert_weights_mx(...) of every chosen e."""
    xq = _payload(np.asarray(x_t, dtype=np.float64)[None, :], act4)
    y = 0.0
    for j in np.argsort(np.asarray(idx_t), kind="stable"):
        e = int(idx_t[j])
        ab = R.gate_up(xq, W[e]["gu_q"])
        s = R.scaled_swiglu(ab, np.array([p_t[j]], dtype=np.float64))
        y = y + R.down(mx_rows(s), W[e]["w2_q"])[0]
    return y


def row_backward_mx(x_t, dy_t, p_r, We, act4=False):
    """(dXp row, dp) of the permuted row of token t at one expert, whose
    weights We come from expert_weights_mx(..., backward=True)."""
    xq = _payload(np.asarray(x_t, dtype=np.float64)[None, :], act4)
    ab = R.bf16_round(R.gate_up(xq, We["gu_q"]))
    do_q = mx_rows(np.asarray(dy_t, dtype=np.float64)[None, :])
    dab, dp = R.down_backward(do_q, ab, np.array([p_r], dtype=np.float64),
                              We["w2_c"])
    return R.gate_up_dgrad(mx_rows(dab), We["gu_c"])[0], dp[0]


def _gate_up_cols(x_e, w_gu_e, cols, act4=False):
    """Columns ``cols`` of the expert's AB (bf16 as kept), from x quantized
    along d and the needed W_gu rows quantized along d."""
    xq = _payload(np.asarray(x_e, dtype=np.float64), act4)
    wr = mx_rows(np.asarray(w_gu_e, dtype=np.float64)[cols])
    return R.bf16_round(xq @ wr.T)


def dw2_column_mx(x_e, dy_e, w_e, w_gu_e, j, act4=False):
    """Column j of the expert's dW2 (all d entries): dO (bf16 dY rows) and
    S[:, j] (bf16 S from the MX forward) quantized along the expert's
    tokens.  x_e, dy_e, w_e: the expert's rows in permuted order."""
    f = np.asarray(w_gu_e).shape[0] // 2
    xq = _payload(np.asarray(x_e, dtype=np.float64), act4)
    wr = mx_rows(np.asarray(w_gu_e, dtype=np.float64)[[j, f + j]])
    ab = xq @ wr.T
    s = R.bf16_round(np.asarray(w_e, dtype=np.float64) *
                     R.silu(ab[:, 0]) * ab[:, 1])
    n = s.shape[0]
    s_t = mx_tokens(s[:, None], [0, n])[:, 0]
    do_t = mx_tokens(np.asarray(dy_e, dtype=np.float64), [0, n])
    return do_t.T @ s_t


def dw_gu_row_mx(x_e, dy_e, w_e, w_gu_e, w2_e, i, act4=False):
    """Row i of the expert's dW_gu (gate row for i < f, up row f + i' for
    i = f + i'): dAB[:, i] (bf16, from dS = dO quantized along d times W2
    quantized along d) and Xp quantized along the expert's tokens."""
    w_gu_e = np.asarray(w_gu_e, dtype=np.float64)
    f = w_gu_e.shape[0] // 2
    c = i % f
    ab = _gate_up_cols(x_e, w_gu_e, [c, f + c], act4)
    g, u = ab[:, 0], ab[:, 1]
    do_q = mx_rows(np.asarray(dy_e, dtype=np.float64))
    w2col = mx_rows(np.asarray(w2_e, dtype=np.float64)[:, c][None, :])[0]
    ds = do_q @ w2col
    dh = np.asarray(w_e, dtype=np.float64) * ds
    sg = R.sigmoid(g)
    dab = dh * u * sg * (1.0 + g * (1.0 - sg)) if i < f else dh * R.silu(g)
    dab = R.bf16_round(dab)
    n = dab.shape[0]
    dab_t = mx_tokens(dab[:, None], [0, n])[:, 0]
    x_e = np.asarray(x_e, dtype=np.float64)
    xp_t = (mx4_tokens(mx4_rows(x_e), [0, n]) if act4
            else mx_tokens(x_e, [0, n]))
    return dab_t @ xp_t
