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
backward, dAB for the weight gradients).  Arithmetic between quantization
points is float64.  Each function is the plain composition of the float64
step functions of ``moe_ref`` and the codec of ``mx_ref``; nothing is
blocked or fused.

Pinned by tests/test_oracle_mx_layer_pins.py: a dense masked formulation
(every expert on every token, no dispatch plan) whose quantizer is torch's
float8_e4m3fn cast with independently computed block scales; exactness on
inputs that are MX-representable along the documented axis only; the
reduction to the plain layer when no block loses precision; and the
per-element MX error bound.
"""

import numpy as np

from . import moe_ref as R
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


def experts_forward_mx(x, idx, p, w_gu, w2):
    """Forward with routing given.  Returns the bf16 path's dict plus the
    dequantized GEMM operands (xq, w_gu_q, w2_q, s_q)."""
    x = np.asarray(x, dtype=np.float64)
    w_gu = np.asarray(w_gu, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    E = w_gu.shape[0]
    f = w_gu.shape[1] // 2
    d = x.shape[1]
    counts, offsets, pos, src = R.dispatch_plan(idx, E)
    xq = mx_rows(x)
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
                ab=ab, s=s, s_q=s_q, o=o, y=y)


def moe_forward_mx(x, logits, w_gu, w2, k, renorm=True):
    """Route on the given scores, then the MX forward."""
    idx, p = R.topk_route(logits, k, renorm)
    return experts_forward_mx(x, idx, p, w_gu, w2)


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
    xp_t = mx_tokens(xp, offsets)
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
