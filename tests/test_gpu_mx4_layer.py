"""GPU parity of the MXFP4-activation variant (MOE_MXFP4: MXFP8 GEMMs, the
dispatched x and the saved fc1 input as MXFP4) against the oracle
(oracle/moe_mx.py with act4=True).

Stage tests: the gate_up GEMM with its FP4 x operand, and the weight
gradient GEMM with an FP4 B operand, on the very same codes as the oracle
(the GPU's codes are checked bit-exact against the oracle codec first), to
the MFMA bound of the MXFP8 stage tests (2^-10 sum |a b| element by
element, propagated through SwiGLU).  Layer tests: MoEPathMX(act_fp4=True)
forward and backward against the MX-emulating oracle on seeded inputs,
gated on the relative RMS error at 1e-2 as the MXFP8 layer (the reasoning
is the same: single E4M3 codes of the epilogue-quantized S and dAB flip
with the MFMA's rounding; the MXFP4 payload and its token-axis conversion
are bit-exact on both sides), max|err|/rms reported; stage entries equal
the fused ones bitwise; reruns are bitwise equal.
"""

import numpy as np
import pytest
import torch

from mixture_experts_expert_top_amd import inputs as I
from oracle import moe_mx as X
from oracle import moe_ref as R
from oracle import mx4_ref as M4

gpu = pytest.mark.gpu
if torch.cuda.is_available():
    from mixture_experts_expert_top_amd import moe
    from mixture_experts_expert_top_amd.layer import MoEPathMX, StageTimers

# the MXFP8 layer test module supplies the shared stage helpers
from test_gpu_mx_layer import (MFMA_REL, SHAPES, IDS, _dev, _plan,  # noqa
                               _quant_rows_both, _segs, excess, h64,
                               mfma_err, mx_rounding_check, rel, rel_rms,
                               sig, tok_check, u8)

TOL_MX_RMS = 1e-2


def _quant_rows4_both(t):
    """GPU and oracle MXFP4 row quantization of a bf16 [R, C]; asserts the
    packed codes and scales agree; returns (codes_d, scales_d, float64
    dequantized)."""
    R_, C = t.shape
    q = torch.empty(R_, C // 2, dtype=torch.uint8, device=t.device)
    s = torch.empty(R_, C // 32, dtype=torch.uint8, device=t.device)
    moe.moe_mxfp4_quantize(t, 0, None, q, s)
    cq, cs = M4.quantize_rows4(h64(t))
    np.testing.assert_array_equal(u8(q), M4.pack_nibbles(cq))
    np.testing.assert_array_equal(u8(s), cs)
    return q, s, M4.dequantize_rows4(cq, cs)


@gpu
@pytest.mark.parametrize("name,T,d,f,E,k,bias", SHAPES, ids=IDS)
def test_mx4_gate_up_swiglu_stage(name, T, d, f, E, k, bias):
    dev = _dev()
    P = _plan(T, E, k, bias, seed=31)
    Tk = T * k
    xp = I.make_tensor((Tk, d), seed=1, device=dev)
    xp[::7] *= 50.0
    w_gu = I.make_tensor((E, 2 * f, d), seed=2, scale=0.1, device=dev)
    xq, xs, xd = _quant_rows4_both(xp)
    wq, ws, wd = _quant_rows_both(w_gu)
    ab = torch.empty(Tk, 2 * f, dtype=torch.bfloat16, device=dev)
    s = torch.empty(Tk, f, dtype=torch.bfloat16, device=dev)
    sq = torch.empty(Tk, f, dtype=torch.uint8, device=dev)
    ss = torch.empty(Tk, f // 32, dtype=torch.uint8, device=dev)
    tp = moe.moe_mxfp8_padded_rows(Tk, E)
    st = torch.full((f, tp), 0xA5, dtype=torch.uint8, device=dev)
    sts = torch.full((f, tp // 32), 0xA5, dtype=torch.uint8, device=dev)
    moe.moe_mx_gate_up_swiglu_fwd(xq, xs, P["offsets_d"], wq, ws,
                                  P["w_perm_d"], ab, s, sq, ss, s_tok=st,
                                  s_tok_scales=sts, x_fp4=True)
    torch.cuda.synchronize()
    ab_ref = np.zeros((Tk, 2 * f))
    ab_err = np.zeros((Tk, 2 * f))
    s_ref = np.zeros((Tk, f))
    for e, r0, r1 in _segs(P, E):
        ab_ref[r0:r1] = R.gate_up(xd[r0:r1], wd[e])
        ab_err[r0:r1] = mfma_err(xd[r0:r1], wd[e])
        s_ref[r0:r1] = R.scaled_swiglu(ab_ref[r0:r1], P["w_perm"][r0:r1])
    g, u = ab_ref[:, :f], ab_ref[:, f:]
    dg, du = ab_err[:, :f], ab_err[:, f:]
    sg = sig(g)
    s_err = np.abs(P["w_perm"])[:, None] * (
        np.abs(sg * (1 + g * (1 - sg)) * u) * dg + np.abs(g * sg) * du)
    ex = {"ab": excess(h64(ab), ab_ref, 2.0 ** -8 * np.abs(ab_ref) + ab_err),
          "s": excess(h64(s), s_ref, 2.0 ** -8 * np.abs(s_ref) + s_err)}
    ratio, sdiff = mx_rounding_check(u8(sq), u8(ss), s_ref, s_err)
    tratio, tdiff = tok_check(u8(st), u8(sts), P["offsets"], s_ref,
                              s_err + 2.0 ** -8 * np.abs(s_ref))
    print(name, ex, "S-mx", ratio, sdiff, "S-tok", tratio, tdiff)
    assert max(ex.values()) <= 1.0, ex
    assert ratio <= 1.0 and sdiff <= 1e-2
    assert tratio <= 1.0 and tdiff <= 1e-2


@gpu
@pytest.mark.parametrize("name,T,d,f,E,k,bias", SHAPES, ids=IDS)
def test_mx4_wgrad_stage(name, T, d, f, E, k, bias):
    """c[e] = A_e^T B_e with A E4M3 and B E2M1, both along the tokens."""
    dev = _dev()
    P = _plan(T, E, k, bias, seed=35)
    Tk = T * k
    a = I.make_tensor((Tk, d), seed=10, device=dev)
    b = I.make_tensor((Tk, f), seed=11, device=dev)
    a[::5] *= 30.0
    b[::3] *= 0.01
    tp = moe.moe_mxfp8_padded_rows(Tk, E)
    aq = torch.empty(d, tp, dtype=torch.uint8, device=dev)
    as_ = torch.empty(d, tp // 32, dtype=torch.uint8, device=dev)
    moe.moe_mxfp8_quantize(a, 1, P["offsets_d"], aq, as_, tp)
    bq = torch.empty(f, tp // 2, dtype=torch.uint8, device=dev)
    bs = torch.empty(f, tp // 32, dtype=torch.uint8, device=dev)
    moe.moe_mxfp4_quantize(b, 1, P["offsets_d"], bq, bs, tp)
    c = torch.full((E, d, f), 7.0, dtype=torch.bfloat16, device=dev)
    moe.moe_mx_grouped_wgrad(aq, as_, bq, bs, P["offsets_d"], Tk, c,
                             b_fp4=True)
    torch.cuda.synchronize()
    ad = X.mx_tokens(h64(a), P["offsets"])
    bd = X.mx4_tokens(h64(b), P["offsets"])
    c_ref = np.zeros((E, d, f))
    c_err = np.zeros((E, d, f))
    for e, r0, r1 in _segs(P, E):
        if r1 > r0:
            c_ref[e] = R.wgrad(ad[r0:r1], bd[r0:r1])
            c_err[e] = mfma_err(ad[r0:r1].T, bd[r0:r1].T)
    ex = excess(h64(c), c_ref, 2.0 ** -8 * np.abs(c_ref) + c_err)
    print(name, "c", ex)
    assert ex <= 1.0
    for e in np.nonzero(P["counts"] == 0)[0]:
        assert torch.count_nonzero(c[e]).item() == 0


LAYER_SHAPES = [
    ("small", 64, 128, 128, 4, 2, False, 0.0),
    ("ragged", 300, 256, 384, 5, 2, False, 0.01),
    ("skew", 600, 128, 256, 16, 4, True, 0.0),
    ("outliers", 400, 256, 256, 8, 2, False, 0.05),
]


def _run(T, d, f, E, k, bias, outliers, seed, timers=None):
    dev = _dev()
    inp = I.make_custom(T, d, f, E, k, seed=seed, device=dev,
                        router_bias=bias, outlier_frac=outliers)
    path = MoEPathMX(T, d, f, E, k, device=dev, act_fp4=True)
    path.forward(inp["x"], inp["w_gu"], inp["w2"], logits=inp["logits"],
                 timers=timers)
    path.backward(inp["dy"], inp["w_gu"], inp["w2"], timers=timers)
    torch.cuda.synchronize()
    return inp, path


@gpu
@pytest.mark.parametrize("name,T,d,f,E,k,bias,outliers", LAYER_SHAPES,
                         ids=[s[0] for s in LAYER_SHAPES])
def test_mx4_layer_parity(name, T, d, f, E, k, bias, outliers):
    inp, path = _run(T, d, f, E, k, bias, outliers, seed=len(name) + 40)
    h = {n: (h64(v) if v is not None and v.is_floating_point() else v)
         for n, v in inp.items()}
    fwd = X.moe_forward_mx(h["x"], h["logits"], h["w_gu"], h["w2"], k,
                           act4=True)
    bwd = X.moe_backward_mx(fwd, h["dy"], h["w_gu"], h["w2"])
    np.testing.assert_array_equal(path.topk_idx.cpu().numpy(), fwd["idx"])
    np.testing.assert_array_equal(path.pos.cpu().numpy(), fwd["pos"])
    # the payload is bit-exact: MXFP4 rows of x, permuted
    xc, xs = M4.quantize_rows4(h["x"])
    src = fwd["src"]
    np.testing.assert_array_equal(u8(path.xpq), M4.pack_nibbles(xc)[src])
    np.testing.assert_array_equal(u8(path.xps), xs[src])
    gpu_out = {"y": path.y, "dx": path.dx, "dw_gu": path.dw_gu,
               "dw2": path.dw2, "dp": path.dp}
    ref = {"y": fwd["y"], "dx": bwd["dx"], "dw_gu": bwd["dw_gu"],
           "dw2": bwd["dw2"], "dp": bwd["dp"]}
    bar = {n: rel_rms(h64(gpu_out[n]), ref[n]) for n in gpu_out}
    mx_max = {n: rel(h64(gpu_out[n]), ref[n]) for n in gpu_out}
    efwd = R.moe_forward(h["x"], h["logits"], h["w_gu"], h["w2"], k)
    exact_y = rel(h64(path.y), efwd["y"])
    print(name, "vs MXFP4-act oracle: relative RMS",
          {n: f"{v:.2e}" for n, v in bar.items()}, "max|err|/rms",
          {n: f"{v:.2e}" for n, v in mx_max.items()},
          f"y vs exact layer {exact_y:.2e}")
    bad = {n: v for n, v in bar.items() if not v <= TOL_MX_RMS}
    assert not bad, bad
    for e in np.nonzero(fwd["counts"] == 0)[0]:
        assert torch.count_nonzero(path.dw_gu[e]).item() == 0
        assert torch.count_nonzero(path.dw2[e]).item() == 0


@gpu
def test_mx4_stage_entries_equal_fused_entries():
    outs = []
    for timers in (None, StageTimers()):
        _, path = _run(500, 256, 256, 6, 2, False, 0.02, seed=9,
                       timers=timers)
        outs.append([t.clone() for t in (path.y, path.dx, path.dw_gu,
                                         path.dw2, path.dp)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@gpu
def test_mx4_layer_deterministic():
    outs = []
    for _ in range(2):
        _, path = _run(300, 256, 384, 5, 2, False, 0.01, seed=3)
        outs.append([t.clone() for t in (path.y, path.dx, path.dw_gu,
                                         path.dw2, path.dp)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
