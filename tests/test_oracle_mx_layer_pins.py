"""Pins of the MXFP8 layer oracle (oracle/moe_mx.py) to things other than
itself.

1. An independent formulation: per expert, the token list comes from the
   routing mask (no dispatch plan, offsets or positions); the MX codec is
   torch's float8_e4m3fn cast (round to nearest even) after clamping to
   +-448, with the block exponent floor(log2 amax) - 8 taken from
   numpy.log2; the SwiGLU backward and the routing-weight gradient come
   from torch autograd in float64.
2. Axis checks: inputs built to be MX-representable along the documented
   axis only come through the oracle's quantizers unchanged, and would not
   along the other axis.
3. With every quantizer replaced by the identity, the MX layer is the plain
   layer of oracle/moe_ref.py.
4. The MX layer differs from the exact layer by the few to some tens of
   percent (relative RMS) that 3-bit mantissas give, and not by zero.
"""

import numpy as np
import pytest
import torch

from oracle import moe_mx as X
from oracle import moe_ref as R

T, D, F, E, K = 48, 64, 96, 4, 2


def _problem(seed, empty_expert=False):
    rng = np.random.default_rng(seed)
    bf = R.bf16_round
    x = bf(rng.standard_normal((T, D)))
    x[5] *= 100.0                                       # an outlier row
    logits = rng.standard_normal((T, E))
    if empty_expert:
        logits[:, 2] -= 100.0                           # expert 2 gets none
    w_gu = bf(rng.standard_normal((E, 2 * F, D)) * 0.2)
    w2 = bf(rng.standard_normal((E, D, F)) * 0.2)
    dy = bf(rng.standard_normal((T, D)))
    return x, logits, w_gu, w2, dy


# ------------------------------------------------------------ 1. independent

def _tq_last(a):
    """Quantize-dequantize along the last axis with torch's E4M3 cast."""
    a = np.asarray(a, dtype=np.float64)
    sh = a.shape
    b = a.reshape(-1, 32)
    amax = np.abs(b).max(axis=1)
    e = np.full(amax.shape, -127.0)
    nz = amax > 0
    e[nz] = np.clip(np.floor(np.log2(amax[nz])) - 8.0, -127.0, 127.0)
    scale = np.exp2(e)[:, None]
    v = np.clip(b / scale, -448.0, 448.0)
    q = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return (q * scale).reshape(sh)


def _tq_rows_of_list(a):
    """Quantize-dequantize along rows in blocks of 32 consecutive rows (the
    last block may be short: zero rows pad it and are dropped again)."""
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    for b0 in range(0, a.shape[0], 32):
        blk = a[b0:b0 + 32]
        pad = np.zeros((32, a.shape[1]))
        pad[:blk.shape[0]] = blk
        out[b0:b0 + 32] = _tq_last(pad.T).T[:blk.shape[0]]
    return out


def _independent(x, logits, w_gu, w2, dy):
    L = torch.from_numpy(logits)
    top = torch.topk(L, K, dim=1)            # float64 logits: no ties here
    idx = top.indices.numpy()
    p = torch.softmax(top.values, dim=1).numpy()
    xq = _tq_last(x)
    dyq = _tq_last(dy)
    y = np.zeros((T, D))
    dx = np.zeros((T, D))
    dp = np.zeros((T, K))
    dw_gu = np.zeros_like(w_gu)
    dw2 = np.zeros_like(w2)
    for e in range(E):
        tok, slot = np.nonzero(idx == e)     # ascending token, one slot each
        if tok.size == 0:
            continue
        pe = torch.tensor(p[tok, slot], requires_grad=True)
        ab = xq[tok] @ _tq_last(w_gu[e]).T
        ag = torch.tensor(R.bf16_round(ab[:, :F]), requires_grad=True)
        au = torch.tensor(R.bf16_round(ab[:, F:]), requires_grad=True)
        s = (torch.from_numpy(p[tok, slot])[:, None] *
             torch.nn.functional.silu(torch.from_numpy(ab[:, :F])) *
             torch.from_numpy(ab[:, F:])).numpy()
        y[tok] += _tq_last(s) @ _tq_last(w2[e]).T
        # backward
        ds = dyq[tok] @ _tq_last(w2[e].T).T          # W2 along d
        s_saved = pe[:, None] * torch.nn.functional.silu(ag) * au
        s_saved.backward(torch.from_numpy(ds))
        dab = np.concatenate([ag.grad.numpy(), au.grad.numpy()], axis=1)
        dp[tok, slot] = pe.grad.numpy()
        dx[tok] += _tq_last(dab) @ _tq_last(w_gu[e].T).T   # W_gu along 2f
        dw2[e] = _tq_rows_of_list(dy[tok]).T @ \
            _tq_rows_of_list(R.bf16_round(s))
        dw_gu[e] = _tq_rows_of_list(R.bf16_round(dab)).T @ \
            _tq_rows_of_list(x[tok])
    return dict(y=y, dx=dx, dp=dp, dw_gu=dw_gu, dw2=dw2)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b * b)), 1e-300)


@pytest.mark.parametrize("seed,empty", [(0, False), (1, True), (2, False)])
def test_mx_layer_matches_independent_formulation(seed, empty):
    x, logits, w_gu, w2, dy = _problem(seed, empty)
    fwd = X.moe_forward_mx(x, logits, w_gu, w2, K)
    bwd = X.moe_backward_mx(fwd, dy, w_gu, w2)
    ref = _independent(x, logits, w_gu, w2, dy)
    assert _rel(fwd["y"], ref["y"]) < 1e-12
    for name in ("dx", "dp", "dw_gu", "dw2"):
        assert _rel(bwd[name], ref[name]) < 1e-12, name
    if empty:
        assert fwd["counts"][2] == 0
        assert np.all(bwd["dw_gu"][2] == 0) and np.all(bwd["dw2"][2] == 0)


# ------------------------------------------------------------ 2. axes

def _row_exact(shape, rng):
    """Rows of c_row * m / 16 with |m| <= 14 and one m = 14 per row: the
    block exponent puts every element at 32 m (at most 448, four
    significant bits), exact in E4M3, as long as a block stays inside one
    row.  Row magnitudes differ by up to 2^40, so blocks across rows lose
    the small rows."""
    m = rng.integers(-14, 15, shape).astype(np.float64)
    m[..., 0] = 14.0                             # every row has its max
    c = np.exp2(rng.integers(-20, 21, shape[:-1] + (1,)).astype(np.float64))
    return c * m / 16.0


def test_mx_forward_quantizes_x_and_weights_along_their_rows():
    rng = np.random.default_rng(3)
    x = _row_exact((T, D), rng)
    w_gu = _row_exact((E, 2 * F, D), rng)
    w2 = _row_exact((E, D, F), rng)
    logits = rng.standard_normal((T, E))
    fwd = X.moe_forward_mx(x, logits, w_gu, w2, K)
    assert np.array_equal(fwd["xq"], x)
    assert np.array_equal(fwd["w_gu_q"], w_gu)
    assert np.array_equal(fwd["w2_q"], w2)
    # the other axis would have changed them
    assert not np.array_equal(X.mx_tokens(x, np.array([0, T])), x)
    assert not np.array_equal(X.mx_cols(w2), w2)


def test_mx_backward_quantizes_weights_along_their_columns():
    rng = np.random.default_rng(4)
    w_gu = np.stack([_row_exact((D, 2 * F), rng).T for _ in range(E)])
    w2 = np.stack([_row_exact((F, D), rng).T for _ in range(E)])
    x = R.bf16_round(rng.standard_normal((T, D)))
    dy = _row_exact((T, D), rng)
    logits = rng.standard_normal((T, E))
    fwd = X.moe_forward_mx(x, logits, w_gu, w2, K)
    bwd = X.moe_backward_mx(fwd, dy, w_gu, w2)
    assert np.array_equal(bwd["w2_c"], w2)
    assert np.array_equal(bwd["w_gu_c"], w_gu)
    assert np.array_equal(bwd["do_q"], dy[fwd["src"]])
    assert not np.array_equal(X.mx_rows(w2), w2)


def test_token_blocks_restart_at_segments():
    """Each expert's rows are scaled per 32-row block counted from its own
    first row: a segment of one huge-magnitude row next to a segment of
    small rows leaves the small rows exact."""
    rows = np.concatenate([np.full((1, 32), 2.0 ** 30),
                           np.full((33, 32), 0.375)])
    offs = np.array([0, 1, 34])
    q = X.mx_tokens(rows, offs)
    assert np.array_equal(q, rows)
    q_one = X.mx_tokens(rows, np.array([0, 34]))       # no restart
    assert not np.array_equal(q_one, rows)


# ------------------------------------------------------------ 3. reduction

def test_identity_quantizers_reduce_to_the_plain_layer(monkeypatch):
    x, logits, w_gu, w2, dy = _problem(5)
    ident = lambda a, *rest: np.asarray(a, dtype=np.float64)  # noqa: E731
    for name in ("mx_rows", "mx_cols", "mx_tokens"):
        monkeypatch.setattr(X, name, ident)
    fwd = X.moe_forward_mx(x, logits, w_gu, w2, K)
    plain = R.moe_forward(x, logits, w_gu, w2, K)
    assert _rel(fwd["y"], plain["y"]) < 1e-12
    kept = R.moe_forward(x, logits, w_gu, w2, K, bf16_act=True)
    assert np.array_equal(fwd["ab"], kept["ab"])
    assert np.array_equal(fwd["s"], kept["s"])
    bwd = X.moe_backward_mx(fwd, dy, w_gu, w2)
    ref = R.moe_backward(kept, dy, w_gu, w2, bf16_act=True)
    for name in ("dw2", "dw_gu", "dp", "dab"):
        assert _rel(bwd[name], ref[name]) < 1e-12, name


# ------------------------------------------------------------ 4. size of error

def test_mx_layer_error_is_small_but_nonzero():
    x, logits, w_gu, w2, dy = _problem(6)
    fwd = X.moe_forward_mx(x, logits, w_gu, w2, K)
    bwd = X.moe_backward_mx(fwd, dy, w_gu, w2)
    plain = R.moe_forward(x, logits, w_gu, w2, K)
    pb = R.moe_backward(plain, dy, w_gu, w2)
    rr = lambda a, b: np.sqrt(np.mean((a - b) ** 2) / np.mean(b * b))  # noqa
    for got, ref in ((fwd["y"], plain["y"]), (bwd["dx"], pb["dx"]),
                     (bwd["dw_gu"], pb["dw_gu"]), (bwd["dw2"], pb["dw2"]),
                     (bwd["dp"], pb["dp"])):
        # E4M3 keeps 3 mantissa bits: each quantized operand carries about
        # 2^-4/sqrt(3) relative RMS error, and the backward chains up to
        # three quantized GEMMs
        assert 1e-3 < rr(got, ref) < 0.3


# ------------------------------------------------------------ 5. sampled

def test_sampled_helpers_match_the_full_layer():
    """The single-output helpers used at full size give the full layer's
    values (same definition, evaluated for one token, row or column)."""
    x, logits, w_gu, w2, dy = _problem(7)
    fwd = X.moe_forward_mx(x, logits, w_gu, w2, K)
    bwd = X.moe_backward_mx(fwd, dy, w_gu, w2)
    W = {e: X.expert_weights_mx(w_gu[e], w2[e], backward=True)
         for e in range(E)}
    idx, p, pos = fwd["idx"], fwd["p"], fwd["pos"]
    for t in (0, 5, 17, T - 1):
        y_t = X.token_forward_mx(x[t], idx[t], p[t], W)
        assert np.max(np.abs(y_t - fwd["y"][t])) <= 1e-12 * np.max(
            np.abs(fwd["y"]))
        for j in range(K):
            dxp, dp = X.row_backward_mx(x[t], dy[t], p[t, j], W[idx[t, j]])
            r = pos[t, j]
            assert np.allclose(dxp, bwd["dxp"][r], rtol=1e-12, atol=1e-12)
            assert abs(dp - bwd["dp"][t, j]) <= 1e-12 * max(
                1.0, abs(bwd["dp"][t, j]))
    off, src = fwd["offsets"], fwd["src"]
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        rows = src[r0:r1]
        we = fwd["w_perm"][r0:r1]
        for j in (0, F - 1):
            col = X.dw2_column_mx(x[rows], dy[rows], we, w_gu[e], j)
            assert np.allclose(col, bwd["dw2"][e][:, j], rtol=1e-12,
                               atol=1e-12 * np.max(np.abs(bwd["dw2"])))
        for i in (1, F + 2):
            row = X.dw_gu_row_mx(x[rows], dy[rows], we, w_gu[e], w2[e], i)
            assert np.allclose(row, bwd["dw_gu"][e][i], rtol=1e-12,
                               atol=1e-12 * np.max(np.abs(bwd["dw_gu"])))
