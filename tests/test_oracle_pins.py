"""Pins of the CPU oracle against things other than itself: hand-derived
closed forms, a pure-Python sort, scipy's softmax, a dense masked brute
force, the E=1,k=1 plain SwiGLU MLP, torch autograd in float64, central
finite differences, and structural invariants of the dispatch plan.
CPU only."""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_ref as R
from mixture_experts_expert_top_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _s(a):
    return 1.0 / (1.0 + math.exp(-a))


def _silu(a):
    return a * _s(a)


def _ev(expr):
    return eval(expr, {"math": math, "s": _s, "silu": _silu})


def _evtree(t):
    if isinstance(t, str):
        return _ev(t)
    return [_evtree(u) for u in t]


def _f64(t):
    return t.to(torch.float64).cpu().numpy()


# ---------------------------------------------------------------- closed forms

def _golden_cases():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_closed_forms(case):
    x = np.array(case["x"], dtype=np.float64)
    L = np.array(case["logits"], dtype=np.float64)
    w_gu = np.array(case["w_gu"], dtype=np.float64)
    w2 = np.array(case["w2"], dtype=np.float64)
    fwd = R.moe_forward(x, L, w_gu, w2, case["k"], case["renorm"])
    if "expect_idx" in case:
        np.testing.assert_array_equal(fwd["idx"],
                                      np.array(case["expect_idx"]))
        np.testing.assert_allclose(fwd["p"], _evtree(case["expect_p"]),
                                   rtol=1e-14, atol=0)
        np.testing.assert_allclose(fwd["y"], _evtree(case["expect_y"]),
                                   rtol=1e-14, atol=1e-300)
    if "dy" in case:
        bwd = R.moe_backward(fwd, np.array(case["dy"]), w_gu, w2)
        np.testing.assert_allclose(bwd["dp"], _evtree(case["expect_dp"]),
                                   rtol=1e-14, atol=1e-300)
        np.testing.assert_allclose(bwd["dx"], _evtree(case["expect_dx"]),
                                   rtol=1e-14, atol=1e-300)
        np.testing.assert_allclose(bwd["dw2"], _evtree(case["expect_dw2"]),
                                   rtol=1e-14, atol=1e-300)
        np.testing.assert_allclose(bwd["dw_gu"],
                                   _evtree(case["expect_dw_gu"]),
                                   rtol=1e-14, atol=1e-300)


def _router_cases():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as fh:
        return json.load(fh)["router_cases"]


@pytest.mark.parametrize("case", _router_cases(), ids=lambda c: c["name"])
def test_router_logits_closed_forms(case):
    x = np.array(case["x"], dtype=np.float64)
    w_g = np.array(case["w_g"], dtype=np.float64)
    bias = None if case["bias"] is None else np.array(case["bias"])
    got = R.router_logits(x, w_g, bias)
    want = np.array(_evtree(case["expect_logits"]), dtype=np.float64)
    assert got.shape == want.shape
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------- routing

def _python_topk(L, k):
    out = []
    for row in L.tolist():
        order = sorted(range(len(row)), key=lambda e: (-row[e], e))
        out.append(order[:k])
    return np.array(out)


@pytest.mark.parametrize("T,E,k", [(50, 4, 2), (33, 8, 2), (40, 64, 8),
                                   (7, 5, 5), (9, 3, 1), (12, 130, 7)])
def test_topk_matches_python_sort(T, E, k):
    L = _f64(I.make_custom(T, 8, 8, E, k, seed=T + E)["logits"])
    idx, _ = R.topk_route(L, k)
    np.testing.assert_array_equal(idx, _python_topk(L, k))


@pytest.mark.parametrize("E,k", [(4, 2), (8, 3), (16, 16), (6, 1)])
def test_topk_ties_go_to_lower_id(E, k):
    L = _f64(I.make_tied_logits(64, E, seed=E * 10 + k))
    idx, _ = R.topk_route(L, k)
    # python's sort compares -0.0 == 0.0, as float comparison does
    np.testing.assert_array_equal(idx, _python_topk(L, k))
    for t in range(L.shape[0]):
        assert len(set(idx[t].tolist())) == k


def test_topk_nan_ranks_below_every_number():
    """A NaN score ranks below every number, -inf included; NaNs among
    themselves go by ascending id (the reading the routing kernel follows
    for scores the pages never meet)."""
    nan, inf = float("nan"), float("inf")
    L = np.array([[nan, 1.0, nan, -inf], [inf, nan, 0.0, 0.0],
                  [nan, nan, nan, nan], [2.0, -inf, nan, 3.0]])
    idx, p = R.topk_route(L, 4)
    want = []
    for row in L.tolist():
        want.append(sorted(range(4), key=lambda e: (math.isnan(row[e]),
                                                    -row[e] if not
                                                    math.isnan(row[e]) else 0,
                                                    e)))
    np.testing.assert_array_equal(idx, np.array(want))
    np.testing.assert_array_equal(idx[0], [1, 3, 0, 2])
    idx2, p2 = R.topk_route(L[3:], 2)
    np.testing.assert_array_equal(idx2, [[3, 0]])
    assert np.all(np.isfinite(p2))


@pytest.mark.parametrize("renorm", [True, False])
def test_weights_against_scipy_softmax(renorm):
    L = _f64(I.make_custom(100, 8, 8, 8, 3, seed=5)["logits"])
    idx, p = R.topk_route(L, 3, renorm)
    if renorm:
        chosen = np.take_along_axis(L, idx.astype(np.int64), axis=1)
        ref = scipy.special.softmax(chosen, axis=1)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    else:
        full = scipy.special.softmax(L, axis=1)
        ref = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(p, ref, rtol=1e-13, atol=0)
    # weights follow the descending score order of the chosen experts
    assert np.all(np.diff(p, axis=1) <= 0)


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,E,k,bias", [(64, 4, 2, False), (300, 64, 8, True),
                                        (17, 9, 3, False), (1, 4, 4, False)])
def test_dispatch_invariants(T, E, k, bias):
    inp = I.make_custom(T, 8, 8, E, k, seed=T, router_bias=bias)
    idx, _ = R.topk_route(_f64(inp["logits"]), k)
    counts, offsets, pos, src = R.dispatch_plan(idx, E)
    assert counts.sum() == T * k and offsets[E] == T * k
    assert offsets[0] == 0 and np.all(np.diff(offsets) == counts)
    # pos is a bijection onto [0, T*k) and src inverts it
    assert sorted(pos.reshape(-1).tolist()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            r = pos[t, j]
            assert src[r] == t
            e = idx[t, j]
            assert offsets[e] <= r < offsets[e + 1]
    # token-ascending inside each expert segment
    for e in range(E):
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
    # counts equal a plain histogram
    np.testing.assert_array_equal(counts,
                                  np.bincount(idx.reshape(-1), minlength=E))


def test_skewed_bias_leaves_experts_empty():
    inp = I.make_custom(512, 8, 8, 64, 8, seed=1, router_bias=True)
    idx, _ = R.topk_route(_f64(inp["logits"]), 8)
    counts, _, _, _ = R.dispatch_plan(idx, 64)
    assert (counts == 0).any()
    assert counts.max() <= 512          # an expert appears once per token


# ---------------------------------------------------------------- forward

def _dense_bruteforce(x, L, w_gu, w2, k, renorm=True):
    """Every expert on every token, then masked by the top-k indicator and
    weighted by the routing weight (no grouping, no permutation)."""
    T = x.shape[0]
    E, two_f, _ = w_gu.shape
    f = two_f // 2
    idx, p = R.topk_route(L, k, renorm)
    weight = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            weight[t, idx[t, j]] = p[t, j]
    y = np.zeros_like(x)
    for e in range(E):
        g = x @ w_gu[e, :f].T
        u = x @ w_gu[e, f:].T
        h = g / (1.0 + np.exp(-g)) * u
        y += weight[:, e:e + 1] * (h @ w2[e].T)
    return y


def _tiny(T, d, f, E, k, seed, bias=False):
    inp = I.make_custom(T, d, f, E, k, seed=seed, router_bias=bias)
    return {n: (_f64(v) if v is not None and v.is_floating_point() else v)
            for n, v in inp.items()}


@pytest.mark.parametrize("T,d,f,E,k,bias", [
    (64, 32, 64, 4, 2, False),       # the tiny workload's shape
    (40, 16, 24, 8, 3, False),
    (48, 8, 8, 16, 4, True),          # skew: some experts empty
    (5, 8, 16, 3, 3, False),          # k == E
])
def test_forward_matches_dense_bruteforce(T, d, f, E, k, bias):
    a = _tiny(T, d, f, E, k, seed=T + d, bias=bias)
    a["w_gu"] *= 25.0                 # make the activations O(1)
    fwd = R.moe_forward(a["x"], a["logits"], a["w_gu"], a["w2"], k)
    ref = _dense_bruteforce(a["x"], a["logits"], a["w_gu"], a["w2"], k)
    scale = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(fwd["y"] - ref)) <= 1e-12 * scale


def test_e1_k1_is_plain_swiglu_mlp():
    a = _tiny(32, 16, 24, 1, 1, seed=3)
    a["w_gu"] *= 25.0
    fwd = R.moe_forward(a["x"], a["logits"], a["w_gu"], a["w2"], 1)
    np.testing.assert_array_equal(fwd["p"], 1.0)
    x = torch.from_numpy(a["x"])
    w1 = torch.from_numpy(a["w_gu"][0, :24])
    w3 = torch.from_numpy(a["w_gu"][0, 24:])
    w2 = torch.from_numpy(a["w2"][0])
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(x, w1))
        * torch.nn.functional.linear(x, w3), w2).numpy()
    np.testing.assert_allclose(fwd["y"], ref, rtol=1e-12, atol=1e-15)


def test_permute_then_unpermute_is_identity():
    a = _tiny(50, 12, 8, 6, 1, seed=9)
    idx, _ = R.topk_route(a["logits"], 1)
    _, _, pos, src = R.dispatch_plan(idx, 6)
    xp = R.permute_rows(a["x"], src)
    back = R.combine(xp, pos, idx)            # k=1: exact identity
    np.testing.assert_array_equal(back, a["x"])
    # weighted un-permute with renormalised weights reproduces x (k=3)
    idx3, p3 = R.topk_route(a["logits"], 3)
    _, _, pos3, src3 = R.dispatch_plan(idx3, 6)
    xp3 = R.permute_rows(a["x"], src3)
    w = R.permuted_weights(p3, pos3)
    back3 = R.combine(xp3 * w[:, None], pos3, idx3)
    np.testing.assert_allclose(back3, a["x"], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- backward

def _torch_dense_layer(x, idx, p, w_gu, w2):
    """Dense float64 torch formulation (every expert on every token, masked),
    used only through autograd."""
    T = x.shape[0]
    E, two_f, _ = w_gu.shape
    f = two_f // 2
    y = torch.zeros_like(x)
    for e in range(E):
        g = x @ w_gu[e, :f].T
        u = x @ w_gu[e, f:].T
        h = torch.nn.functional.silu(g) * u
        mask = torch.zeros(T, dtype=torch.float64)
        for t in range(T):
            for j in range(idx.shape[1]):
                if idx[t, j] == e:
                    mask = mask + torch.nn.functional.one_hot(
                        torch.tensor(t), T).double() * p[t, j]
        y = y + mask[:, None] * (h @ w2[e].T)
    return y


@pytest.mark.parametrize("T,d,f,E,k,bias", [(12, 6, 5, 4, 2, False),
                                            (16, 4, 6, 8, 3, True)])
def test_backward_matches_torch_autograd(T, d, f, E, k, bias):
    a = _tiny(T, d, f, E, k, seed=T * k, bias=bias)
    a["w_gu"] *= 25.0
    a["w2"] *= 10.0
    idx, p = R.topk_route(a["logits"], k)
    fwd = R.experts_forward(a["x"], idx, p, a["w_gu"], a["w2"])
    bwd = R.moe_backward(fwd, a["dy"], a["w_gu"], a["w2"])
    xt = torch.tensor(a["x"], requires_grad=True)
    pt = torch.tensor(p, requires_grad=True)
    wgu = torch.tensor(a["w_gu"], requires_grad=True)
    w2 = torch.tensor(a["w2"], requires_grad=True)
    y = _torch_dense_layer(xt, idx, pt, wgu, w2)
    np.testing.assert_allclose(fwd["y"], y.detach().numpy(), rtol=1e-12,
                               atol=1e-14)
    y.backward(torch.tensor(a["dy"]))
    for name, ref in [("dx", xt.grad), ("dp", pt.grad), ("dw_gu", wgu.grad),
                      ("dw2", w2.grad)]:
        np.testing.assert_allclose(bwd[name], ref.numpy(), rtol=1e-11,
                                   atol=1e-13, err_msg=name)


def test_backward_finite_differences():
    T, d, f, E, k = 5, 4, 3, 3, 2
    a = _tiny(T, d, f, E, k, seed=77)
    a["w_gu"] *= 25.0
    a["w2"] *= 10.0
    idx, p = R.topk_route(a["logits"], k)
    dy = a["dy"]

    def loss(x, p_, w_gu, w2):
        return float(np.sum(R.experts_forward(x, idx, p_, w_gu, w2)["y"]
                            * dy))

    fwd = R.experts_forward(a["x"], idx, p, a["w_gu"], a["w2"])
    bwd = R.moe_backward(fwd, dy, a["w_gu"], a["w2"])
    h = 1e-6
    args = {"x": a["x"], "p": p, "w_gu": a["w_gu"], "w2": a["w2"]}
    grads = {"x": bwd["dx"], "p": bwd["dp"], "w_gu": bwd["dw_gu"],
             "w2": bwd["dw2"]}
    for name, arr in args.items():
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            plus = {n: v.copy() for n, v in args.items()}
            minus = {n: v.copy() for n, v in args.items()}
            plus[name][i] += h
            minus[name][i] -= h
            fd[i] = (loss(plus["x"], plus["p"], plus["w_gu"], plus["w2"])
                     - loss(minus["x"], minus["p"], minus["w_gu"],
                            minus["w2"])) / (2 * h)
        scale = max(np.max(np.abs(grads[name])), 1e-30)
        assert np.max(np.abs(fd - grads[name])) <= 1e-6 * scale, name


def test_empty_expert_gets_exact_zero_weight_grads():
    T, d, f, E, k = 20, 8, 8, 6, 1
    a = _tiny(T, d, f, E, k, seed=2)
    a["logits"][:, 5] = -1e9                  # nobody picks expert 5
    fwd = R.moe_forward(a["x"], a["logits"], a["w_gu"], a["w2"], k)
    assert fwd["counts"][5] == 0
    bwd = R.moe_backward(fwd, a["dy"], a["w_gu"], a["w2"])
    assert np.all(bwd["dw_gu"][5] == 0.0) and np.all(bwd["dw2"][5] == 0.0)


# ---------------------------------------------------------------- sampled

def test_sampled_helpers_match_full_layer():
    T, d, f, E, k = 24, 16, 12, 5, 2
    a = _tiny(T, d, f, E, k, seed=11)
    a["w_gu"] *= 25.0
    fwd = R.moe_forward(a["x"], a["logits"], a["w_gu"], a["w2"], k)
    bwd = R.moe_backward(fwd, a["dy"], a["w_gu"], a["w2"])
    for t in (0, 7, 23):
        y_t = R.token_forward(a["x"][t], fwd["idx"][t], fwd["p"][t],
                              a["w_gu"], a["w2"])
        np.testing.assert_allclose(y_t, fwd["y"][t], rtol=1e-13, atol=1e-15)
        for j in range(k):
            e = fwd["idx"][t, j]
            r = fwd["pos"][t, j]
            dab, dxp, dp_r, ab, s = R.row_backward(
                a["x"][t], a["dy"][t], fwd["p"][t, j], a["w_gu"][e],
                a["w2"][e])
            np.testing.assert_allclose(dab, bwd["dab"][r], rtol=1e-13,
                                       atol=1e-15)
            np.testing.assert_allclose(dxp, bwd["dxp"][r], rtol=1e-13,
                                       atol=1e-15)
            assert abs(dp_r - bwd["dp"][t, j]) <= 1e-13 * max(1, abs(dp_r))
            np.testing.assert_allclose(ab, fwd["ab"][r], rtol=1e-13)
            np.testing.assert_allclose(s, fwd["s"][r], rtol=1e-13)


def test_sampled_weight_grads_match_full_layer():
    T, d, f, E, k = 30, 16, 12, 4, 2
    a = _tiny(T, d, f, E, k, seed=21)
    a["w_gu"] *= 25.0
    fwd = R.moe_forward(a["x"], a["logits"], a["w_gu"], a["w2"], k)
    bwd = R.moe_backward(fwd, a["dy"], a["w_gu"], a["w2"])
    for e in range(E):
        r0, r1 = fwd["offsets"][e], fwd["offsets"][e + 1]
        xp_e = fwd["xp"][r0:r1]
        do_e = bwd["do"][r0:r1]
        w_e = fwd["w_perm"][r0:r1]
        for j in (0, 5, f - 1):
            np.testing.assert_allclose(
                R.dw2_column(xp_e, do_e, w_e, a["w_gu"][e], j),
                bwd["dw2"][e][:, j], rtol=1e-12, atol=1e-14)
        for i in (0, 3, f, 2 * f - 1):
            np.testing.assert_allclose(
                R.dw_gu_row(xp_e, do_e, w_e, a["w_gu"][e], a["w2"][e], i),
                bwd["dw_gu"][e][i], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- bf16 mode

def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(4)
    v = np.concatenate([
        rng.standard_normal(200000) * 2.0 ** rng.integers(-60, 60, 200000),
        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 2.0 ** -126, 2.0 ** -130,
         -3.0e38, 1.0e-40]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    got = R.bf16_round(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(ref))


def test_bf16_round_is_nearest_for_float64_values():
    """Brute force: the nearest of the bfloat16 neighbours of v (found by
    stepping the bit pattern), ties to the even pattern."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal(20000) * 2.0 ** rng.integers(-20, 20, 20000)
    v[:100] = (np.arange(100) + 0.5) * 2.0 ** -7 + 1.0     # exact ties
    got = R.bf16_round(v)
    base = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    bits = base.view(torch.int16).numpy().astype(np.int32)
    for i in range(v.size):
        cands = []
        for db in (-1, 0, 1):
            b = np.array([bits[i] + db], dtype=np.int32).astype(np.int16)
            c = torch.from_numpy(b).view(torch.bfloat16).double().item()
            cands.append((abs(c - v[i]), (bits[i] + db) & 1, c))
        best = min(cands)[0]
        tied = [c for c in cands if c[0] == best]
        want = min(tied, key=lambda c: c[1])[2]
        assert got[i] == want, (v[i], got[i], want)


def test_bf16_activation_mode_stores_bf16_values():
    T, d, f, E, k = 40, 16, 24, 4, 2
    a = _tiny(T, d, f, E, k, seed=31)
    a["w_gu"] *= 25.0
    fwd = R.moe_forward(a["x"], a["logits"], a["w_gu"], a["w2"], k,
                        bf16_act=True)
    bwd = R.moe_backward(fwd, a["dy"], a["w_gu"], a["w2"], bf16_act=True)
    for name, arr in (("ab", fwd["ab"]), ("s", fwd["s"]),
                      ("dab", bwd["dab"])):
        np.testing.assert_array_equal(R.bf16_round(arr), arr, err_msg=name)
    exact = R.moe_forward(a["x"], a["logits"], a["w_gu"], a["w2"], k)
    # S is the rounded exact S; AB is the rounded exact AB
    np.testing.assert_array_equal(fwd["s"], R.bf16_round(exact["s"]))
    np.testing.assert_array_equal(fwd["ab"], R.bf16_round(exact["ab"]))
    # the output moves by no more than the storage roundings allow
    assert rel_err(fwd["y"], exact["y"]) < 2e-2


def rel_err(got, ref):
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))


def test_bf16_activation_closed_form():
    """k1_two_tokens of the closed forms with S stored as bfloat16:
    silu(1) = 0.731058... rounds to 187/256 and 1.0757... (= silu(-1)*(-4))
    to 138/128, so y = (187/256, 3*138/128)."""
    case = [c for c in _golden_cases() if c["name"] == "k1_two_tokens"][0]
    fwd = R.moe_forward(np.array(case["x"]), np.array(case["logits"]),
                        np.array(case["w_gu"]), np.array(case["w2"]), 1,
                        bf16_act=True)
    np.testing.assert_array_equal(fwd["y"], [[187 / 256], [3 * 138 / 128]])
