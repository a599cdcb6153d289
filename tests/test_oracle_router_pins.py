"""Pins of the router backward and the balancing loss (oracle/moe_ref.py)
against torch float64 autograd of the forward definitions, central finite
differences, and closed-form special cases."""

import numpy as np
import pytest
import torch

from oracle import moe_ref as R


def _problem(seed, T=40, E=8, k=2):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E))
    idx, p = R.topk_route(L, k)
    dp = rng.standard_normal((T, k))
    return L, idx, p, dp


def _torch_weights(L, idx, renorm):
    Lt = torch.tensor(L, requires_grad=True)
    it = torch.tensor(idx.astype(np.int64))
    if renorm:
        p = torch.softmax(torch.gather(Lt, 1, it), dim=1)
    else:
        p = torch.gather(torch.softmax(Lt, dim=1), 1, it)
    return Lt, p


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("seed", [0, 1])
def test_routing_weight_backward_matches_autograd(renorm, seed):
    L, idx, p, dp = _problem(seed)
    if not renorm:
        p = R.topk_route(L, idx.shape[1], renorm=False)[1]
    Lt, pt = _torch_weights(L, idx, renorm)
    assert np.allclose(pt.detach().numpy(), p, rtol=1e-14, atol=0)
    (pt * torch.tensor(dp)).sum().backward()
    got = R.routing_weight_backward(L, idx, p, dp, renorm)
    assert np.max(np.abs(got - Lt.grad.numpy())) <= 1e-14


def test_routing_weight_backward_finite_differences():
    L, idx, p, dp = _problem(3, T=6, E=5, k=3)
    got = R.routing_weight_backward(L, idx, p, dp)
    h = 1e-6
    for t in range(L.shape[0]):
        for e in range(L.shape[1]):
            Lp, Lm = L.copy(), L.copy()
            Lp[t, e] += h
            Lm[t, e] -= h
            # selection held fixed: evaluate the weights of the same idx
            fp = np.sum(dp * _renorm_weights(Lp, idx))
            fm = np.sum(dp * _renorm_weights(Lm, idx))
            assert abs((fp - fm) / (2 * h) - got[t, e]) <= 1e-8


def _renorm_weights(L, idx):
    c = np.take_along_axis(L, idx.astype(np.int64), axis=1)
    z = np.exp(c - c.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def test_routing_weight_backward_special_cases():
    # k = 1 renormalised: p = 1 whatever the score, so no gradient at all
    L, idx, p, dp = _problem(4, k=1)
    assert np.all(R.routing_weight_backward(L, idx, p, dp) == 0)
    # equal upstream gradients: sum_j p_j = 1 is constant, gradient 0
    L, idx, p, _ = _problem(5, k=3)
    dp = np.full(p.shape, 0.7)
    assert np.max(np.abs(R.routing_weight_backward(L, idx, p, dp))) < 1e-15
    # rows sum to zero (softmax Jacobian), unchosen columns zero
    L, idx, p, dp = _problem(6, k=3)
    g = R.routing_weight_backward(L, idx, p, dp)
    assert np.max(np.abs(g.sum(axis=1))) < 1e-15
    mask = np.zeros_like(g, dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert np.all(g[~mask] == 0)


def test_aux_loss_matches_autograd_and_closed_forms():
    L, idx, p, dp = _problem(7, T=50, E=6, k=2)
    counts, _, _, _ = R.dispatch_plan(idx, 6)
    alpha = 0.01
    loss, dL = R.aux_loss(L, counts, alpha)
    Lt = torch.tensor(L, requires_grad=True)
    f = torch.tensor(counts / counts.sum())
    lt = alpha * 6 * (f * torch.softmax(Lt, dim=1).mean(dim=0)).sum()
    lt.backward()
    assert abs(lt.item() - loss) <= 1e-15
    assert np.max(np.abs(Lt.grad.numpy() - dL)) <= 1e-16
    # uniform scores and uniform load: loss alpha * E * sum (1/E)(1/E) = alpha
    Lu = np.zeros((12, 4))
    loss_u, dL_u = R.aux_loss(Lu, np.full(4, 6), 0.5)
    assert abs(loss_u - 0.5) < 1e-15 and np.all(np.abs(dL_u) < 1e-17)


def test_router_backward_is_the_linear_map_gradient():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((20, 16))
    w = rng.standard_normal((5, 16))
    dL = rng.standard_normal((20, 5))
    dw, db, dx = R.router_backward(x, w, dL)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.zeros(5, dtype=torch.float64, requires_grad=True)
    ((xt @ wt.T + bt) * torch.tensor(dL)).sum().backward()
    assert np.allclose(dw, wt.grad.numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(db, bt.grad.numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(dx, xt.grad.numpy(), rtol=1e-13, atol=1e-13)
