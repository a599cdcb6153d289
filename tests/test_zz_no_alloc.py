"""The allocation-free permutation (moe_permute_noalloc, per-GPU fixed
scratch) against moe_permute with a caller workspace, through the C-ABI:
bit-identical plans and permuted rows on two calls in a row, the second
one smaller (it must not see the first call's scratch contents), in bf16
and in MXFP8."""

import numpy as np
import pytest
import torch

from mixture_experts_expert_top_amd import inputs as I

gpu = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_expert_top_amd import moe


def _case(T, E, k, d, seed, prec):
    dev = torch.device("cuda:0")
    L = I.make_custom(T, 8, 8, E, k, seed=seed, device=dev,
                      router_bias=True)["logits"]
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    moe.moe_route(L, k, True, idx, w)
    x_bf = I.make_tensor((T, d), seed=seed + 1, device=dev)
    if prec == moe.MOE_BF16:
        x, xs = x_bf, None
    else:
        x = torch.empty(T, d, dtype=torch.uint8, device=dev)
        xs = torch.empty(T, d // 32, dtype=torch.uint8, device=dev)
        moe.moe_mxfp8_quantize(x_bf, 0, None, x, xs)
    return idx, w, x, xs


def _outputs(T, E, k, d, x, prec, dev):
    z = lambda *s, dt: torch.full(s, -7, dtype=dt, device=dev)  # noqa: E731
    o = {"counts": z(E, dt=torch.int32), "offsets": z(E + 1, dt=torch.int32),
         "pos": z(T, k, dt=torch.int32), "src": z(T * k, dt=torch.int32),
         "w_perm": z(T * k, dt=torch.float32),
         "x_perm": torch.zeros(T * k, *x.shape[1:], dtype=x.dtype,
                               device=dev)}
    o["x_perm_scales"] = (torch.zeros(T * k, d // 32, dtype=torch.uint8,
                                      device=dev)
                          if prec != moe.MOE_BF16 else None)
    return o


@gpu
@pytest.mark.parametrize("prec", [0, 1], ids=["bf16", "mxfp8"])
def test_noalloc_permute_matches_workspace_permute(prec):
    dev = torch.device("cuda:0")
    # large first, then smaller: the second call runs on scratch that still
    # holds the first call's counts
    for T, E, k, d in ((16384, 64, 8, 256), (300, 6, 2, 64)):
        idx, w, x, xs = _case(T, E, k, d, seed=T + E, prec=prec)
        ref = _outputs(T, E, k, d, x, prec, dev)
        got = _outputs(T, E, k, d, x, prec, dev)
        ws = torch.empty(max(moe.moe_workspace_bytes(0, prec, T, E, k, d, 64),
                             16), dtype=torch.uint8, device=dev)
        moe.moe_permute(prec, idx, w, E, x, xs, ref["counts"],
                        ref["offsets"], ref["pos"], ref["src"],
                        ref["w_perm"], ref["x_perm"], ref["x_perm_scales"],
                        ws)
        moe.moe_permute_noalloc(prec, idx, w, E, x, xs, got["counts"],
                                got["offsets"], got["pos"], got["src"],
                                got["w_perm"], got["x_perm"],
                                got["x_perm_scales"])
        torch.cuda.synchronize()
        for n in ref:
            if ref[n] is None:
                continue
            a = ref[n].view(torch.uint8).cpu().numpy()
            b = got[n].view(torch.uint8).cpu().numpy()
            np.testing.assert_array_equal(b, a, err_msg=f"{n} T={T} E={E}")
        assert int(got["offsets"][-1]) == T * k
