"""The layer step captured as a HIP graph and replayed (StepGraph): every
replay, with the program's own eager work and synchronizations between
replays and the outputs cleared before each, reproduces the eager step bit
for bit (the path is deterministic)."""

import pytest
import torch

from mixture_experts_expert_top_amd import inputs as I

gpu = pytest.mark.gpu
if torch.cuda.is_available():
    from mixture_experts_expert_top_amd.layer import (MoEPath, MoEPathMX,
                                                      StepGraph)

CASES = [
    # name, T, d, f, E, k, router bias, MX
    ("tiny", 64, 32, 64, 4, 2, False, False),
    ("ragged_bias", 300, 136, 200, 5, 2, True, False),
    ("mx_small", 200, 128, 128, 4, 2, False, True),
]


def _outputs(path):
    names = ["y", "dx", "dw_gu", "dw2", "dp", "dw_g", "aux_loss"]
    return {n: getattr(path, n) for n in names}


@gpu
@pytest.mark.parametrize("name,T,d,f,E,k,bias,mx", CASES,
                         ids=[c[0] for c in CASES])
def test_graph_replay_equals_eager(name, T, d, f, E, k, bias, mx):
    dev = torch.device("cuda:0")
    inp = I.make_custom(T, d, f, E, k, seed=11, device=dev,
                        router_bias=bias)
    path = (MoEPathMX(T, d, f, E, k, device=dev) if mx
            else MoEPath(T, d, f, E, k, device=dev))

    def step():
        path.forward(inp["x"], inp["w_gu"], inp["w2"], w_g=inp["w_g"],
                     bias=inp["bias"])
        path.backward(inp["dy"], inp["w_gu"], inp["w2"])

    step()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in _outputs(path).items()}
    g = StepGraph(step)
    other = torch.randn(512, 512, device=dev)
    for rep in range(3):
        for t in _outputs(path).values():
            t.zero_()                       # eager fill, outside the graph
        other = other @ other.t() / 512.0   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in _outputs(path).items():
            assert torch.equal(t, ref[n]), (name, rep, n)
