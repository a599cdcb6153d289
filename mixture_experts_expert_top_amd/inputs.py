"""Seeded synthetic inputs shared by the GPU path's tests, the oracle's tests
and the benchmark.

This module draws random numbers and nothing else: it holds none of the
layer's arithmetic.  Every tensor is drawn in float32 from one seeded torch
generator on the requested device, in a fixed order, scaled, then rounded to
the dtype the library consumes (bfloat16 for activations and weights,
float32 for router scores and the router bias).

Workloads (sizes of the pages' Mixtral-8x7B layer and a fine-grained,
skewed variant; all values synthetic, no dataset or trained weight):

  tiny      T=64    d=32   f=64    E=4  k=2
  mixtral   T=8192  d=4096 f=14336 E=8  k=2           (forward / fwd+bwd)
  mixtral_long T=32768, otherwise the same (fwd+bwd)
  finegrain T=16384 d=2048 f=1408  E=64 k=8  router bias -2*ln(rank)
  mxfp8     T=16384 d=4096 f=14336 E=8  k=2  1% of token rows scaled x100

Distributions: x ~ N(0,1); router weight ~ N(0, 1/d); expert weights
~ N(0, 0.02^2); upstream gradient ~ N(0,1).  Router scores for the routing
parity chain are drawn directly as N(0,1) per (token, expert) -- the law of
x . W_g under the distributions above -- times 100 on the outlier rows, plus
the per-expert bias where the workload has one.
"""

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    renorm: bool = True
    router_bias: bool = False
    outlier_frac: float = 0.0
    outlier_scale: float = 100.0
    prec: str = "bf16"          # "bf16", "mxfp8" or "mxfp4" (MXFP8 GEMMs
                                # with MXFP4 activations)
    backward: bool = True

    @property
    def Tk(self):
        return self.T * self.k


WORKLOADS = {
    "tiny": Workload("tiny", 64, 32, 64, 4, 2, backward=True),
    "tiny_fwd": Workload("tiny_fwd", 64, 32, 64, 4, 2, backward=False),
    "mixtral_fwd": Workload("mixtral_fwd", 8192, 4096, 14336, 8, 2,
                            backward=False),
    "mixtral": Workload("mixtral", 8192, 4096, 14336, 8, 2),
    # long-sequence variant (4 x 8192 tokens): past the size at which any
    # single activation tensor of the layer exceeds 2 GiB (AB and dAB are
    # 3.8 GB)
    "mixtral_long": Workload("mixtral_long", 32768, 4096, 14336, 8, 2),
    "finegrain": Workload("finegrain", 16384, 2048, 1408, 64, 8,
                          router_bias=True),
    "mxfp8": Workload("mxfp8", 16384, 4096, 14336, 8, 2, outlier_frac=0.01,
                      prec="mxfp8"),
    "mxfp4": Workload("mxfp4", 16384, 4096, 14336, 8, 2, outlier_frac=0.01,
                      prec="mxfp4"),
}


def router_bias_values(E):
    """Per-expert bias 2*log(1/rank), rank = expert id + 1 (natural log)."""
    return torch.tensor([-2.0 * math.log(e + 1) for e in range(E)],
                        dtype=torch.float64).to(torch.float32)


def make_inputs(wl, seed=0, device="cpu", with_weights=True, with_dy=True):
    """Draw every input of workload ``wl`` (a Workload) on ``device``.

    Returns a dict: x [T,d] bf16, w_g [E,d] bf16, bias [E] f32 or None,
    w_gu [E,2f,d] bf16 (gate rows first), w2 [E,d,f] bf16, dy [T,d] bf16,
    logits [T,E] f32, outlier_rows (int64 indices).
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    T, d, f, E = wl.T, wl.d, wl.f, wl.E

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=device,
                           dtype=torch.float32)

    out = {}
    x = randn(T, d)
    n_out = int(round(wl.outlier_frac * T))
    if n_out:
        rows = torch.randperm(T, generator=g, device=device)[:n_out]
        rows = torch.sort(rows).values
        x[rows] *= wl.outlier_scale
    else:
        rows = torch.zeros(0, dtype=torch.int64, device=device)
    out["x"] = x.to(torch.bfloat16)
    out["outlier_rows"] = rows
    del x
    out["w_g"] = (randn(E, d) / math.sqrt(d)).to(torch.bfloat16)
    out["bias"] = (router_bias_values(E).to(device) if wl.router_bias
                   else None)
    if with_weights:
        out["w_gu"] = (randn(E, 2 * f, d) * 0.02).to(torch.bfloat16)
        out["w2"] = (randn(E, d, f) * 0.02).to(torch.bfloat16)
    if with_dy:
        out["dy"] = randn(T, d).to(torch.bfloat16)
    logits = randn(T, E)
    if n_out:
        logits[rows] *= wl.outlier_scale
    if out["bias"] is not None:
        logits += out["bias"][None, :]
    out["logits"] = logits
    return out


def make_custom(T, d, f, E, k, seed=0, device="cpu", router_bias=False,
                outlier_frac=0.0):
    """Inputs for an arbitrary (T, d, f, E, k), same distributions."""
    wl = Workload("custom", T, d, f, E, k, router_bias=router_bias,
                  outlier_frac=outlier_frac)
    return make_inputs(wl, seed=seed, device=device)


def make_tied_logits(T, E, seed=0, levels=3, device="cpu"):
    """Router scores drawn from a few discrete levels so that exact ties
    (including +0.0 / -0.0) are common: exercises the lower-id tie rule."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    lv = torch.randint(0, levels, (T, E), generator=g, device=device)
    vals = lv.to(torch.float32) - (levels // 2)
    sign = torch.randint(0, 2, (T, E), generator=g, device=device)
    # turn some zeros into negative zeros
    vals = torch.where((vals == 0) & (sign == 1),
                       torch.full_like(vals, -0.0), vals)
    return vals


def make_tensor(shape, seed, scale=1.0, dtype=torch.bfloat16, device="cpu"):
    """N(0, scale^2) values of the given shape, rounded to dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return (t * scale).to(dtype)
