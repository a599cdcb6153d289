"""Benchmark of the MoE expert-MLP hot path on one MI355X.

One step = the whole path over one batch of synthetic input, forward and
backward: router scores (x . W_g), top-k routing, permutation, the grouped
gate_up GEMM with the fused ScaledSwiGLU epilogue, the grouped down GEMM,
the combine, the permutation of dY, the fused down-projection backward
(dS, dSwiGLU, routing-weight gradient partials), their reduction, both
variable-K weight-gradient GEMMs, the gate_up data gradient, the combine
of dX (fp32) and the router backward (score gradient with the balancing
term, dW_g, db, and the router's share of dX added before its rounding).
Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  Default workload: the Mixtral-8x7B-shaped layer,
forward+backward in bf16 (T=8192 tokens as 2 x 4096, d=4096, f=14336, E=8,
top-2, renormalised), random weights and inputs.  ``--workload mxfp8`` runs
the same layer at T=16384 with MXFP8 GEMM operands (the quantization of x,
of the weights, of dY and of every backward operand inside the step).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("MoE-layer fwd+bwd tokens/s & TFLOP/s (% MFMA peak), "
          "Mixtral shape, 1 MI355X")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 (MX) MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published

# Measured HBM traffic of the dominant kernel (rocprofv3 FETCH_SIZE and
# WRITE_SIZE per dispatch, with the same counters' reading of a plain 1 GiB
# device copy); valid only for the kernel source it was taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Recorded whole-chip MFMA ceiling with random operands (power-limited
# clock): a measured figure, read as data.
CEILING_FILE = os.path.join(ROOT, "profiles", "mfma_ceiling.json")
# the grouped GEMM kernel's sources: the recorded traffic is valid only
# for the sources it was measured on
GEMM_SOURCES = [os.path.join(ROOT, "mixture_experts_expert_top_amd", "csrc", n)
                for n in ("gemm.hip", "common.cuh", "internal.h", "mx.cuh")]


def gemm_source_sha256():
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()

# the five named configurations and the workloads that implement them
CONFIGS = {"C1": "tiny_fwd", "C2": "mixtral_fwd", "C3": "mixtral",
           "C4": "finegrain", "C5": "mxfp8"}

GEMM_STAGES = ("gate_up_swiglu_fwd", "down_fwd", "down_swiglu_bwd",
               "wgrad_down", "gate_up_dgrad", "wgrad_gate_up")


def stage_flops(name, T, d, f, E, k):
    Tk = T * k
    return {
        "router_logits": 2.0 * T * d * E,
        "router_backward": 4.0 * T * d * E,
        "gate_up_swiglu_fwd": 4.0 * Tk * d * f,
        "down_fwd": 2.0 * Tk * d * f,
        "down_swiglu_bwd": 2.0 * Tk * d * f,
        "wgrad_down": 2.0 * Tk * d * f,
        "gate_up_dgrad": 4.0 * Tk * d * f,
        "wgrad_gate_up": 4.0 * Tk * d * f,
    }.get(name, 0.0)


def stage_bytes(name, T, d, f, E, k, planes=1, mx=False, act4=False):
    """Algorithmic HBM bytes of the memory-bound stages (each tensor read
    or written once; the fp32 rows the combines read come as `planes`
    partial-sum planes; an MXFP8 row of n codes is n * 33/32 bytes, an
    MXFP4 row n * 17/32)."""
    Tk = T * k
    q4 = 17.0 / 32.0                           # bytes per MXFP4 value
    q = 33.0 / 32.0                            # bytes per MXFP8 value
    xb = (q4 if act4 else q) if mx else 2.0    # bytes per permuted x value
    return {
        "route": T * E * 4 + Tk * 8,
        "permute": Tk * 8 + T * d * xb + Tk * d * xb + Tk * 12 + E * 8,
        "unpermute_y": Tk * 4 + planes * Tk * d * 4 + T * d * 2,
        "permute_dy": Tk * 4 + T * d * 2 + Tk * d * 2,
        "permute_x": Tk * 4 + T * d * 2 + Tk * d * 2,
        "unpermute_dx": Tk * 4 + planes * Tk * d * 4 + T * d * 4,
        "router_backward": (T * E * 4 * 3 + Tk * 12 + T * d * 2 + E * d * 2
                            + T * d * 4 + T * d * 2 + E * d * 4),
        "quant_x": T * d * (2 + xb),
        # training: both MX layouts of each weight from one bf16 read
        "quant_weights": 3 * E * d * f * (2 + 2 * q),
        "quant_bwd_operands": Tk * d * (2 + q),
        # dO along tokens from bf16, and Xp from bf16 (MXFP8) or from the
        # MXFP4 payload (MXFP4 activations)
        "quant_tokens": Tk * d * (2 + q) + Tk * d * ((q4 + q4) if act4
                                                    else (2 + q)),
    }.get(name, 0)


def measured_traffic(workload, stage):
    """HBM bytes per launch of ``stage`` from the recorded counter runs,
    scaled by the copy calibration; None when there is no record for this
    workload and stage or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
        sha = gemm_source_sha256()
    except (OSError, ValueError):
        return None
    st = rec.get("stages", {}).get(stage)
    if (rec.get("workload") != workload or st is None
            or rec.get("kernel_source_sha256") != sha):
        return None
    fetch = st["fetch_kib"] * rec["copy_bytes"] / rec["copy_fetch_kib"]
    write = st["write_kib"] * rec["copy_bytes"] / rec["copy_write_kib"]
    return round(fetch + write)


def measured_ceiling(prec):
    """TFLOP/s that MFMAs alone sustain on the whole chip with random
    operands of the path's GEMM type; None when not recorded."""
    key = "bf16" if prec == "bf16" else "fp8"
    try:
        with open(CEILING_FILE) as fh:
            rec = json.load(fh)
        return float(rec[key]["random"]["tflops"])
    except (OSError, ValueError, KeyError):
        return None


def copy_calibration():
    """A plain device copy of 1 GiB, five times: the reference that scales
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = 1 << 28                                   # fp32 elements = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(6):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 4 * n, "copies": 6}), flush=True)


def cpu_baseline(inp, wl, n_tokens):
    """The float64 oracle, untuned, on the first n_tokens tokens of the same
    workload (router scores, routing, experts, combine and backward)."""
    import numpy as np
    from oracle import moe_ref
    blas = "blas"
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in infos] or [1])
        if infos:
            blas = infos[0].get("internal_api", "blas")
    except Exception:  # pragma: no cover - informational only
        threads = len(os.sched_getaffinity(0))
    h = lambda t: t.double().cpu().numpy()  # noqa: E731
    x = h(inp["x"][:n_tokens])
    dy = h(inp["dy"][:n_tokens])
    w_g = h(inp["w_g"])
    bias = None if inp["bias"] is None else h(inp["bias"])
    w_gu = h(inp["w_gu"])
    w2 = h(inp["w2"])
    t0 = time.perf_counter()
    logits = moe_ref.router_logits(x, w_g, bias)
    fwd = moe_ref.moe_forward(x, logits, w_gu, w2, wl.k)
    if wl.backward:
        bwd = moe_ref.moe_backward(fwd, dy, w_gu, w2)
        dl = moe_ref.routing_weight_backward(logits, fwd["idx"], fwd["p"],
                                             bwd["dp"], wl.renorm)
        dl = dl + moe_ref.aux_loss(logits, fwd["counts"], 0.01)[1]
        moe_ref.router_backward(x, w_g, dl)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"first {n_tokens} tokens of the {wl.name} workload, "
                       f"{'fwd+bwd' if wl.backward else 'fwd'}, float64 numpy "
                       f"per-expert loop with the full weights ({dt:.1f} s, "
                       f"{blas}, {threads} threads)")}


def cpu_baseline_mx(inp, wl, d_slice=384, f_slice=1344):
    """The float64 MX oracle, untuned, on every token of the workload but a
    slice of the layer's features (the first d_slice hidden and f_slice
    intermediate features of every expert), forward and backward with every
    quantization inside the timed region, scaled by d*f / (d_slice*f_slice):
    the oracle's GEMMs and its codec work are proportional to d*f.  Its
    routing, dispatch plan and per-token loops are not, and are scaled too,
    so the value is a lower bound on the oracle's full-layer rate.  The full
    layer is out of reach for a bounded run: the oracle's codec spends about
    15 s on one 28672 x 4096 weight matrix, and a step quantizes 24."""
    from oracle import moe_mx, moe_ref
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in infos] or [1])
        blas = infos[0].get("internal_api", "blas") if infos else "blas"
    except Exception:  # pragma: no cover - informational only
        threads, blas = len(os.sched_getaffinity(0)), "blas"
    T, d, f = wl.T, wl.d, wl.f
    ds, fs = min(d_slice, d), min(f_slice, f)
    h = lambda t: t.double().cpu().numpy()  # noqa: E731
    x = h(inp["x"][:, :ds])
    dy = h(inp["dy"][:, :ds])
    w_gu = inp["w_gu"]
    w_gu = h(torch_cat_gate_up(w_gu, f, fs, ds))
    w2 = h(inp["w2"][:, :ds, :fs])
    logits = h(inp["logits"])
    act4 = wl.prec == "mxfp4"
    t0 = time.perf_counter()
    fwd = moe_mx.moe_forward_mx(x, logits, w_gu, w2, wl.k, act4=act4)
    bwd = moe_mx.moe_backward_mx(fwd, dy, w_gu, w2)
    moe_ref.routing_weight_backward(logits, fwd["idx"], fwd["p"], bwd["dp"],
                                    wl.renorm)
    dt = time.perf_counter() - t0
    scale = (d * f) / (ds * fs)
    return {"value": T / (dt * scale), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"all {T} tokens of the {wl.name} workload, fwd+bwd, "
                       f"float64 numpy MX oracle on the first {ds} hidden and "
                       f"{fs} intermediate features of every expert "
                       f"({dt:.1f} s, {blas}, {threads} threads), scaled by "
                       f"d*f/({ds}*{fs}) = {scale:.0f}, which scales the "
                       f"oracle's per-token loops too: a lower bound on its "
                       f"full-layer rate)")}


def torch_cat_gate_up(w_gu, f, fs, ds):
    """The gate rows [0, fs) and up rows [f, f + fs) of every expert, first
    ds columns."""
    import torch
    return torch.cat([w_gu[:, :fs, :ds], w_gu[:, f:f + fs, :ds]], dim=1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral",
                    help="mixtral (default), mixtral_fwd, mxfp8, mxfp4, "
                         "finegrain, tiny, tiny_fwd")
    ap.add_argument("--config", choices=sorted(CONFIGS),
                    help="C1..C5: the tiny, Mixtral forward, Mixtral "
                         "fwd+bwd, fine-grained and MXFP8 workloads")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured as a HIP graph and "
                         "replayed (reported under 'graph')")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 1 GiB device copy that calibrates "
                         "the HBM traffic counters")
    args = ap.parse_args()
    if args.config:
        args.workload = CONFIGS[args.config]
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not "
              "supported (this build has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    from mixture_experts_expert_top_amd import inputs, moe
    from mixture_experts_expert_top_amd.layer import (MoEPath, MoEPathMX,
                                                      StageTimers, StepGraph)

    wl = inputs.WORKLOADS[args.workload]
    mx = wl.prec in ("mxfp8", "mxfp4")
    peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    ceiling = measured_ceiling(wl.prec)
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.k
    dev = torch.device("cuda:0")
    inp = inputs.make_inputs(wl, seed=0, device=dev)
    if mx:
        path = MoEPathMX(T, d, f, E, k, device=dev,
                         act_fp4=wl.prec == "mxfp4")
    else:
        path = MoEPath(T, d, f, E, k, device=dev)

    def step(timers=None):
        path.forward(inp["x"], inp["w_gu"], inp["w2"], w_g=inp["w_g"],
                     bias=inp["bias"], timers=timers)
        if wl.backward:
            path.backward(inp["dy"], inp["w_gu"], inp["w2"], timers=timers)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    timers = StageTimers()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step(timers)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(end) / args.steps

    stage_ms = timers.mean_ms()
    gemm_stages = [n for n in GEMM_STAGES if n in stage_ms]
    gemm_flops = sum(stage_flops(n, T, d, f, E, k) for n in gemm_stages)
    all_flops = gemm_flops + sum(stage_flops(n, T, d, f, E, k)
                                 for n in ("router_logits", "router_backward")
                                 if n in stage_ms)
    tokens_s = T / (ms / 1e3)
    dom = max(gemm_stages, key=lambda n: stage_ms[n])
    dom_tflops = stage_flops(dom, T, d, f, E, k) / (stage_ms[dom] / 1e3) / 1e12
    gemm_ms = sum(stage_ms[n] for n in gemm_stages)
    stages = {}
    for n, v in stage_ms.items():
        e = {"ms": round(v, 4)}
        fl = stage_flops(n, T, d, f, E, k)
        by = stage_bytes(n, T, d, f, E, k, planes=moe.row_planes(f), mx=mx,
                         act4=wl.prec == "mxfp4")
        if fl:
            e["tflops"] = round(fl / (v / 1e3) / 1e12, 1)
        if by:
            e["gbs"] = round(by / (v / 1e3) / 1e9, 1)
        stages[n] = e

    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"mxfp8": "mxfp8-e4m3", "mxfp4": "mxfp8-e4m3+mxfp4-act",
                  "bf16": "bf16"}[wl.prec],
        "data": "synthetic",
        "config": {"workload": f"{wl.name} {'fwd+bwd' if wl.backward else 'fwd'}",
                   "T": T, "d": d, "f": f,
                   "E": E, "k": k, "renorm": wl.renorm,
                   "router_bias": wl.router_bias},
        "tflops": round(all_flops / (ms / 1e3) / 1e12, 1),
        "pct_mfma_peak": round(100.0 * all_flops / (ms / 1e3) / 1e12
                               / peak, 2),
        "gemm_tflops": round(gemm_flops / (gemm_ms / 1e3) / 1e12, 1),
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(dom_tflops, 1),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(dom_tflops / peak, 4),
            "traffic": measured_traffic(wl.name, dom),
            "ceiling_random_operands": ceiling,
            "frac_of_ceiling": (round(dom_tflops / ceiling, 4)
                                if ceiling else None),
        },
        "stages": stages,
        "wall_s": round(wall, 3),
    }
    if args.graph:
        g = StepGraph(step)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        gs = torch.cuda.Event(enable_timing=True)
        ge = torch.cuda.Event(enable_timing=True)
        gs.record()
        for _ in range(args.steps):
            g.replay()
        ge.record()
        torch.cuda.synchronize()
        gms = gs.elapsed_time(ge) / args.steps
        out["graph"] = {"ms_per_step": round(gms, 4),
                        "tokens_per_s": round(T / (gms / 1e3), 1)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline_mx(inp, wl) if mx else
                               cpu_baseline(inp, wl, min(args.cpu_tokens, T)))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
