"""Benchmark of the MoE expert-MLP hot path on one MI355X.

One step = the whole path over one batch of synthetic input, forward and
backward: router scores (x . W_g), top-k routing, permutation, the grouped
gate_up GEMM with the fused ScaledSwiGLU epilogue, the grouped down GEMM,
the combine, the permutation of dY, the fused down-projection backward
(dS, dSwiGLU, routing-weight gradient partials), their reduction, both
variable-K weight-gradient GEMMs, the gate_up data gradient, the router
backward (score gradient with the balancing term, dW_g, db) and the combine
of dX with the router's share of it added before its one rounding.
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

# Measured HBM traffic of the grouped GEMMs of a workload (rocprofv3
# FETCH_SIZE and WRITE_SIZE per dispatch, with the same counters' reading of
# a plain 1 GiB device copy), one file a workload; valid only for the kernel
# source it was taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{}.json")
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
        "router_backward": 2.0 * T * d * E,     # dW_g (dX's share: combine)
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
        # dX leaves in bf16 with the router's share (its score gradients
        # and weight) added
        "unpermute_dx": (Tk * 4 + planes * Tk * d * 4 + T * d * 2
                         + T * E * 4 + E * d * 2),
        "router_backward": (T * E * 4 * 3 + Tk * 12 + T * d * 2
                            + E * d * 4),
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
    # a forward-only workload runs the forward kernels of the fwd+bwd
    # workload of the same name, whose record covers them
    names = [workload] + ([workload[:-4]] if workload.endswith("_fwd")
                          else [])
    rec = None
    for name in names:
        try:
            with open(TRAFFIC_FILE.format(name)) as fh:
                rec = json.load(fh)
            workload = name
            break
        except (OSError, ValueError):
            continue
    if rec is None:
        return None
    sha = gemm_source_sha256()
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


# ---------------------------------------------------------------------------
# Counter summaries (``--summarize-counters DIR``, no GPU needed).  DIR holds
# the CSV output (``-d DIR/<run> -o run --output-format csv``) of these
# rocprofv3 runs of this script, each in a process of its own:
#   trace      --kernel-trace --stats              --steps 5 --warmup 1
#   fetch      --pmc FETCH_SIZE --kernel-trace     --steps 2 --warmup 1
#   write      --pmc WRITE_SIZE --kernel-trace     --steps 2 --warmup 1
#   mfma       --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16
#              GRBM_GUI_ACTIVE SQ_BUSY_CYCLES --kernel-trace
#                                                  --steps 2 --warmup 1
#   cal_fetch, cal_write   the same two counters over --copy-calibration
#                          (in DIR or in its parent)
# Each run's dispatches of this library are cut into steps at the router
# score kernel; the first step of each run is dropped (cold caches) and the
# rest are averaged per position in the step.

# the library's kernels in the order one step launches them, per stage
STEP_KERNELS = {
    "bf16": [
        ("router_logits", ["router_logits_kernel"]),
        ("route", ["route_kernel"]),
        ("permute", ["plan_rank_kernel", "plan_scan_kernel",
                     "scatter_kernel"]),
        ("gate_up_swiglu_fwd", ["grouped_gemm_kernel"]),
        ("down_fwd", ["grouped_gemm_kernel"]),
        ("unpermute_y", ["unpermute_kernel"]),
        ("permute_dy", ["permute_rows_kernel"]),
        ("down_swiglu_bwd", ["grouped_gemm_kernel"]),
        ("dp_reduce", ["dp_reduce_kernel"]),
        ("wgrad_down", ["grouped_gemm_kernel"]),
        ("gate_up_dgrad", ["grouped_gemm_kernel"]),
        ("wgrad_gate_up", ["grouped_gemm_kernel"]),
        ("router_backward", ["router_dlogits_kernel",
                             "router_dwg_partial_kernel",
                             "router_dwg_reduce_kernel",
                             "router_aux_final_kernel"]),
        ("unpermute_dx", ["unpermute_kernel"]),
    ],
    "mxfp8": [
        ("router_logits", ["router_logits_kernel"]),
        ("route", ["route_kernel"]),
        ("quant_x", ["quant_rows_kernel"]),
        ("permute", ["plan_rank_kernel", "plan_scan_kernel",
                     "scatter_kernel"]),
        ("quant_weights", ["quant_tokens_kernel", "quant_tokens_kernel"]),
        ("gate_up_swiglu_fwd", ["grouped_gemm_kernel"]),
        ("down_fwd", ["grouped_gemm_kernel"]),
        ("unpermute_y", ["unpermute_kernel"]),
        ("permute_dy", ["permute_rows_kernel"]),
        ("permute_x", ["permute_rows_kernel"]),
        ("quant_bwd_operands", ["quant_rows_kernel"]),
        ("down_swiglu_bwd", ["grouped_gemm_kernel"]),
        ("dp_reduce", ["dp_reduce_kernel"]),
        ("gate_up_dgrad", ["grouped_gemm_kernel"]),
        ("quant_tokens", ["quant_tokens_kernel", "quant_tokens_kernel"]),
        ("wgrad_down", ["grouped_gemm_kernel"]),
        ("wgrad_gate_up", ["grouped_gemm_kernel"]),
        ("router_backward", ["router_dlogits_kernel",
                             "router_dwg_partial_kernel",
                             "router_dwg_reduce_kernel",
                             "router_aux_final_kernel"]),
        ("unpermute_dx", ["unpermute_kernel"]),
    ],
    "mxfp4": [
        ("router_logits", ["router_logits_kernel"]),
        ("route", ["route_kernel"]),
        ("quant_x", ["quant_rows4_kernel"]),
        ("permute", ["plan_rank_kernel", "plan_scan_kernel",
                     "scatter_kernel"]),
        ("quant_weights", ["quant_tokens_kernel", "quant_tokens_kernel"]),
        ("gate_up_swiglu_fwd", ["grouped_gemm_kernel"]),
        ("down_fwd", ["grouped_gemm_kernel"]),
        ("unpermute_y", ["unpermute_kernel"]),
        ("permute_dy", ["permute_rows_kernel"]),
        ("quant_bwd_operands", ["quant_rows_kernel"]),
        ("down_swiglu_bwd", ["grouped_gemm_kernel"]),
        ("dp_reduce", ["dp_reduce_kernel"]),
        ("gate_up_dgrad", ["grouped_gemm_kernel"]),
        ("quant_tokens", ["quant_tokens_kernel", "quant_tokens4_kernel"]),
        ("wgrad_down", ["grouped_gemm_kernel"]),
        ("wgrad_gate_up", ["grouped_gemm_kernel"]),
        ("router_backward", ["router_dlogits_kernel",
                             "router_dwg_partial_kernel",
                             "router_dwg_reduce_kernel",
                             "router_aux_final_kernel"]),
        ("unpermute_dx", ["unpermute_kernel"]),
    ],
}

# MFMA flops one SQ_INSTS_VALU_MFMA_MOPS_* count stands for
MOPS_FLOPS = 512
# SIMDs on the chip (256 CUs x 4), and XCDs (GRBM_GUI_ACTIVE is summed
# over the XCDs' own copies)
N_SIMDS, N_XCDS = 1024, 8


def gemm_alg_bytes(stage, T, d, f, E, k, planes, ntiles):
    """Algorithmic (read, write) HBM bytes of a bf16 GEMM stage: each
    operand read once and each result written once (planes: fp32 partial
    planes of the split-K outputs; ntiles: column tiles of the
    routing-weight gradient partials)."""
    Tk = T * k
    return {
        "gate_up_swiglu_fwd": (Tk * d * 2 + E * 2 * f * d * 2 + Tk * 4,
                               Tk * 2 * f * 2 + Tk * f * 2),
        "down_fwd": (Tk * f * 2 + E * d * f * 2, planes * Tk * d * 4),
        "down_swiglu_bwd": (Tk * d * 2 + E * d * f * 2 + Tk * 2 * f * 2
                            + Tk * 4,
                            Tk * 2 * f * 2 + Tk * ntiles * 4),
        "wgrad_down": (Tk * d * 2 + Tk * f * 2, E * d * f * 2),
        "gate_up_dgrad": (Tk * 2 * f * 2 + E * 2 * f * d * 2,
                          planes * Tk * d * 4),
        "wgrad_gate_up": (Tk * 2 * f * 2 + Tk * d * 2, E * 2 * f * d * 2),
    }.get(stage)


def _base_kernel(name):
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    n = n.replace("moe::", "")
    n = n.split("(")[0]
    return n, n.split("<")[0]


def _steps_of(path, counters):
    """Dispatches of the library's kernels in a rocprofv3 CSV, cut into
    steps: lists of dicts {name, base, grid, ns, <counter>: value}."""
    import csv
    rows = list(csv.DictReader(open(path)))
    by_disp = {}
    for r in rows:
        if "moe::" not in r["Kernel_Name"]:
            continue
        key = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
        ent = by_disp.get(key)
        if ent is None:
            full, base = _base_kernel(r["Kernel_Name"])
            grid = r.get("Grid_Size") or r.get("Grid_Size_X")
            ent = {"name": full, "base": base, "grid": int(grid),
                   "start": int(r["Start_Timestamp"]),
                   "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])}
            by_disp[key] = ent
        if counters and r.get("Counter_Name") in counters:
            ent[r["Counter_Name"]] = (ent.get(r["Counter_Name"], 0.0)
                                      + float(r["Counter_Value"]))
    seq = sorted(by_disp.values(), key=lambda e: e["start"])
    steps, cur = [], None
    for e in seq:
        if e["base"] == "router_logits_kernel":
            cur = []
            steps.append(cur)
        if cur is not None:
            cur.append(e)
    return steps


def _average_steps(steps, keys):
    """Per-position means over the steps after the first."""
    use = steps[1:] if len(steps) > 1 else steps
    n = min(len(s) for s in use)
    out = []
    for i in range(n):
        e = dict(use[0][i])
        for key in keys:
            vals = [s[i][key] for s in use if key in s[i]]
            if vals:
                e[key] = sum(vals) / len(vals)
        out.append(e)
    return out


def _label_stages(seq, family):
    spec = [(st, b) for st, bases in STEP_KERNELS.get(family, [])
            for b in bases]
    p = 0
    for e in seq:
        if p < len(spec) and e["base"] == spec[p][1]:
            e["stage"] = spec[p][0]
            p += 1
        else:
            e["stage"] = "?"
    return seq


def _calibration(path, counter):
    """KiB the counter reads for the plain 1 GiB copies (mean of the last
    five of the six)."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if r["Counter_Name"] == counter and "opy" in r["Kernel_Name"]]
    vals = vals[-5:]
    return sum(vals) / len(vals)


def summarize_counters(root, workload):
    """Print a markdown summary of the counter runs under ``root`` and
    write the grouped-GEMM traffic record ``root/traffic_<workload>.json``
    (the form of profiles/traffic_<workload>.json)."""
    from mixture_experts_expert_top_amd import inputs, moe
    wl = inputs.WORKLOADS[workload]
    T, d, f, E, k = wl.T, wl.d, wl.f, wl.E, wl.k
    mx = wl.prec in ("mxfp8", "mxfp4")
    family = wl.prec
    planes, ntiles = moe.row_planes(f), moe.moe_dp_tiles(f)
    csvp = lambda run, kind: os.path.join(  # noqa: E731
        root, run, f"run_{kind}.csv")
    kt = _average_steps(_steps_of(csvp("trace", "kernel_trace"), None), [
        "ns"])
    fe = _average_steps(_steps_of(csvp("fetch", "counter_collection"),
                                  {"FETCH_SIZE"}), ["FETCH_SIZE"])
    wr = _average_steps(_steps_of(csvp("write", "counter_collection"),
                                  {"WRITE_SIZE"}), ["WRITE_SIZE"])
    mf_keys = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
               "GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "ns"]
    mf = _average_steps(_steps_of(csvp("mfma", "counter_collection"),
                                  set(mf_keys)), mf_keys)
    n = min(len(kt), len(fe), len(wr), len(mf))
    for seq in (fe, wr, mf):
        for i in range(n):
            if seq[i]["base"] != kt[i]["base"]:
                raise SystemExit(f"runs disagree at step position {i}: "
                                 f"{kt[i]['name']} vs {seq[i]['name']}")
    _label_stages(kt, family)
    # the copy calibration runs sit beside the workload's runs or one up
    cal_root = root if os.path.isdir(os.path.join(root, "cal_fetch")) \
        else os.path.dirname(os.path.abspath(root))
    cal_f = _calibration(os.path.join(cal_root, "cal_fetch",
                                      "run_counter_collection.csv"),
                         "FETCH_SIZE")
    cal_w = _calibration(os.path.join(cal_root, "cal_write",
                                      "run_counter_collection.csv"),
                         "WRITE_SIZE")
    gib = float(1 << 30)
    bf, bw = gib / cal_f, gib / cal_w
    peak_mfma = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    lines = []
    mode = "fwd+bwd" if wl.backward else "fwd"
    lines.append(f"# Kernel time and counters, {workload} {mode} (T={T}, "
                 f"d={d}, f={f}, E={E}, k={k}), {wl.prec}")
    lines.append("")
    lines.append("Made on one MI355X with these commands (from /tmp, "
                 "TMPDIR=/tmp; <repo> is the repository root, <out> the "
                 "output folder), then summarized by the last one, which "
                 "uses no GPU:")
    lines.append("")
    lines.append("```")
    run = (f"python3 <repo>/bench.py --workload {workload} "
           "--no-cpu-baseline")
    lines.append(f"rocprofv3 --kernel-trace --stats -d <out>/trace -o run "
                 f"--output-format csv -- {run} --steps 5 --warmup 1")
    for name, ctr in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE"),
                      ("mfma", "SQ_VALU_MFMA_BUSY_CYCLES "
                               "SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE "
                               "SQ_BUSY_CYCLES")):
        lines.append(f"rocprofv3 --pmc {ctr} --kernel-trace -d <out>/{name} "
                     f"-o run --output-format csv -- {run} --steps 2 "
                     "--warmup 1")
    for name, ctr in (("cal_fetch", "FETCH_SIZE"),
                      ("cal_write", "WRITE_SIZE")):
        lines.append(f"rocprofv3 --pmc {ctr} --kernel-trace -d <out>/{name} "
                     f"-o run --output-format csv -- python3 <repo>/bench.py "
                     "--copy-calibration")
    lines.append(f"python3 <repo>/bench.py --summarize-counters <out> "
                 f"--workload {workload}")
    lines.append("```")
    lines.append("")
    lines.append("Per dispatch, averaged over the steps after the first. "
                 "HBM GB/s = (read + write) / duration with the counters "
                 "scaled by the copy calibration below.  MFMA busy = "
                 "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 "
                 "SIMDs) (GRBM_GUI_ACTIVE sums the 8 XCDs' cycles); counted "
                 "TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / duration "
                 "(bf16 MFMAs only; tiles that pass an expert's last row "
                 "are counted whole); clock = GRBM_GUI_ACTIVE / 8 / duration.")
    lines.append("")
    lines.append(f"Copy calibration: a plain 1 GiB device copy reads "
                 f"FETCH_SIZE {cal_f:.0f} KiB and WRITE_SIZE {cal_w:.0f} KiB, "
                 f"so one counted KiB stands for {bf:.1f} B read and "
                 f"{bw:.1f} B written.")
    lines.append("")
    lines.append("| # | stage | kernel | grid | us | read MB | write MB | "
                 "HBM GB/s | % of 8 TB/s | MFMA busy | counted TFLOP/s | "
                 f"% of {peak_mfma / 1000:.1f} PF | clock GHz |")
    lines.append("|---:|---|---|---:|---:|---:|---:|---:|---:|---:|---:|"
                 "---:|---:|")
    stages = {}
    step_us = 0.0
    for i in range(n):
        e = kt[i]
        us = e["ns"] / 1e3
        step_us += us
        rd = fe[i].get("FETCH_SIZE", 0.0) * bf
        wt = wr[i].get("WRITE_SIZE", 0.0) * bw
        gbs = (rd + wt) / (e["ns"] * 1e-9) / 1e9
        m = mf[i]
        gui = m.get("GRBM_GUI_ACTIVE", 0.0)
        busy = m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        util = busy / (gui / N_XCDS * N_SIMDS) if gui else 0.0
        mops = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        tfl = mops * MOPS_FLOPS / (m["ns"] * 1e-9) / 1e12 if mops else 0.0
        clk = gui / N_XCDS / m["ns"] if m["ns"] else 0.0
        is_gemm = e["base"] == "grouped_gemm_kernel"
        short = e["name"].replace("grouped_gemm_kernel", "gg")
        mfma_cols = (f"{util:.3f} | {tfl:.0f} | "
                     f"{100 * tfl / peak_mfma:.1f} | {clk:.2f}"
                     if is_gemm and not mx else
                     (f"{util:.3f} | - | - | {clk:.2f}" if is_gemm
                      else "- | - | - | -"))
        lines.append(f"| {i} | {e['stage']} | `{short}` | {e['grid']} | "
                     f"{us:.1f} | {rd / 1e6:.1f} | {wt / 1e6:.1f} | "
                     f"{gbs:.0f} | {100 * gbs / PEAK_HBM_GBS:.1f} | "
                     f"{mfma_cols} |")
        if is_gemm:
            alg = None if mx else gemm_alg_bytes(e["stage"], T, d, f, E, k,
                                                  planes, ntiles)
            stages[e["stage"]] = {
                "fetch_kib": fe[i].get("FETCH_SIZE", 0.0),
                "write_kib": wr[i].get("WRITE_SIZE", 0.0),
                "us": round(us, 1),
                "mfma_busy": round(util, 4),
                "counted_tflops": round(tfl, 1) if not mx else None,
                "algorithmic_read_bytes": alg[0] if alg else None,
                "algorithmic_write_bytes": alg[1] if alg else None,
            }
    lines.append("")
    lines.append(f"Sum of the step's kernel times: {step_us / 1e3:.3f} ms.")
    # every kernel of the traced run, this library's and torch's (input
    # generation happens outside the timed steps)
    import csv
    stats = list(csv.DictReader(open(csvp("trace", "kernel_stats"))))
    total_ns = sum(float(r["TotalDurationNs"]) for r in stats)
    lines.append("")
    lines.append("Kernel time of the whole traced run (rocprofv3 --stats):")
    lines.append("")
    lines.append("| kernel | calls | avg us | total ms | % |")
    lines.append("|---|---:|---:|---:|---:|")
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        full, base = _base_kernel(r["Name"])
        name = full if "grouped_gemm" in full or "moe" in r["Name"] \
            else "torch:" + base.split("::")[-1][:40]
        lines.append(f"| `{name}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{100 * float(r['TotalDurationNs']) / total_ns:.2f} |")
    if not mx:
        lines.append("")
        lines.append("| GEMM stage | read GB | write GB | algorithmic read GB"
                     " | algorithmic write GB | read / alg | write / alg |")
        lines.append("|---|---:|---:|---:|---:|---:|---:|")
        for st, v in stages.items():
            rd = v["fetch_kib"] * bf
            wt = v["write_kib"] * bw
            ar, aw = v["algorithmic_read_bytes"], v["algorithmic_write_bytes"]
            lines.append(f"| {st} | {rd / 1e9:.3f} | {wt / 1e9:.3f} | "
                         f"{ar / 1e9:.3f} | {aw / 1e9:.3f} | {rd / ar:.2f} | "
                         f"{wt / aw:.2f} |")
    rec = {"workload": workload, "copy_bytes": 1 << 30,
           "kernel_source_sha256": gemm_source_sha256(),
           "copy_fetch_kib": cal_f, "copy_write_kib": cal_w,
           "stages": stages}
    with open(os.path.join(root, f"traffic_{workload}.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print("\n".join(lines))


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
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print the summary of the rocprofv3 counter runs "
                         "under DIR for --workload and write "
                         "DIR/traffic_<workload>.json (no GPU used)")
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
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload)
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
