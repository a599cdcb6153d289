"""Host logic of bench.py that needs no GPU: the recorded ceilings and
traffic are read back as stored, and --gpus above 1 is refused."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_ceiling_matches_record():
    with open(bench.CEILING_FILE) as fh:
        rec = json.load(fh)
    assert bench.measured_ceiling("bf16") == rec["bf16"]["random"]["tflops"]
    assert bench.measured_ceiling("mxfp8") == rec["fp8"]["random"]["tflops"]
    assert bench.measured_ceiling("mxfp4") == rec["fp8"]["random"]["tflops"]
    # the random-operand ceiling sits below the nominal peaks
    assert 0 < bench.measured_ceiling("bf16") < bench.PEAK_BF16_TFLOPS
    assert 0 < bench.measured_ceiling("mxfp8") < bench.PEAK_FP8_TFLOPS


def test_traffic_is_null_for_other_workloads():
    assert bench.measured_traffic("no-such-workload", "gate_up_dgrad") is None
    assert bench.measured_traffic("mixtral", "no-such-stage") is None


def test_multi_gpu_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                          "--gpus", "2"], capture_output=True, text=True,
                         timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
