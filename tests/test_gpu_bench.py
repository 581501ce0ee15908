"""bench.py end to end on the GPU: the JSON line carries every field of the
bench contract, the roofline and CPU-oracle legs included, and the oracle
leg's sample agrees with the GPU result.

Small and short runs: the 128 x 128 x 256 workload for the multiply path, and
the box workload with two timed calls per op.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
          "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline",
          "cpu_baseline")


def run_bench(*args):
    print(f"[test_gpu_bench] bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def check_line(d, unit):
    for f in FIELDS:
        assert f in d, f
    assert d["n_gpus"] == 1 and d["data"] == "synthetic" and d["vs_baseline"] is None
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["unit"] == unit
    rf = d["roofline"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) <= 5.1e-5   # frac has 4 decimals
    assert rf["bound"] in ("mfma", "hbm") and rf["avg_launch_us"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["sample_matches_gpu"] is True


def test_bench_small_multiply():
    d = run_bench("--workload", "gemm_128x128x256_bf16_ctensor", "--steps", "3", "--warmup", "1",
                  "--cpu-seconds", "0.5")
    check_line(d, "TFLOP/s")
    assert d["config"]["workload"] == "gemm_128x128x256_bf16_ctensor"
    assert d["dtype"] == "bf16"


@pytest.mark.parametrize("op", ["box_copy", "box_store", "box_reduce_add"])
def test_bench_box_mode(op):
    d = run_bench("--op", op, "--steps", "2", "--warmup", "1", "--cpu-seconds", "0.5")
    check_line(d, "GB/s")
    assert d["config"]["op"] == op and d["roofline"]["bound"] == "hbm"
    assert d["dtype"] == "f32"
