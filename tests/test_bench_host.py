"""Host logic of bench.py (no GPU): the one-GPU guard and the box mode's
oracle leg.

On a box workload whose boxes tile the tensor exactly (start (0, 0), one box
height per repeat), the three box operations have numpy closed forms: the
copy is a reshape of the tensor, a store from any tensor leaves the image
reshaped, and the add is tensor + image in float32. The oracle leg must find
these equal to its own result, and must report a planted difference.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


SMALL = workloads.BoxWorkload("box_small", 64 * 24, 256, 64)


def closed_form(op, inp):
    G, img = inp["tensor"], inp["image"]
    if op == "box_copy":
        return G.reshape(SMALL.n_repeat, SMALL.box_rows, SMALL.cols).copy()
    if op == "box_store":
        return img.reshape(SMALL.rows, SMALL.cols).copy()
    return G + img.reshape(SMALL.rows, SMALL.cols)


@pytest.mark.parametrize("op", workloads.BOX_OPS)
def test_box_oracle_leg_matches_closed_form(op):
    inp = workloads.make_box_inputs(SMALL, seed=3)
    got = closed_form(op, inp)
    assert got.dtype == np.float32
    rec = bench.box_cpu_baseline(SMALL, op, inp, got, seconds=0.05)
    assert rec["sample_matches_gpu"] is True
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["value"] > 0
    # a difference in the first box must be seen: the sample always covers it
    bad = got.copy()
    bad.reshape(-1)[5] += np.float32(1.0)
    assert bench.box_cpu_baseline(SMALL, op, inp, bad, seconds=0.05)["sample_matches_gpu"] is False


def test_box_workload_bytes():
    bw = workloads.BOX_WORKLOADS["box_f32_524288x256_64x256"]
    assert bw.n_repeat == 8192 and bw.image_bytes == 512 << 20
    assert bw.algorithmic_bytes("box_copy") == bw.algorithmic_bytes("box_store") == 1 << 30
    assert bw.algorithmic_bytes("box_reduce_add") == 3 * (512 << 20)
