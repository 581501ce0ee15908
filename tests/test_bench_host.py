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
                       capture_output=True, text=True, timeout=300)
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


def test_traffic_records_per_configuration():
    """A traffic record applies to the configuration it was taken in: the plain
    k = 16 multiply at 8192^3 has one (and it is current), a variant such as
    the alpha/beta form or split-K reports none."""
    import json
    from bf16_matrix_multiply_amd.profile_run import source_sha
    rec = json.load(open(os.path.join(ROOT, "profiles",
                                      "traffic_mma_tile_gemm_8192_bf16_ctensor.json")))
    assert rec["source_sha"] == source_sha("mma_tile")
    got = bench.traffic_from_profiles("mma_tile", "gemm_8192_bf16_ctensor")
    assert got == rec["hbm_bytes_per_launch"] and got > rec["algorithmic_bytes_per_launch"]
    for variant in ("scaled", "k8", "splitk2", "tiled128"):
        assert bench.traffic_from_profiles("mma_tile", "gemm_8192_bf16_ctensor", variant) is None
    # a multiply record holds only for the kernel it was taken with
    assert rec["mma_kernel"] == "tiled"
    assert bench.traffic_from_profiles("mma_tile", "gemm_8192_bf16_ctensor", "", "tiled") == got
    assert bench.traffic_from_profiles("mma_tile", "gemm_8192_bf16_ctensor", "", "skinny") is None
    assert bench.traffic_from_profiles("pack_operand_kmajor", "gemm_8192_bf16_ctensor") > 0


# The shape of `amd-smi metric -p -c --json` for one GPU (two of its eight XCD
# clocks shown), as the tool printed it on an MI355X machine.
AMD_SMI_SAMPLE = """{
    "gpu_data": [
        {
            "gpu": 0,
            "power": {
                "socket_power": {
                    "value": 1397,
                    "unit": "W"
                },
                "gfx_voltage": "N/A",
                "throttle_status": "N/A"
            },
            "clock": {
                "gfx_0": {
                    "clk": {
                        "value": 1558,
                        "unit": "MHz"
                    },
                    "min_clk": {
                        "value": 500,
                        "unit": "MHz"
                    }
                },
                "gfx_1": {
                    "clk": {
                        "value": 1498,
                        "unit": "MHz"
                    }
                }
            }
        }
    ]
}"""


def test_parse_amd_smi_metric():
    assert bench.parse_amd_smi_metric(AMD_SMI_SAMPLE) == (1397, [1558, 1498])
    assert bench.parse_amd_smi_metric("") == (None, [])
    assert bench.parse_amd_smi_metric("command not found") == (None, [])


def test_summarize_power_drops_unsettled_and_ragged_samples():
    """Samples before the settle time are left out; a sample that lists fewer
    XCD clocks than the others still counts for power but not for the clocks."""
    samples = [(0.5, 900, [2400, 2400]), (1.2, 1398, [1800, 1900]), (1.6, 1400, [1820]),
               (2.1, 1396, [1840, 1880]), (2.6, 1399, [])]
    p = bench.summarize_power(samples, 1.0, 740.04)
    assert p["samples"] == 4 and p["socket_w_max"] == 1400
    assert p["socket_w_median"] == 1398.5
    assert p["gfx_clock_mhz_median_per_xcd"] == [1820, 1890]
    assert p["us_per_call_wall"] == 740.0
    assert bench.summarize_power(samples[:1], 1.0, 740.0) is None
    assert bench.summarize_power([(1.5, 1390, [])], 1.0, 1.0)["gfx_clock_mhz_median_per_xcd"] is None


def test_extra_records_name_the_two_roofline_configs():
    """The extra records of the default run are the two other configurations
    with a roofline target: 4096^3 against the MFMA peak, the skinny shape
    against HBM."""
    assert bench.EXTRA_RECORDS == ("gemm_4096_f16_quarter", "skinny_16x16384x16384_bf16")
    for name in bench.EXTRA_RECORDS:
        w = workloads.WORKLOADS[name]
        hbm = w.flops / w.algorithmic_bytes < bench.RIDGE_FLOP_PER_BYTE
        assert hbm == (name.startswith("skinny"))
