"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import pins


@pytest.fixture(scope="module")
def o():
    oracle.build()
    return oracle.default()


@pytest.mark.parametrize("name", sorted(pins.ALL_PINS))
def test_pin(o, name):
    pins.ALL_PINS[name](o)


def test_bf16_quantiser_matches_torch():
    """The input generator's bf16 rounding is round-to-nearest-even (torch's
    float32 -> bfloat16 conversion), including exact ties."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000, dtype=np.float32) * np.float32(3.0)
    ties = (np.arange(-300, 300, dtype=np.int64).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    for v in (x, ties, np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38], np.float32)):
        ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(workloads.f32_to_bf16_bits(v), ref)


def test_workload_table():
    """The five workloads have the shapes, dtypes and repeat counts stated for
    them, and the worked example is K_repeat = 2."""
    W = workloads.WORKLOADS
    assert [(w.M, w.N, w.K, w.dtype) for w in W.values()] == [
        (16, 8, 32, "f16"), (128, 128, 256, "bf16"), (4096, 4096, 4096, "f16"),
        (16, 16384, 16384, "bf16"), (8192, 8192, 8192, "bf16")]
    w = W["tile_16x8x32_f16"]
    assert (w.M_rep, w.N_rep, w.K_rep) == (1, 1, 2)
    assert W["gemm_8192_bf16_ctensor"].algorithmic_bytes == 805306368
    assert W["skinny_16x16384x16384_bf16"].algorithmic_bytes == 538443776


def test_page_example_inputs_match_generator():
    """workloads draws the worked example exactly as the page's recipe does."""
    w = workloads.WORKLOADS["tile_16x8x32_f16"]
    x = workloads.make_inputs(w)
    rng = np.random.default_rng(0)
    a = (rng.integers(-4, 5, (16, 32)) / 4).astype("float16")
    b = (rng.integers(-4, 5, (8, 32)) / 4).astype("float16")
    assert np.array_equal(x["a"][0], a.view(np.uint16))
    assert np.array_equal(x["b"][0], b.view(np.uint16))
