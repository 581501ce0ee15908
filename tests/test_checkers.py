"""The GPU tests' whole-output checkers, run on the CPU against the oracle's
own results: they accept the oracle's output and reject a single changed
output (so a GPU result that passes them has every output right)."""
import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as gu


@pytest.mark.parametrize("dtype,dist", [("bf16", "quarter"), ("f16", "quarter"),
                                        ("bf16", "ternary"), ("f16", "ternary")])
@pytest.mark.parametrize("c_tensor", [True, False])
def test_quarter_sums_accept_oracle_and_catch_one_output(c_tensor, dtype, dist):
    w = workloads.custom(2, 48, 40, 96, dtype, dist, dist, c_tensor=c_tensor,
                         c_scalar=-1.25, name="checker")
    inp = workloads.make_inputs(w, seed=2)
    A, B = oracle.pack(inp["a"], 16), oracle.pack(inp["b"], 8)
    D = oracle.mma(A, B, inp["c_tensor"], inp["c_scalar"], w.dtype)
    gu.assert_quarter_sums(w, inp, D)
    for pos, delta in (((1, 2, 3, 7, 5), 1 / 16), ((0, 0, 0, 0, 0), -1 / 16)):
        bad = D.copy()
        bad[pos] += np.float32(delta)
        with pytest.raises(AssertionError):
            gu.assert_quarter_sums(w, inp, bad)
    nan = D.copy()
    nan[0, 1, 1, 3, 2] = np.nan
    with pytest.raises(AssertionError):
        gu.assert_quarter_sums(w, inp, nan)


def test_per_tile_indices_cover_every_tile():
    w = workloads.custom(1, 8192, 8192, 32, "bf16", name="cover")
    idx = gu.per_tile_indices(w, 256, 256, per_tile=2)
    tiles = {(int(m) // 256, int(n) // 256) for _, m, n in idx}
    assert len(tiles) == 32 * 32
    assert idx[:, 1].max() < w.M and idx[:, 2].max() < w.N and idx.min() >= 0
    w2 = workloads.custom(1, 272, 520, 32, "bf16", name="ragged")
    idx2 = gu.per_tile_indices(w2, 256, 128, per_tile=1)
    assert {(int(m) // 256, int(n) // 128) for _, m, n in idx2} == \
        {(a, b) for a in range(2) for b in range(5)}
    assert idx2[:, 1].max() < w2.M and idx2[:, 2].max() < w2.N
