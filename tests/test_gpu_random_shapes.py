"""Seeded random shapes through every kernel, both atom-K layouts and the
split-K form, against the oracle.

The data are quarter integers (every product and every partial sum exact in
fp32), so any accumulation order gives the oracle's bits: each result must
equal the oracle's D bit for bit. The shapes (batch 1-2, M a multiple of 16 up
to 512, N a multiple of 8 up to 512, K a multiple of 16 up to 1024, zero
included) cross tile edges, K tails and single-atom extents that the fixed
cases do not.
"""
import numpy as np
import pytest
import torch

import bf16_matrix_multiply_amd as bmm
import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

KERNELS = ["direct", "tiled", "skinny", "tiled128", "tiled256x128"]


def _cases():
    rng = np.random.default_rng(2026)
    cases = []
    for i in range(16):
        batch = int(rng.integers(1, 3))
        M = 16 * int(rng.integers(1, 33))
        N = 8 * int(rng.integers(1, 65))
        K = 16 * int(rng.integers(0, 65))
        dtype = "f16" if i % 2 else "bf16"
        c_tensor = bool(i % 3 != 0)
        cases.append(workloads.custom(batch, M, N, K, dtype, "quarter", "quarter",
                                      c_tensor=c_tensor, c_scalar=0.0 if c_tensor else 0.75,
                                      name=f"rand{i}_{batch}x{M}x{N}x{K}_{dtype}"))
    return cases


CASES = _cases()


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_random_shape_all_forms(w):
    inp = workloads.make_inputs(w, seed=5)
    Ao, Bo = gu.oracle_operands(w, inp)
    ref = oracle.mma(Ao, Bo, inp["c_tensor"], inp["c_scalar"], w.dtype)
    a, b = gu.dev_u16(inp["a"]), gu.dev_u16(inp["b"])
    C = None if inp["c_tensor"] is None else torch.from_numpy(inp["c_tensor"]).cuda()
    c = float(inp["c_scalar"])
    shape = (w.batch, w.M_rep, w.N_rep, 16, 8)
    for ka in (16, 8):
        A = bmm.pack_operand(a, 16, atom_k=ka)
        B = bmm.pack_operand(b, 8, atom_k=ka)
        for kernel in KERNELS:
            out = torch.full(shape, float("nan"), device="cuda")
            D = bmm.mma_tile(A, B, C, c, w.dtype, out=out, kernel=kernel).cpu().numpy()
            bad = np.argwhere(D.view(np.uint32) != ref.view(np.uint32))
            assert bad.size == 0, f"{w.name} k={ka} {kernel}: {len(bad)} mismatches, first {bad[:3].tolist()}"
        out = torch.full(shape, float("nan"), device="cuda")
        D = bmm.mma_tile_splitk(A, B, C, c, w.dtype, 3, out=out).cpu().numpy()
        bad = np.argwhere(D.view(np.uint32) != ref.view(np.uint32))
        assert bad.size == 0, f"{w.name} k={ka} split-K: {len(bad)} mismatches, first {bad[:3].tolist()}"


@pytest.mark.parametrize("w", CASES[:8], ids=[w.name for w in CASES[:8]])
def test_random_shape_scaled(w):
    """alpha/beta form with alpha = 0.5, beta = -1.5: on quarter-integer data
    every term is exact and fma(alpha, P, fl(beta * C)) rounds nothing, so each
    kernel must give the oracle's bits."""
    inp = workloads.make_inputs(w, seed=9)
    Ao, Bo = gu.oracle_operands(w, inp)
    ref = oracle.mma_scaled(Ao, Bo, inp["c_tensor"], inp["c_scalar"], 0.5, -1.5, w.dtype)
    A = bmm.pack_operand(gu.dev_u16(inp["a"]), 16)
    B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8)
    C = None if inp["c_tensor"] is None else torch.from_numpy(inp["c_tensor"]).cuda()
    for kernel in KERNELS:
        out = torch.full((w.batch, w.M_rep, w.N_rep, 16, 8), float("nan"), device="cuda")
        D = bmm.mma_tile(A, B, C, float(inp["c_scalar"]), w.dtype, out=out, kernel=kernel,
                         alpha=0.5, beta=-1.5).cpu().numpy()
        bad = np.argwhere(D.view(np.uint32) != ref.view(np.uint32))
        assert bad.size == 0, f"{w.name} {kernel} scaled: {len(bad)} mismatches, first {bad[:3].tolist()}"
