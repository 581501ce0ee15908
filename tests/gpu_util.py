"""Helpers for the GPU parity tests: move seeded inputs to the GPU, run the
HIP path through the binding, and compare with the oracle."""
import numpy as np
import torch

import bf16_matrix_multiply_amd as bmm
import oracle
import workloads
from tests import util

DEV = "cuda"
BOUND_SCALE = 1e-3   # normal inputs: |D - D_ref| <= 1e-3 * (|A||B|^T + |C|)


def dev_u16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)


def host_u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def gpu_run(w, inp, kernel="auto", c_override=None):
    """Pack on the GPU and multiply; returns (A_dev, B_dev, C_dev, D_host)."""
    a, b = dev_u16(inp["a"]), dev_u16(inp["b"])
    A = bmm.pack_operand(a, 16)
    B = bmm.pack_operand(b, 8)
    C = None if inp["c_tensor"] is None else torch.from_numpy(inp["c_tensor"]).to(DEV)
    out = torch.full((w.batch, w.M_rep, w.N_rep, 16, 8), float("nan"), device=DEV)
    D = bmm.mma_tile(A, B, C, float(inp["c_scalar"]), w.dtype, out=out, kernel=kernel)
    torch.cuda.synchronize()
    return A, B, C, D.cpu().numpy()


def oracle_operands(w, inp):
    return oracle.pack(inp["a"], 16), oracle.pack(inp["b"], 8)


def assert_parity_full(w, inp, D, kernel=""):
    """Whole-output comparison with the oracle."""
    A, B = oracle_operands(w, inp)
    ref = oracle.mma(A, B, inp["c_tensor"], inp["c_scalar"], w.dtype)
    assert not np.isnan(D).any(), f"{w.name}/{kernel}: unwritten (NaN-poisoned) outputs"
    if w.exact:
        bad = np.argwhere(D != ref)
        assert bad.size == 0, f"{w.name}/{kernel}: {len(bad)} mismatches, first {bad[:4].tolist()}"
    else:
        bnd = oracle.bound(A, B, inp["c_tensor"], inp["c_scalar"], w.dtype)
        err = np.abs(D.astype(np.float64) - ref)
        ratio = float((err / (BOUND_SCALE * bnd.astype(np.float64) + 1e-300)).max())
        assert (err <= BOUND_SCALE * bnd).all(), f"{w.name}/{kernel}: worst err/bound {ratio}"


def assert_parity_sampled(w, inp, D, count=2048, seed=11, A=None, B=None):
    """Sampled outputs (random + corners) against the oracle computed one by one."""
    if A is None:
        A, B = oracle_operands(w, inp)
    rng = np.random.default_rng(seed)
    idx = util.sample_indices(rng, w.batch, w.M, w.N, count)
    ref = oracle.mma_sampled(A, B, inp["c_tensor"], inp["c_scalar"], w.dtype, idx)
    Dl = util.tile_to_logical(D)
    got = Dl[idx[:, 0], idx[:, 1], idx[:, 2]]
    assert not np.isnan(Dl).any(), f"{w.name}: unwritten (NaN-poisoned) outputs"
    if w.exact:
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, f"{w.name}: {bad.size} sampled mismatches, e.g. {idx[bad[:4]].tolist()}"
    else:
        bnd = oracle.bound(A, B, inp["c_tensor"], inp["c_scalar"], w.dtype, idx)
        err = np.abs(got.astype(np.float64) - ref)
        assert (err <= BOUND_SCALE * bnd).all(), \
            f"{w.name}: worst err/bound {float((err / (BOUND_SCALE * bnd)).max())}"
    return A, B
