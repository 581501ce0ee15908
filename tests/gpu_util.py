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


def per_tile_indices(w, tile_m=256, tile_n=256, per_tile=2, seed=13):
    """(count, 3) samples with ``per_tile`` random outputs inside every
    tile_m x tile_n block of D (every macro tile, so every workgroup slot and
    every XCD of the launch), plus the last row and column."""
    rng = np.random.default_rng(seed)
    out = []
    for b in range(w.batch):
        for m0 in range(0, w.M, tile_m):
            hm = min(tile_m, w.M - m0)
            for n0 in range(0, w.N, tile_n):
                hn = min(tile_n, w.N - n0)
                for _ in range(per_tile):
                    out.append((b, m0 + rng.integers(0, hm), n0 + rng.integers(0, hn)))
        out += [(b, w.M - 1, n) for n in (0, w.N - 1)] + [(b, m, w.N - 1) for m in (0, w.M // 2)]
    return np.array(out, np.int64)


def assert_quarter_sums(w, inp, D):
    """Quarter-integer operands (and C on the quarter grid): every product and
    partial sum is exact in fp32, so 16*D is an integer matrix whose every row
    sum and column sum equals its int64 closed form
    16*C + sum_k (4a)(4b) (mma.sync page, worked 16x8 example: the result is
    a.b^T exactly). Checks every output of D through its row and column."""
    assert w.exact
    Dl = util.tile_to_logical(D).astype(np.float64)
    assert not np.isnan(Dl).any(), f"{w.name}: unwritten (NaN-poisoned) outputs"
    D16 = np.rint(Dl * 16).astype(np.int64)
    assert np.array_equal(D16.astype(np.float64), Dl * 16), f"{w.name}: off the 1/16 grid"
    if inp["c_tensor"] is not None:
        C16 = np.rint(util.tile_to_logical(inp["c_tensor"]).astype(np.float64) * 16).astype(np.int64)
    else:
        C16 = np.full(D16.shape, int(round(16 * float(inp["c_scalar"]))), np.int64)
    # The operands are multiples of 1/4 with |x| <= 1, so every product and
    # every partial sum of these row and column totals is a multiple of 1/16
    # far below 2^48: float64 (BLAS) computes them exactly.
    chunk = 1 << 18   # K values decoded at a time (long-K cases hold GBs of operands)
    for b in range(w.batch):
        rows = np.zeros(w.M, np.float64)
        cols = np.zeros(w.N, np.float64)
        half = torch.bfloat16 if w.dtype == "bf16" else torch.float16
        for k0 in range(0, w.K, chunk):
            # decoded on the host by torch's own half -> float64 conversion
            ai = torch.from_numpy(np.ascontiguousarray(inp["a"][b][:, k0:k0 + chunk])
                                  .view(np.int16)).view(half).to(torch.float64)
            bi = torch.from_numpy(np.ascontiguousarray(inp["b"][b][:, k0:k0 + chunk])
                                  .view(np.int16)).view(half).to(torch.float64)
            assert float(ai.abs().max()) <= 1 and float(bi.abs().max()) <= 1
            rows += (ai @ bi.sum(dim=0)).numpy()
            cols += (bi @ ai.sum(dim=0)).numpy()
        assert max(np.abs(rows).max(), np.abs(cols).max()) < 2.0 ** 44
        r16, c16 = rows * 16, cols * 16
        assert np.array_equal(r16, np.rint(r16)) and np.array_equal(c16, np.rint(c16))
        rows = C16[b].sum(axis=1) + r16.astype(np.int64)
        cols = C16[b].sum(axis=0) + c16.astype(np.int64)
        bad_r = np.nonzero(D16[b].sum(axis=1) != rows)[0]
        bad_c = np.nonzero(D16[b].sum(axis=0) != cols)[0]
        assert bad_r.size == 0 and bad_c.size == 0, \
            f"{w.name}: rows {bad_r[:4].tolist()} and columns {bad_c[:4].tolist()} differ"


def assert_parity_sampled(w, inp, D, count=2048, seed=11, A=None, B=None, idx=None):
    """Sampled outputs (random + corners, or the given ``idx``) against the
    oracle computed one by one."""
    if A is None:
        A, B = oracle_operands(w, inp)
    rng = np.random.default_rng(seed)
    if idx is None:
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
