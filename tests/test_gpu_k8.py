"""GPU parity of the k = 8 atom layout (the m16n8k8 form of the mma.sync page):
bmm_pack_operand_k8 against the oracle's k = 8 packer bit for bit, and
bmm_mma_tile_opts with atom_k = 8 against the oracle's k = 8 product.

Cases take K a multiple of 8 but not of 16 (an odd number of k = 8 atoms, the
shapes the k = 16 layout cannot hold), with ragged M and N tails, on every
kernel. Where K is a multiple of 16 the two layouts hold the same 32 K values
in each hardware step, so the GPU results of the two must agree bit for bit
even on normal data.
"""
import numpy as np
import pytest
import torch

import bf16_matrix_multiply_amd as bmm
import oracle
import workloads
from tests import gpu_util as gu
from tests import util

pytestmark = pytest.mark.gpu

KERNELS = ["direct", "tiled", "skinny", "tiled128", "tiled256x128"]
C = workloads.custom

CASES = {
    "q_min_16x8x8": C(1, 16, 8, 8, "bf16", "quarter", "quarter", c_scalar=0.5),
    "q_odd_b2_48x40x88": C(2, 48, 40, 88, "f16", "quarter", "quarter", c_tensor=True),
    "q_tails_272x264x328": C(1, 272, 264, 328, "bf16", "quarter", "quarter", c_tensor=True),
    "q_skinny_16x1032x1048": C(1, 16, 1032, 1048, "f16", "quarter", "quarter"),
    "n_528x264x296_ct": C(1, 528, 264, 296, "bf16", c_tensor=True),
    "n_f16_b3_80x136x264": C(3, 80, 136, 264, "f16", c_tensor=True),
}


def run_k8(w, inp, kernel, alpha=None, beta=None):
    A = bmm.pack_operand(gu.dev_u16(inp["a"]), 16, atom_k=8)
    B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8, atom_k=8)
    Cd = None if inp["c_tensor"] is None else torch.from_numpy(inp["c_tensor"]).cuda()
    out = torch.full((w.batch, w.M_rep, w.N_rep, 16, 8), float("nan"), device="cuda")
    D = bmm.mma_tile(A, B, Cd, float(inp["c_scalar"]), w.dtype, out=out, kernel=kernel,
                     alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    return A, B, D.cpu().numpy()


@pytest.mark.parametrize("shape", [(1, 16, 8, 16), (2, 48, 40, 24), (1, 16, 104, 8),
                                   (1, 32, 16, 1032)])
def test_pack_k8_bits(shape):
    """Packed words equal the oracle's k = 8 packer, for A (R = 16) and B (R = 8),
    with a row pitch wider than K."""
    batch, rows16, rows8, K = shape
    rng = np.random.default_rng(3)
    for rows, R in ((rows16, 16), (rows8, 8)):
        x = util.random_bits(rng, (batch, rows, K + 8))
        got = bmm.pack_operand(gu.dev_u16(x), R, K=K, atom_k=8)
        assert tuple(got.shape) == (batch, rows // R, K // 8, R, 4)
        ref = oracle.pack_k8(np.ascontiguousarray(x[:, :, :K]), R)
        assert np.array_equal(gu.host_u32(got), ref)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", sorted(CASES))
def test_k8_parity(case, kernel):
    w = CASES[case]
    inp = workloads.make_inputs(w, seed=0)
    _, _, D = run_k8(w, inp, kernel)
    Ao, Bo = oracle.pack_k8(inp["a"], 16), oracle.pack_k8(inp["b"], 8)
    ref = oracle.mma_k8(Ao, Bo, inp["c_tensor"], inp["c_scalar"], w.dtype)
    assert not np.isnan(D).any()
    if w.exact:
        bad = np.argwhere(D != ref)
        assert bad.size == 0, f"{case}/{kernel}: {len(bad)} mismatches, first {bad[:4].tolist()}"
    else:
        # |A||B|^T + |C| from the logical operands (the k = 16 routine over
        # zero-padded K gives the same magnitudes)
        pad = (-w.K) % 16
        a16 = np.pad(inp["a"], ((0, 0), (0, 0), (0, pad)))
        b16 = np.pad(inp["b"], ((0, 0), (0, 0), (0, pad)))
        bnd = oracle.bound(oracle.pack(a16, 16), oracle.pack(b16, 8), inp["c_tensor"],
                           inp["c_scalar"], w.dtype).astype(np.float64)
        err = np.abs(D.astype(np.float64) - ref)
        assert (err <= gu.BOUND_SCALE * bnd).all(), \
            f"{case}/{kernel}: worst err/bound {float((err / (gu.BOUND_SCALE * bnd)).max())}"


@pytest.mark.parametrize("kernel", KERNELS)
def test_k8_equals_k16_bitwise(kernel):
    """Normal bf16 data, K a multiple of 16: the k = 8 and k = 16 layouts of the
    same operands give identical results."""
    w = C(1, 528, 264, 2064, "bf16", c_tensor=True)
    inp = workloads.make_inputs(w, seed=4)
    _, _, D8 = run_k8(w, inp, kernel)
    _, _, _, D16 = gu.gpu_run(w, inp, kernel)
    assert np.array_equal(D8, D16)


@pytest.mark.parametrize("kernel", KERNELS)
def test_k8_scaled(kernel):
    """alpha/beta form on k = 8 operands: quarter data with power-of-two
    alpha, beta is bit-exact against the oracle's alpha/beta form (K padded
    with zeros to the k = 16 layout, which adds exact zeros)."""
    w = C(2, 48, 40, 88, "bf16", "quarter", "quarter", c_tensor=True)
    inp = workloads.make_inputs(w, seed=2)
    _, _, D = run_k8(w, inp, kernel, alpha=0.5, beta=-2.0)
    a16 = np.pad(inp["a"], ((0, 0), (0, 0), (0, 8)))
    b16 = np.pad(inp["b"], ((0, 0), (0, 0), (0, 8)))
    ref = oracle.mma_scaled(oracle.pack(a16, 16), oracle.pack(b16, 8), inp["c_tensor"], 0.0,
                            0.5, -2.0, "bf16")
    assert np.array_equal(D, ref)


@pytest.mark.parametrize("name", ["gemm_8192_bf16_ctensor", "skinny_16x16384x16384_bf16"])
def test_k8_full_size_sampled(name):
    """The large bf16 shapes in the k = 8 layout: sampled outputs against the
    oracle's k = 8 product, within the normal-data bound."""
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w, seed=0)
    _, _, D = run_k8(w, inp, "auto")
    Ao, Bo = oracle.pack_k8(inp["a"], 16), oracle.pack_k8(inp["b"], 8)
    idx = util.sample_indices(np.random.default_rng(9), w.batch, w.M, w.N, 1024)
    ref = oracle.mma_k8_sampled(Ao, Bo, inp["c_tensor"], inp["c_scalar"], w.dtype, idx)
    bnd = oracle.bound(oracle.pack(inp["a"], 16), oracle.pack(inp["b"], 8), inp["c_tensor"],
                       inp["c_scalar"], w.dtype, idx).astype(np.float64)
    Dl = util.tile_to_logical(D)
    assert not np.isnan(Dl).any()
    got = Dl[idx[:, 0], idx[:, 1], idx[:, 2]].astype(np.float64)
    assert (np.abs(got - ref) <= gu.BOUND_SCALE * bnd).all()
