"""GPU parity of the store direction of the box transfer (bmm_box_store,
bmm_box_reduce_add) and of the split-K form (bmm_mma_tile_splitk) against
the oracle.

Box stores and integer / float adds move or combine individual elements with
one rounding each, so they must match the oracle bit for bit. Split-K sums
each 32-value step in the MFMA's own order, so, as for the plain product,
quarter-integer data must be bit-exact and normal data within
1e-3 (|A||B|^T + |C|).
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

C = workloads.custom

# (dtype, shape, box, coords, n_repeat, coord_step): partly outside boxes,
# repeats that overlap (launched one after another) and that do not; outer
# byte strides are multiples of 16 as the boundary requires
STORE_CASES = [
    (np.uint32, (16, 16), (8, 16), (-3, 5), 3, (6, -4)),
    (np.uint16, (5, 7, 16), (4, 4, 8), (3, -2, 12), 2, (-4, 3, 1)),
    (np.uint8, (37,), (32,), (20,), 2, (-25,)),
    (np.uint64, (9, 12), (3, 5), (0, 0), 4, (1, 2)),
    (np.uint32, (8, 8), (4, 4), (2, 2), 3, (0, 0)),
    (np.uint32, (64, 256), (64, 256), (0, 0), 1, (0, 0)),   # a 64 KB image
]


def _dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint64:
        return torch.from_numpy(x.view(np.int64)).cuda()
    if x.dtype == np.uint32:
        return torch.from_numpy(x.view(np.int32)).cuda()
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda()
    if x.dtype == np.uint8:
        return torch.from_numpy(x).cuda()
    return torch.from_numpy(x).cuda()


def _host(t, dtype):
    return t.cpu().numpy().view(dtype)


@pytest.mark.parametrize("swizzle", [0, 3])
@pytest.mark.parametrize("case", range(len(STORE_CASES)))
def test_box_store(case, swizzle):
    dtype, shape, box, coords, rep, step = STORE_CASES[case]
    rng = np.random.default_rng(20 + case)
    G = rng.integers(1, 200, shape).astype(dtype)
    img = rng.integers(1, 200, (rep, *box)).astype(dtype)
    Gd = _dev(G)
    nbytes = bmm.box_store(Gd, _dev(img), box, coords, rep, step, swizzle=swizzle)
    ref, ref_bytes = oracle.box_store(G, img, box, coords, rep, step)
    assert np.array_equal(_host(Gd, dtype), ref)
    assert nbytes == ref_bytes


# 16-byte-path descriptors: partly outside in every dimension; the last two
# have overlapping repeats (launched one after another)
CHUNK_STORE_CASES = [
    (np.uint32, (20, 48), (8, 16), (-4, -8), 4, (6, 12)),
    (np.uint16, (6, 5, 40), (3, 4, 16), (4, -2, -8), 3, (-2, 3, 24)),
    (np.uint8, (3, 80), (2, 48), (1, -16), 3, (1, 48)),
    (np.uint64, (9, 12), (3, 4), (-1, -2), 3, (4, 6)),
    (np.uint32, (16, 64), (8, 32), (2, 8), 3, (1, 4)),
    (np.uint16, (12, 64), (4, 32), (-1, 8), 4, (2, -8)),
    # 64 KiB boxes (the limit), partly outside, the second overlapping its neighbours
    (np.uint32, (300, 300), (64, 256), (-16, 64), 3, (100, 16)),
    (np.uint16, (130, 520), (128, 256), (-4, 8), 3, (2, 136)),
]


def chunk_path(itemsize, shape, box, coords, step):
    """Whether the library takes its 16-byte box path for this descriptor."""
    return all((v * itemsize) % 16 == 0 for v in (box[-1], coords[-1], step[-1], shape[-1]))


@pytest.mark.parametrize("swizzle", [0, 2])
@pytest.mark.parametrize("case", range(len(CHUNK_STORE_CASES)))
def test_box_store_chunk_path(case, swizzle):
    dtype, shape, box, coords, rep, step = CHUNK_STORE_CASES[case]
    assert chunk_path(np.dtype(dtype).itemsize, shape, box, coords, step)
    rng = np.random.default_rng(50 + case)
    G = rng.integers(1, 200, shape).astype(dtype)
    img = rng.integers(1, 200, (rep, *box)).astype(dtype)
    Gd = _dev(G)
    nbytes = bmm.box_store(Gd, _dev(img), box, coords, rep, step, swizzle=swizzle)
    ref, ref_bytes = oracle.box_store(G, img, box, coords, rep, step)
    assert np.array_equal(_host(Gd, dtype), ref)
    assert nbytes == ref_bytes


@pytest.mark.parametrize("etype", ["f32", "f16", "bf16", "i32", "i64"])
@pytest.mark.parametrize("overlap", [False, True])
def test_box_reduce_add_chunk_path(etype, overlap):
    """The 16-byte add path on random finite operands (ties, subnormals,
    overflow to inf for 16-bit types; wrap-around for integers), partly outside
    in both dimensions; with overlap, repeats add into the same elements in
    order."""
    rng = np.random.default_rng(77)
    eb = {"f32": 4, "f16": 2, "bf16": 2, "i32": 4, "i64": 8}[etype]
    shape, box, coords = (40, 64), (16, 32), (30, -16)
    rep, step = (3, (1, 16)) if overlap else (2, (16, 48))
    assert chunk_path(eb, shape, box, coords, step)
    if etype == "f32":
        G = (rng.standard_normal(shape) * 1e3).astype(np.float32)
        img = rng.standard_normal((rep, *box)).astype(np.float32)
    elif etype in ("f16", "bf16"):
        G, img = _finite_bits(rng, shape, etype), _finite_bits(rng, (rep, *box), etype)
    else:
        it = np.int32 if etype == "i32" else np.int64
        info = np.iinfo(it)
        G = rng.integers(info.min, info.max, shape, dtype=it)
        img = rng.integers(info.min, info.max, (rep, *box), dtype=it)
    Gd = _dev(G)
    bmm.box_reduce_add(Gd, _dev(img), box, coords, etype, rep, step, swizzle=1)
    ref, _ = oracle.box_store(G, img, box, coords, rep, step, op="add", elem_type=etype)
    got = _host(Gd, G.dtype)
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), etype


def _finite_bits(rng, shape, dt):
    bits = rng.integers(0, 1 << 16, shape, dtype=np.uint32).astype(np.uint16)
    ones = 0x7C00 if dt == "f16" else 0x7F80
    return np.where((bits & ones) == ones, bits & ~np.uint16(0x4000), bits)


@pytest.mark.parametrize("etype", ["f32", "f16", "bf16", "i32", "i64"])
@pytest.mark.parametrize("overlap", [False, True])
def test_box_reduce_add(etype, overlap):
    """Random finite operands (ties, subnormals, overflow to inf for the
    16-bit types; wrap-around for integers), partly outside boxes; with
    overlap, three repeats hit the same elements and are added in order."""
    rng = np.random.default_rng(31)
    shape, box, coords = (40, 72), (16, 32), (30, 50)
    rep, step = (3, (1, 2)) if overlap else (2, (16, -32))
    if etype == "f32":
        G = (rng.standard_normal(shape) * 1e3).astype(np.float32)
        img = rng.standard_normal((rep, *box)).astype(np.float32)
    elif etype in ("f16", "bf16"):
        G, img = _finite_bits(rng, shape, etype), _finite_bits(rng, (rep, *box), etype)
    else:
        it = np.int32 if etype == "i32" else np.int64
        info = np.iinfo(it)
        G = rng.integers(info.min, info.max, shape, dtype=it)
        img = rng.integers(info.min, info.max, (rep, *box), dtype=it)
    Gd = _dev(G)
    bmm.box_reduce_add(Gd, _dev(img), box, coords, etype, rep, step, swizzle=2)
    ref, _ = oracle.box_store(G, img, box, coords, rep, step, op="add", elem_type=etype)
    got = _host(Gd, G.dtype)
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), etype


def test_box_reduce_add_tie_order():
    """1 + 2^-24 + 2^-24 added one repeat at a time stays 1."""
    G = torch.ones((4, 4), device="cuda")
    img = torch.full((2, 4, 4), 2.0 ** -24, device="cuda")
    bmm.box_reduce_add(G, img, (4, 4), (0, 0), "f32", 2, (0, 0))
    assert (G == 1.0).all()


# ---- split-K ----

SPLIT_CASES = {
    # quarter-integer data: bit-exact against the oracle's split-K form
    "q_272x264x1040_ct": C(1, 272, 264, 1040, "bf16", "quarter", "quarter", c_tensor=True),
    "q_f16_b2_48x40x4112_scalar": C(2, 48, 40, 4112, "f16", "quarter", "quarter", c_scalar=1.25),
    # K = 16384, where the split-K form switches to 256 x 256 tiles; ragged M and N
    "q_272x264x16384_ct": C(1, 272, 264, 16384, "bf16", "quarter", "quarter", c_tensor=True),
    # normal data: within bound
    "n_528x264x8208_ct": C(1, 528, 264, 8208, "bf16", c_tensor=True),
}


def _split_inputs(w, atom_k=16):
    inp = workloads.make_inputs(w, seed=0)
    A = bmm.pack_operand(gu.dev_u16(inp["a"]), 16, atom_k=atom_k)
    B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8, atom_k=atom_k)
    Cd = None if inp["c_tensor"] is None else torch.from_numpy(inp["c_tensor"]).cuda()
    if atom_k == 16:
        Ao, Bo = oracle.pack(inp["a"], 16), oracle.pack(inp["b"], 8)
    else:
        Ao, Bo = oracle.pack_k8(inp["a"], 16), oracle.pack_k8(inp["b"], 8)
    return inp, A, B, Cd, Ao, Bo


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 1000])
@pytest.mark.parametrize("case", sorted(SPLIT_CASES))
def test_splitk_parity(case, splits):
    w = SPLIT_CASES[case]
    inp, A, B, Cd, Ao, Bo = _split_inputs(w)
    out = torch.full((w.batch, w.M_rep, w.N_rep, 16, 8), float("nan"), device="cuda")
    D = bmm.mma_tile_splitk(A, B, Cd, float(inp["c_scalar"]), w.dtype, splits, out=out)
    D = D.cpu().numpy()
    ref = oracle.mma_splitk(Ao, Bo, inp["c_tensor"], inp["c_scalar"], w.dtype, splits)
    assert not np.isnan(D).any()
    if w.exact:
        bad = np.argwhere(D != ref)
        assert bad.size == 0, f"{case}/S={splits}: {len(bad)} mismatches, first {bad[:4].tolist()}"
    else:
        bnd = oracle.bound(Ao, Bo, inp["c_tensor"], inp["c_scalar"], w.dtype).astype(np.float64)
        err = np.abs(D.astype(np.float64) - ref)
        assert (err <= gu.BOUND_SCALE * bnd).all(), \
            f"{case}/S={splits}: worst err/bound {float((err / (gu.BOUND_SCALE * bnd)).max())}"


def test_splitk_k8_in_place_and_deterministic():
    """k = 8 operands with an odd atom count, D == C in place: equal to the
    out-of-place result and to the oracle (quarter data, bit-exact); two runs
    give identical bits."""
    w = C(1, 272, 136, 1032, "bf16", "quarter", "quarter", c_tensor=True)
    inp, A, B, Cd, Ao, Bo = _split_inputs(w, atom_k=8)
    D1 = bmm.mma_tile_splitk(A, B, Cd, 0.0, "bf16", 5)
    D2 = bmm.mma_tile_splitk(A, B, Cd, 0.0, "bf16", 5)
    assert torch.equal(D1, D2)
    ref = oracle.mma_splitk(Ao, Bo, inp["c_tensor"], 0.0, "bf16", 5)
    assert np.array_equal(D1.cpu().numpy(), ref)
    bmm.mma_tile_splitk(A, B, Cd, 0.0, "bf16", 5, out=Cd)
    assert torch.equal(Cd, D1)


def test_splitk_k_zero_copies_c():
    Cn = np.random.default_rng(3).standard_normal((1, 2, 3, 16, 8)).astype(np.float32)
    Cn[0, 0, 0, 0, :3] = -0.0
    A = torch.zeros((1, 2, 0, 16, 8), dtype=torch.int32, device="cuda")
    B = torch.zeros((1, 3, 0, 8, 8), dtype=torch.int32, device="cuda")
    D = bmm.mma_tile_splitk(A, B, torch.from_numpy(Cn).cuda(), 0.0, "bf16", 4)
    assert np.array_equal(D.cpu().numpy().view(np.uint32), Cn.view(np.uint32))


def test_splitk_deep_k_sampled():
    """1024 x 1024 x 65536 bf16 (16 output tiles, 16 splits by default):
    sampled outputs against the oracle's split-K form within bound, and the
    plain tiled kernel's result within twice the bound."""
    w = C(1, 1024, 1024, 65536, "bf16", c_tensor=True, name="deep_k")
    inp, A, B, Cd, Ao, Bo = _split_inputs(w)
    S = bmm.splitk_default(1, w.M_rep, w.N_rep, w.K_rep)
    assert S == 16
    D = util.tile_to_logical(bmm.mma_tile_splitk(A, B, Cd, 0.0, "bf16").cpu().numpy())
    D0 = util.tile_to_logical(bmm.mma_tile(A, B, Cd, 0.0, "bf16", kernel="tiled").cpu().numpy())
    idx = util.sample_indices(np.random.default_rng(8), 1, w.M, w.N, 512)
    ref = oracle.mma_splitk_sampled(Ao, Bo, inp["c_tensor"], 0.0, "bf16", S, idx)
    bnd = oracle.bound(Ao, Bo, inp["c_tensor"], 0.0, "bf16", idx).astype(np.float64)
    got = D[idx[:, 0], idx[:, 1], idx[:, 2]].astype(np.float64)
    assert (np.abs(got - ref) <= gu.BOUND_SCALE * bnd).all()
    got0 = D0[idx[:, 0], idx[:, 1], idx[:, 2]].astype(np.float64)
    assert (np.abs(got - got0) <= 2 * gu.BOUND_SCALE * bnd).all()


@pytest.mark.parametrize("splits", [2, 5])
def test_splitk_reduce_is_the_box_add(splits):
    """The split-K reduce is the box add reduction fused over the partials:
    starting from C and applying bmm_box_reduce_add (float32, one rounding per
    add) to each partial left in the workspace, in split order, gives the
    split-K result bit for bit (normal data)."""
    w = C(1, 512, 512, 4096, "bf16", c_tensor=True, name="splitk_box_add")
    inp = workloads.make_inputs(w, seed=8)
    A = bmm.pack_operand(gu.dev_u16(inp["a"]), 16)
    B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8)
    Cd = torch.from_numpy(inp["c_tensor"]).cuda()
    ws_bytes = bmm.splitk_workspace_bytes(1, w.M_rep, w.N_rep, w.K_rep, 16, splits)
    n = w.M * w.N
    assert ws_bytes == splits * n * 4
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    D = bmm.mma_tile_splitk(A, B, Cd, 0.0, "bf16", splits, workspace=ws)
    rows = n // 256
    D2 = Cd.clone().view(rows, 256)
    for s in range(splits):
        part = ws[s * n:(s + 1) * n].view(rows // 64, 64, 256)
        bmm.box_reduce_add(D2, part, (64, 256), (0, 0), "f32", rows // 64, (64, 0))
    torch.cuda.synchronize()
    got, ref = D.cpu().numpy().reshape(-1), D2.cpu().numpy().reshape(-1)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    gu.assert_parity_full(w, inp, D.cpu().numpy(), f"splitk{splits}")
