"""GPU parity of bmm_mma_tile against the oracle.

Quarter-integer inputs (every product and partial sum exact in fp32) must be
bit-exact; normal inputs must satisfy |D - D_ref| <= 1e-3 (|A||B|^T + |C|)
elementwise. Every kernel accepts every valid shape, so each is forced on the
same cases, which span several 256-wide tiles and ragged tails in M, N and K.
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
SMALL = {
    # the worked example and the 128x128x256 workload as given
    "tile_16x8x32_f16": workloads.WORKLOADS["tile_16x8x32_f16"],
    "gemm_128x128x256_bf16_ctensor": workloads.WORKLOADS["gemm_128x128x256_bf16_ctensor"],
    # quarter-integer (bit-exact) cases with ragged extents
    "q_min_1x1x1": C(1, 16, 8, 16, "bf16", "quarter", "quarter", c_scalar=0.25),
    "q_odd_b2": C(2, 48, 40, 80, "f16", "quarter", "quarter", c_tensor=True),
    "q_tails_272x264x336": C(1, 272, 264, 336, "bf16", "quarter", "quarter", c_tensor=True),
    "q_skinny_16x1032x1040": C(1, 16, 1032, 1040, "f16", "quarter", "quarter"),
    "q_tall_528x24x48": C(1, 528, 24, 48, "bf16", "quarter", "quarter", c_tensor=True),
    # normal-input cases
    "n_512x512x512_ct": C(1, 512, 512, 512, "bf16", c_tensor=True),
    "n_f16_b3_80x136x272": C(3, 80, 136, 272, "f16", c_tensor=True),
    "n_skinny_64x520x2064": C(1, 64, 520, 2064, "bf16", b_scale=0.02),
    "n_kodd_32x256x16": C(1, 32, 256, 16, "bf16", c_tensor=True),
}


def inputs(w):
    return workloads.make_inputs(w, seed=0)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", sorted(SMALL))
def test_small_full_parity(case, kernel):
    w = SMALL[case]
    inp = inputs(w)
    _, _, _, D = gu.gpu_run(w, inp, kernel)
    gu.assert_parity_full(w, inp, D, kernel)


def test_page_example_exact():
    """The worked 16x8 example: equal to a.f32 @ b.f32.T bit for bit."""
    w = workloads.WORKLOADS["tile_16x8x32_f16"]
    inp = inputs(w)
    _, _, _, D = gu.gpu_run(w, inp)
    a = inp["a"][0].view(np.float16).astype(np.float32)
    b = inp["b"][0].view(np.float16).astype(np.float32)
    assert np.array_equal(util.tile_to_logical(D)[0], a @ b.T)


def test_fragment_map_one_hot():
    """One-hot probes through the real path: with A[m0, k0] = 1 and
    B[n0, k0] = 1 only, D is 1 at (m0, n0) and 0 elsewhere, for every (m0, n0)
    of a 16x16 block (batched) and k0 in each lane group of a 32-deep step."""
    for k0 in (0, 9, 18, 31):
        batch = 16 * 16
        a = np.zeros((batch, 16, 32), np.float32)
        b = np.zeros((batch, 16, 32), np.float32)
        for bi in range(batch):
            a[bi, bi // 16, k0] = 1.0
            b[bi, bi % 16, k0] = 1.0
        A = bmm.pack_operand(gu.dev_u16(workloads.f32_to_bf16_bits(a)), 16)
        B = bmm.pack_operand(gu.dev_u16(workloads.f32_to_bf16_bits(b)), 8)
        for kernel in KERNELS:
            D = util.tile_to_logical(bmm.mma_tile(A, B, None, 0.0, "bf16", kernel=kernel).cpu().numpy())
            ref = np.zeros((batch, 16, 16), np.float32)
            for bi in range(batch):
                ref[bi, bi // 16, bi % 16] = 1.0
            assert np.array_equal(D, ref), (k0, kernel)


@pytest.mark.parametrize("kernel", KERNELS)
def test_scalar_equals_filled_tensor(kernel):
    w = C(1, 96, 200, 208, "bf16")
    inp = inputs(w)
    A, B, _, D1 = gu.gpu_run(w, dict(inp, c_scalar=np.float32(0.375)), kernel)
    Cf = torch.full((1, w.M_rep, w.N_rep, 16, 8), 0.375, device="cuda")
    D2 = bmm.mma_tile(A, B, Cf, 0.0, "bf16", kernel=kernel).cpu().numpy()
    assert np.array_equal(D1, D2)


@pytest.mark.parametrize("kernel", KERNELS)
def test_in_place_and_k_chaining(kernel):
    """D == C in place, and the recurrence split over two calls (C -> D -> D):
    bit-exact against one call on quarter-integer inputs."""
    w = C(2, 272, 136, 336, "f16", "quarter", "quarter", c_tensor=True)
    inp = inputs(w)
    A, B, Cd, D = gu.gpu_run(w, inp, kernel)
    gu.assert_parity_full(w, inp, D, kernel)
    Dip = Cd.clone()
    bmm.mma_tile(A, B, Dip, 0.0, w.dtype, out=Dip, kernel=kernel)
    assert np.array_equal(Dip.cpu().numpy(), D)
    cut = 7
    Dc = Cd.clone()
    bmm.mma_tile(A[:, :, :cut].contiguous(), B[:, :, :cut].contiguous(), Dc, 0.0, w.dtype,
                 out=Dc, kernel=kernel)
    bmm.mma_tile(A[:, :, cut:].contiguous(), B[:, :, cut:].contiguous(), Dc, 0.0, w.dtype,
                 out=Dc, kernel=kernel)
    assert np.array_equal(Dc.cpu().numpy(), D)


@pytest.mark.parametrize("kernel", KERNELS)
def test_k_rep_zero_and_zero_a(kernel):
    """K_rep = 0 gives D = C; A = 0 gives D = C bitwise."""
    w = C(1, 64, 64, 64, "bf16", c_tensor=True)
    inp = inputs(w)
    Cd = torch.from_numpy(inp["c_tensor"]).cuda()
    A0 = torch.zeros((1, 4, 0, 16, 8), dtype=torch.int32, device="cuda")
    B0 = torch.zeros((1, 8, 0, 8, 8), dtype=torch.int32, device="cuda")
    D = bmm.mma_tile(A0, B0, Cd, 0.0, "bf16", kernel=kernel)
    assert np.array_equal(D.cpu().numpy(), inp["c_tensor"])
    Az = torch.zeros((1, 4, 4, 16, 8), dtype=torch.int32, device="cuda")
    B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8)
    D = bmm.mma_tile(Az, B, Cd, 0.0, "bf16", kernel=kernel)
    assert np.array_equal(D.cpu().numpy(), inp["c_tensor"])


@pytest.mark.parametrize("kernel", KERNELS)
def test_deterministic_and_stream(kernel):
    """Two runs give identical bits, also on a non-default stream."""
    w = C(1, 256, 264, 1040, "bf16", c_tensor=True)
    inp = inputs(w)
    A, B, Cd, D1 = gu.gpu_run(w, inp, kernel)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        D2 = bmm.mma_tile(A, B, Cd, 0.0, "bf16", kernel=kernel)
    s.synchronize()
    assert np.array_equal(D1, D2.cpu().numpy())


def test_errors_write_nothing():
    """Host-side rejections launch nothing: the output keeps its contents."""
    w = C(1, 32, 32, 32, "bf16")
    inp = inputs(w)
    A = bmm.pack_operand(gu.dev_u16(inp["a"]), 16)
    B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8)
    out = torch.full((1, 2, 4, 16, 8), -5.0, device="cuda")
    L = bmm.lib()
    d, a, b = out.data_ptr(), A.data_ptr(), B.data_ptr()
    assert L.bmm_mma_tile(d, a, b, d + 16, 0.0, 1, 2, 4, 2, 1, None) == -3
    assert "partially overlaps C" in L.bmm_last_error().decode()
    assert L.bmm_mma_tile(d, a, b, None, 0.0, 1, 2, 4, 2, 7, None) == -1
    assert L.bmm_mma_tile(d + 4, a, b, None, 0.0, 1, 2, 4, 2, 1, None) == -2
    with pytest.raises(ValueError):
        bmm.mma_tile(A, B[:, :, :1], None, 0.0, "bf16", out=out)
    torch.cuda.synchronize()
    assert (out == -5.0).all()


# ---- full-size workloads, checked on sampled outputs and exact properties ----

def test_full_gemm_4096_f16_quarter():
    """4096^3 f16 quarter integers: sampled outputs bit-exact, and every row
    and column sum of 16*D equal to its int64 closed form."""
    w = workloads.WORKLOADS["gemm_4096_f16_quarter"]
    inp = inputs(w)
    _, _, _, D = gu.gpu_run(w, inp)
    gu.assert_parity_sampled(w, inp, D)
    Dl = util.tile_to_logical(D)[0].astype(np.float64)
    D16 = np.rint(Dl * 16).astype(np.int64)
    assert np.array_equal(D16.astype(np.float64), Dl * 16)
    ai = np.rint(4 * util.decode(inp["a"][0], "f16")).astype(np.int64)
    bi = np.rint(4 * util.decode(inp["b"][0], "f16")).astype(np.int64)
    assert np.array_equal(D16.sum(axis=1), ai @ bi.sum(axis=0))
    assert np.array_equal(D16.sum(axis=0), bi @ ai.sum(axis=0))


def test_full_skinny_bf16():
    """16 x 16384 x 16384: outputs sampled in every 16 x 64 column block of the
    skinny kernel (one workgroup's share), within bound."""
    w = workloads.WORKLOADS["skinny_16x16384x16384_bf16"]
    inp = inputs(w)
    _, _, _, D = gu.gpu_run(w, inp)
    gu.assert_parity_sampled(w, inp, D, idx=gu.per_tile_indices(w, 16, 64, per_tile=2))


def test_full_gemm_8192_bf16_ctensor():
    """8192^3 with the C tensor: two outputs sampled in every 256 x 256 macro
    tile (all 1024 tiles, so every workgroup slot on every XCD), within bound."""
    w = workloads.WORKLOADS["gemm_8192_bf16_ctensor"]
    inp = inputs(w)
    _, _, _, D = gu.gpu_run(w, inp)
    gu.assert_parity_sampled(w, inp, D, idx=gu.per_tile_indices(w, 256, 256, per_tile=2))


@pytest.mark.parametrize("name", ["shard_n8_8192x1024x8192_bf16_ctensor",
                                  "shard_m8_1024x8192x8192_bf16_ctensor"])
def test_full_shard_256x128_sampled(name):
    """One GPU's share of an 8-way split of the 8192^3 workload, at its real
    shape: AUTO runs the 256 x 128 tile there (256 tiles), sampled outputs
    within bound."""
    w = workloads.EXTRA_WORKLOADS[name]
    assert bmm.select_kernel(w.batch, w.M_rep, w.N_rep, w.K_rep) == "tiled256x128"
    inp = workloads.make_inputs(w, seed=0)
    _, _, _, D = gu.gpu_run(w, inp)
    gu.assert_parity_sampled(w, inp, D, idx=gu.per_tile_indices(w, 256, 128, per_tile=2))


@pytest.mark.parametrize("name", ["shard_n8_8192x1024x8192_bf16_ctensor",
                                  "shard_m8_1024x8192x8192_bf16_ctensor"])
def test_full_shard_256x128_quarter_sums(name):
    """The shard shapes on the 256 x 128 tile with quarter-integer operands and
    C on the quarter grid: every row and column sum of 16*D equals its int64
    closed form, so every output is checked."""
    base = workloads.EXTRA_WORKLOADS[name]
    w = C(1, base.M, base.N, base.K, "bf16", "quarter", "quarter", c_tensor=True,
          name=name + "_quarter")
    inp = workloads.make_inputs(w, seed=4)
    _, _, _, D = gu.gpu_run(w, inp, "tiled256x128")
    gu.assert_quarter_sums(w, inp, D)


@pytest.mark.parametrize("name", ["skinny_16x16384x16384_bf16", "gemm_8192_bf16_ctensor"])
def test_full_quantised_variants(name):
    """The large bf16 shapes with quarter-integer operands and C on the
    quarter grid (|D| <= 16 + K on a 1/16 grid: at most 19 bits, exact): every
    row and column sum of 16*D equals its int64 closed form, and samples in
    every macro tile are bit-exact against the oracle."""
    base = workloads.WORKLOADS[name]
    w = C(base.batch, base.M, base.N, base.K, "bf16", "quarter", "quarter",
          c_tensor=True, name=name + "_quarter")
    inp = workloads.make_inputs(w, seed=1)
    _, _, _, D = gu.gpu_run(w, inp)
    gu.assert_quarter_sums(w, inp, D)
    tm, tn = (256, 256) if w.M >= 256 else (16, 64)
    gu.assert_parity_sampled(w, inp, D, idx=gu.per_tile_indices(w, tm, tn, per_tile=1))


def test_largest_k_of_the_tiled_kernels():
    """The tiled kernels take K < 2^22 values, where one tile's buffer offsets
    reach 2 GB. At K = 2^22 - 4096 with one full 256 x 256 tile, ternary
    operands and C on the quarter grid (every partial sum exact), the three
    tile shapes and the split-K form give the same bits, outputs sampled over
    the tile equal the oracle's, and every row and column sum of 16*D equals
    its int64 closed form."""
    K = (1 << 22) - 4096
    w = C(1, 256, 256, K, "bf16", "ternary", "ternary", c_tensor=True, name="largest_k")
    inp = workloads.make_inputs(w, seed=5)
    print(f"[largest_k] {w.M}x{w.N}x{w.K}", flush=True)
    a, b = gu.dev_u16(inp["a"]), gu.dev_u16(inp["b"])
    A, B = bmm.pack_operand(a, 16), bmm.pack_operand(b, 8)
    del a, b
    Cd = torch.from_numpy(inp["c_tensor"]).cuda()
    shape = (1, w.M_rep, w.N_rep, 16, 8)
    outs = {}
    for k in ("tiled", "tiled256x128", "tiled128"):
        out = torch.full(shape, float("nan"), device="cuda")
        outs[k] = bmm.mma_tile(A, B, Cd, 0.0, "bf16", out=out, kernel=k).cpu().numpy()
    out = torch.full(shape, float("nan"), device="cuda")
    outs["splitk4"] = bmm.mma_tile_splitk(A, B, Cd, 0.0, "bf16", 4, out=out).cpu().numpy()
    del A, B
    torch.cuda.empty_cache()
    ref = outs["tiled"]
    for k, D in outs.items():
        assert np.array_equal(D.view(np.uint32), ref.view(np.uint32)), k
    gu.assert_quarter_sums(w, inp, ref)
    gu.assert_parity_sampled(w, inp, ref, idx=gu.per_tile_indices(w, 32, 32, per_tile=1))


def test_ragged_many_tiles_all_tile_shapes():
    """Two batches of 1232 x 1256 x 1040 (ragged in M, N and K: 5 x 5 tiles of
    256 x 256 per batch, the last ones partial, and an odd K_rep), quarter
    integers with C on the quarter grid: the three tile shapes give the same
    bits, every row and column sum of 16*D equals its int64 closed form, and
    outputs sampled in every 32 x 32 block equal the oracle's."""
    w = C(2, 1232, 1256, 1040, "bf16", "quarter", "quarter", c_tensor=True, name="ragged_tiles")
    inp = workloads.make_inputs(w, seed=8)
    print(f"[ragged_tiles] {w.batch}x{w.M}x{w.N}x{w.K}", flush=True)
    outs = {k: gu.gpu_run(w, inp, k)[3] for k in ("tiled", "tiled256x128", "tiled128")}
    ref = outs["tiled"]
    for k, D in outs.items():
        assert np.array_equal(D.view(np.uint32), ref.view(np.uint32)), k
    gu.assert_quarter_sums(w, inp, ref)
    gu.assert_parity_sampled(w, inp, ref, idx=gu.per_tile_indices(w, 32, 32, per_tile=1))


@pytest.mark.parametrize("shape,kernel", [((2048, 2048, 2048), "auto"),
                                          ((2560, 1536, 4096), "tiled128"),
                                          ((4096, 4096, 4096), "tiled128")])
def test_mid_size_tiled128_sampled(shape, kernel):
    """Mid-size shapes on the 128 x 128 tile (AUTO's pick at 2048^3): normal
    bf16 data with a C tensor, sampled outputs within bound, and the same
    shape with quarter-integer f16 data bit-exact on its samples."""
    M, N, K = shape
    if kernel == "auto":
        assert bmm.select_kernel(1, M // 16, N // 8, K // 16) == "tiled128"
    w = C(1, M, N, K, "bf16", c_tensor=True, name=f"mid_{M}x{N}x{K}")
    inp = inputs(w)
    _, _, _, D = gu.gpu_run(w, inp, kernel)
    gu.assert_parity_sampled(w, inp, D)
    wq = C(1, M, N, K, "f16", "quarter", "quarter", c_tensor=True, name=f"mid_q_{M}x{N}x{K}")
    inpq = workloads.make_inputs(wq, seed=3)
    _, _, _, Dq = gu.gpu_run(wq, inpq, kernel)
    gu.assert_parity_sampled(wq, inpq, Dq)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_tile_shapes_bitwise(dtype):
    """Normal data, ragged M and N, an odd K_rep: the 256 x 256, 256 x 128 and
    128 x 128 tiles each start every output's accumulator at C and then add
    the products of each 32-deep K step in ascending K (one 16x16x32 MFMA, or
    two 32x32x16 half steps), so the three agree bit for bit. The split-K form with a single split forms the partial sum
    from zero and then adds C once, so it gives fl(C + P) with P the product
    that either tile gives for a scalar C of 0."""
    w = C(1, 528, 264, 2064, dtype, c_tensor=True, name=f"tiles_{dtype}")
    inp = workloads.make_inputs(w, seed=6)
    A, B, Cd, D256 = gu.gpu_run(w, inp, "tiled")
    _, _, _, D128 = gu.gpu_run(w, inp, "tiled128")
    _, _, _, D2561 = gu.gpu_run(w, inp, "tiled256x128")
    assert np.array_equal(D256.view(np.uint32), D128.view(np.uint32))
    assert np.array_equal(D256.view(np.uint32), D2561.view(np.uint32))
    gu.assert_parity_full(w, inp, D256, "tiled")
    P = {k: bmm.mma_tile(A, B, None, 0.0, dtype, kernel=k).cpu().numpy()
         for k in ("tiled", "tiled128")}
    assert np.array_equal(P["tiled"].view(np.uint32), P["tiled128"].view(np.uint32))
    out = torch.full(D256.shape, float("nan"), device="cuda")
    D1 = bmm.mma_tile_splitk(A, B, Cd, 0.0, dtype, 1, out=out).cpu().numpy()
    ref1 = inp["c_tensor"] + P["tiled"]
    assert ref1.dtype == np.float32
    assert np.array_equal(D1.view(np.uint32), ref1.view(np.uint32))


# ---- alpha/beta form (bmm_mma_tile_scaled) ----

SCALED = {
    "q_272x264x336_ct": C(1, 272, 264, 336, "bf16", "quarter", "quarter", c_tensor=True),
    "q_f16_b2_48x40x80_scalar": C(2, 48, 40, 80, "f16", "quarter", "quarter", c_scalar=1.25),
    "q_16x1032x1040_ct": C(1, 16, 1032, 1040, "bf16", "quarter", "quarter", c_tensor=True),
    "n_512x520x528_ct": C(1, 512, 520, 528, "bf16", c_tensor=True),
}


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", sorted(SCALED))
def test_scaled_parity(case, kernel):
    """Quarter-integer data with power-of-two alpha, beta: bit-exact against
    the oracle's alpha/beta form; normal data within
    1e-3 (|alpha||A||B|^T + |beta||C|)."""
    w = SCALED[case]
    inp = inputs(w)
    A = bmm.pack_operand(gu.dev_u16(inp["a"]), 16)
    B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8)
    Cd = None if inp["c_tensor"] is None else torch.from_numpy(inp["c_tensor"]).cuda()
    alpha, beta = (0.5, -2.0) if w.exact else (0.7, -1.3)
    out = torch.full((w.batch, w.M_rep, w.N_rep, 16, 8), float("nan"), device="cuda")
    D = bmm.mma_tile(A, B, Cd, float(inp["c_scalar"]), w.dtype, out=out, kernel=kernel,
                     alpha=alpha, beta=beta).cpu().numpy()
    Ao, Bo = gu.oracle_operands(w, inp)
    ref = oracle.mma_scaled(Ao, Bo, inp["c_tensor"], inp["c_scalar"], alpha, beta, w.dtype)
    assert not np.isnan(D).any()
    if w.exact:
        assert np.array_equal(D, ref)
    else:
        prod = oracle.bound(Ao, Bo, None, 0.0, w.dtype)          # |A||B|^T
        cmag = np.abs(inp["c_tensor"]) if inp["c_tensor"] is not None else abs(inp["c_scalar"])
        bnd = abs(alpha) * prod.astype(np.float64) + abs(beta) * cmag
        assert (np.abs(D.astype(np.float64) - ref) <= 1e-3 * bnd).all()


@pytest.mark.parametrize("kernel", KERNELS)
def test_scaled_single_rounding(kernel):
    """The final alpha*acc + beta*C is one fused operation: for acc = 1+2^-23,
    alpha = 1+2^-23, beta*C = -(1+2^-22) the result is 2^-46 (a rounded
    multiply followed by an add would give 0)."""
    from tests import pins
    A, B, Cn, alpha = pins.scaled_rounding_case("bf16")
    Ad = torch.from_numpy(A.view(np.int32)).cuda()
    Bd = torch.from_numpy(B.view(np.int32)).cuda()
    Cd = torch.from_numpy(Cn).cuda()
    D = bmm.mma_tile(Ad, Bd, Cd, 0.0, "bf16", kernel=kernel, alpha=float(alpha), beta=1.0)
    assert D.cpu().numpy()[0, 0, 0, 0, 0] == np.float32(2.0 ** -46)


@pytest.mark.parametrize("kernel", KERNELS)
def test_scaled_in_place(kernel):
    w = C(1, 272, 136, 144, "f16", "quarter", "quarter", c_tensor=True)
    inp = inputs(w)
    A = bmm.pack_operand(gu.dev_u16(inp["a"]), 16)
    B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8)
    Cd = torch.from_numpy(inp["c_tensor"]).cuda()
    ref = bmm.mma_tile(A, B, Cd, 0.0, "f16", kernel=kernel, alpha=0.25, beta=4.0).cpu().numpy()
    bmm.mma_tile(A, B, Cd, 0.0, "f16", out=Cd, kernel=kernel, alpha=0.25, beta=4.0)
    assert np.array_equal(Cd.cpu().numpy(), ref)


def test_scaled_multi_round_grids():
    """The alpha/beta form on grids that take the 4-wave pipeline (256 x 128
    tiles, and more than 256 tiles of 256 x 256) and on the others: 9 batches
    of 1040 x 1288 x 80 (ragged in M, N and K; 270 tiles of 256 x 256, 495 of
    256 x 128), quarter-integer data with C on the quarter grid and
    power-of-two alpha, beta, so every kernel is bit-exact against the oracle's
    alpha/beta form, in place (D = C) as well."""
    w = C(9, 1040, 1288, 80, "bf16", "quarter", "quarter", c_tensor=True, name="scaled_rounds")
    inp = inputs(w)
    print(f"[scaled_rounds] {w.batch}x{w.M}x{w.N}x{w.K}", flush=True)
    A = bmm.pack_operand(gu.dev_u16(inp["a"]), 16)
    B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8)
    Ao, Bo = gu.oracle_operands(w, inp)
    ref = oracle.mma_scaled(Ao, Bo, inp["c_tensor"], 0.0, 0.5, -2.0, w.dtype)
    for kernel in ("tiled", "tiled256x128", "tiled128", "auto"):
        Cd = torch.from_numpy(inp["c_tensor"]).cuda()
        out = torch.full((w.batch, w.M_rep, w.N_rep, 16, 8), float("nan"), device="cuda")
        D = bmm.mma_tile(A, B, Cd, 0.0, w.dtype, out=out, kernel=kernel, alpha=0.5, beta=-2.0)
        assert np.array_equal(D.cpu().numpy(), ref), kernel
        bmm.mma_tile(A, B, Cd, 0.0, w.dtype, out=Cd, kernel=kernel, alpha=0.5, beta=-2.0)
        assert np.array_equal(Cd.cpu().numpy(), ref), kernel + " in place"


def test_scaled_full_8192():
    """8192^3 bf16, C tensor, alpha=0.7, beta=-1.3: sampled outputs within
    1e-3 (|alpha||A||B|^T + |beta||C|) of alpha*P + beta*C, P the oracle's
    product accumulated from zero."""
    w = workloads.WORKLOADS["gemm_8192_bf16_ctensor"]
    inp = inputs(w)
    A = bmm.pack_operand(gu.dev_u16(inp["a"]), 16)
    B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8)
    Cd = torch.from_numpy(inp["c_tensor"]).cuda()
    D = util.tile_to_logical(bmm.mma_tile(A, B, Cd, 0.0, "bf16", alpha=0.7, beta=-1.3).cpu().numpy())
    Ao, Bo = gu.oracle_operands(w, inp)
    idx = util.sample_indices(np.random.default_rng(5), 1, w.M, w.N, 1024)
    P = oracle.mma_sampled(Ao, Bo, None, 0.0, "bf16", idx).astype(np.float64)
    Cl = util.tile_to_logical(inp["c_tensor"])[idx[:, 0], idx[:, 1], idx[:, 2]].astype(np.float64)
    ref = np.float32(0.7) * P + np.float32(-1.3) * Cl
    mag = 0.7 * oracle.bound(Ao, Bo, None, 0.0, "bf16", idx) + 1.3 * np.abs(Cl)
    got = D[idx[:, 0], idx[:, 1], idx[:, 2]].astype(np.float64)
    assert (np.abs(got - ref) <= 1e-3 * mag).all()
