"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees. ``test_oracle.py`` runs them on the real oracle; ``test_oracle_
mutations.py`` runs them on copies of the oracle with a planted mistake and
requires that some pin fails, so that each pin is shown to bite.
"""
import numpy as np

import workloads
from tests import util


def _quarter_bits(rng, shape, dtype):
    return workloads.draw_operand(rng, "quarter", shape, dtype)


def pin_h2f(o):
    """The oracle's half decoder equals numpy (f16) and torch (bf16) on all
    65536 bit patterns; NaN patterns decode to NaN."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dt in ("f16", "bf16"):
        with np.errstate(invalid="ignore"):   # signalling-NaN patterns widen quietly
            got = o.h2f(bits, dt).astype(np.float64)
        ref = util.decode(bits, dt)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), dt
        assert np.array_equal(got[~nan], ref[~nan]), dt


def pin_pack_page_recipe(o):
    """Packer == the page's reshape/transpose/view recipe (mma.sync page,
    worked example host code), for several row and K atoms, both atom heights,
    batch 2, and a row-padded source (ld > K)."""
    rng = np.random.default_rng(1)
    for R, rows, K in ((16, 48, 64), (8, 40, 96), (16, 16, 32)):
        x = util.random_bits(rng, (2, rows, K))
        assert np.array_equal(o.pack(x, R), util.page_recipe_pack(x, R)), (R, rows, K)
        xp = util.random_bits(rng, (2, rows, K + 24))
        assert np.array_equal(o.pack(xp, R, K=K), util.page_recipe_pack(xp[:, :, :K].copy(), R))
    # the page's example: K = 32 packs to (M_repeat, K_repeat, 16, k/2) = (1, 2, 16, 8)
    g = util.golden("mma_sync_worked_example.json")
    P = o.pack(np.zeros((1, 16, 32), np.uint16), 16)
    assert P.shape[1:] == (1, *g["packed_a_shape_uint32"][1:])
    Q = o.pack(np.zeros((1, 8, 32), np.uint16), 8)
    assert Q.shape[1:] == (1, *g["packed_b_shape_uint32"][1:])


def pin_pack_arange(o):
    """Closed form on arange input: word = x | (x+1) << 16 with
    x = (R*r + i)*K + 16*kr + 2*w (the even K value in the low half)."""
    for R, rows, K in ((16, 32, 48), (8, 24, 64)):
        x = np.arange(rows * K, dtype=np.uint32).astype(np.uint16).reshape(1, rows, K)
        P = o.pack(x, R)
        r, kr, i, w = np.meshgrid(np.arange(rows // R), np.arange(K // 16), np.arange(R),
                                  np.arange(8), indexing="ij")
        xv = ((R * r + i) * K + 16 * kr + 2 * w).astype(np.uint32)
        assert np.array_equal(P[0], xv | ((xv + 1) << 16)), (R, rows, K)


def pin_pack_kmajor(o):
    """K-major packer == numpy transpose followed by the row-major packer
    (pinned above), and the arange closed form read through the transpose;
    several atom counts, both atom heights, batch 2, ld > rows."""
    rng = np.random.default_rng(8)
    for R, rows, K, ld in ((16, 48, 64, 48), (8, 40, 96, 56), (16, 16, 16, 24)):
        xt = util.random_bits(rng, (2, K, ld))                      # [b, k, row]
        logical = np.ascontiguousarray(xt[:, :, :rows].transpose(0, 2, 1))
        assert np.array_equal(o.pack_kmajor(xt, R, rows), util.page_recipe_pack(logical, R)), \
            (R, rows, K, ld)
    R, rows, K = 8, 24, 32
    xt = np.arange(K * rows, dtype=np.uint32).astype(np.uint16).reshape(1, K, rows)
    P = o.pack_kmajor(xt, R)
    r, kr, i, w = np.meshgrid(np.arange(rows // R), np.arange(K // 16), np.arange(R),
                              np.arange(8), indexing="ij")
    lo = ((16 * kr + 2 * w) * rows + R * r + i).astype(np.uint32)
    hi = ((16 * kr + 2 * w + 1) * rows + R * r + i).astype(np.uint32)
    assert np.array_equal(P[0], lo | (hi << 16))


def pin_k8_layout(o):
    """Atom K = 8 (m16n8k8 form): the packer equals the page's recipe with
    8-wide atoms; the multiply-accumulate over k=8-packed operands equals the
    one over k=16-packed operands of the same matrices bit for bit (same
    ascending-k recurrence), on normal data with a C tensor, odd K atom
    counts and batch 2; and matches the int64 closed form on quarter data."""
    rng = np.random.default_rng(10)
    for R, rows, K in ((16, 48, 40), (8, 24, 72)):
        x = util.random_bits(rng, (2, rows, K))
        assert np.array_equal(o.pack_k8(x, R), util.page_recipe_pack_k8(x, R)), (R, rows, K)
    dt, batch, Mr, Nr, K = "bf16", 2, 2, 3, 16 * 7
    a = workloads.draw_operand(rng, "normal", (batch, 16 * Mr, K), dt)
    b = workloads.draw_operand(rng, "normal", (batch, 8 * Nr, K), dt)
    C = rng.standard_normal((batch, Mr, Nr, 16, 8), dtype=np.float32)
    D16 = o.mma(o.pack(a, 16), o.pack(b, 8), C, 0.0, dt)
    D8 = o.mma_k8(o.pack_k8(a, 16), o.pack_k8(b, 8), C, 0.0, dt)
    assert np.array_equal(D16, D8)
    K = 8 * 9   # an odd number of k=8 atoms
    a = _quarter_bits(rng, (1, 32, K), dt)
    b = _quarter_bits(rng, (1, 16, K), dt)
    ai = np.rint(4 * util.decode(a, dt)).astype(np.int64)
    bi = np.rint(4 * util.decode(b, dt)).astype(np.int64)
    D = util.tile_to_logical(o.mma_k8(o.pack_k8(a, 16), o.pack_k8(b, 8), None, 0.0, dt))
    assert np.array_equal((D * 16).astype(np.int64), np.einsum("bmk,bnk->bmn", ai, bi))


def pin_roundtrip(o):
    """unpack(pack(x)) == x on all 65536 bit patterns (NaN encodings included),
    for both atom heights: the packer moves bits, never values."""
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(1, 256, 256)
    for R in (16, 8):
        assert np.array_equal(o.unpack(o.pack(x, R), R), x), R


def pin_page_example(o):
    """The worked 16x8 example: the page's recipe, two K16 issues, scalar C=0,
    gives exactly a.f32 @ b.f32.T (the products and sums are exact), which also
    meets the page's rtol=atol=2e-4 check."""
    g = util.golden("mma_sync_worked_example.json")
    r = g["recipe"]
    rng = np.random.default_rng(r["seed"])
    a = (rng.integers(r["integers_low"], r["integers_high_exclusive"], r["a_shape"])
         / r["divide_by"]).astype(r["dtype"])
    b = (rng.integers(r["integers_low"], r["integers_high_exclusive"], r["b_shape"])
         / r["divide_by"]).astype(r["dtype"])
    ap, bp = o.pack(a.view(np.uint16), 16), o.pack(b.view(np.uint16), 8)
    assert ap.reshape(g["packed_a_shape_uint32"]).shape == tuple(g["packed_a_shape_uint32"])
    assert ap.shape[2] == g["K_repeat"] and bp.shape[1] == g["N_repeat"]
    D = o.mma(ap, bp, None, g["scalar_c"], "f16")
    out = util.tile_to_logical(D)[0]
    assert out.shape == tuple(g["out_shape_float32"])
    ref = a.astype(np.float32) @ b.astype(np.float32).T
    np.testing.assert_allclose(out, ref, **g["page_tolerance"])
    assert np.array_equal(out, ref)
    exact16 = (4 * a.astype(np.float64)).astype(np.int64) @ \
        (4 * b.astype(np.float64)).astype(np.int64).T
    assert np.array_equal((out * 16).astype(np.int64), exact16)


def pin_quarter_closed_form(o):
    """Quarter-integer inputs: 16*D = 16*C + sum_k (4a)(4b) in int64 exactly,
    for both dtypes, batch 2, odd repeat counts, tensor and scalar C."""
    rng = np.random.default_rng(2)
    for dt, (batch, Mr, Nr, Kr) in (("f16", (2, 3, 5, 7)), ("bf16", (2, 2, 3, 4)),
                                    ("bf16", (1, 1, 1, 1))):
        M, N, K = 16 * Mr, 8 * Nr, 16 * Kr
        a = _quarter_bits(rng, (batch, M, K), dt)
        b = _quarter_bits(rng, (batch, N, K), dt)
        c_int = rng.integers(-64, 65, (batch, M, N))
        C = util.logical_to_tile((c_int / 4).astype(np.float32))
        ai = (4 * util.decode(a, dt)).astype(np.int64)
        bi = (4 * util.decode(b, dt)).astype(np.int64)
        prod = np.einsum("bmk,bnk->bmn", ai, bi)
        A, B = o.pack(a, 16), o.pack(b, 8)
        D = util.tile_to_logical(o.mma(A, B, C, 0.0, dt))
        assert np.array_equal((D * 16).astype(np.int64), 4 * c_int + prod), (dt, batch, Mr, Nr, Kr)
        D2 = util.tile_to_logical(o.mma(A, B, None, -1.25, dt))
        assert np.array_equal((D2 * 16).astype(np.int64), prod - 20), (dt, "scalar")


def pin_scaled(o):
    """alpha/beta form: with quarter-integer data and power-of-two alpha, beta
    every step is exact, so 16*D = alpha*sum_k(4a)(4b) + beta*16*C in int64;
    alpha=1, beta=1 on the same data equals the plain recurrence; on normal
    data the result is within gamma_K of the float64 value of
    alpha*A*B^T + beta*C, and differs from C-first accumulation somewhere
    (the scaling really happens after the sum)."""
    rng = np.random.default_rng(9)
    dt, batch, Mr, Nr, Kr = "bf16", 2, 2, 3, 5
    M, N, K = 16 * Mr, 8 * Nr, 16 * Kr
    a = _quarter_bits(rng, (batch, M, K), dt)
    b = _quarter_bits(rng, (batch, N, K), dt)
    c_int = rng.integers(-64, 65, (batch, M, N))
    C = util.logical_to_tile((c_int / 4).astype(np.float32))
    A, B = o.pack(a, 16), o.pack(b, 8)
    ai = np.rint(4 * util.decode(a, dt)).astype(np.int64)
    bi = np.rint(4 * util.decode(b, dt)).astype(np.int64)
    prod = np.einsum("bmk,bnk->bmn", ai, bi)
    for alpha, beta in ((0.5, -2.0), (4.0, 0.25), (-1.0, 0.0)):
        D = util.tile_to_logical(o.mma_scaled(A, B, C, 0.0, alpha, beta, dt)).astype(np.float64)
        assert np.array_equal(D * 16, alpha * prod + beta * 4 * c_int), (alpha, beta)
    assert np.array_equal(o.mma_scaled(A, B, C, 0.0, 1.0, 1.0, dt), o.mma(A, B, C, 0.0, dt))
    D = util.tile_to_logical(o.mma_scaled(A, B, None, 1.5, 2.0, -1.0, dt)).astype(np.float64)
    assert np.array_equal(D * 16, 2.0 * prod - 1.5 * 16)
    # normal data
    a = workloads.draw_operand(rng, "normal", (1, 32, 16 * 21), dt)
    b = workloads.draw_operand(rng, "normal", (1, 24, 16 * 21), dt)
    Cn = rng.standard_normal((1, 2, 3, 16, 8), dtype=np.float32)
    A, B = o.pack(a, 16), o.pack(b, 8)
    alpha, beta = np.float32(0.7), np.float32(-1.3)
    D = util.tile_to_logical(o.mma_scaled(A, B, Cn, 0.0, alpha, beta, dt)).astype(np.float64)
    af, bf = util.decode(a, dt), util.decode(b, dt)
    Cl = util.tile_to_logical(Cn).astype(np.float64)
    ref = float(alpha) * (af @ bf.transpose(0, 2, 1)) + float(beta) * Cl
    mag = abs(float(alpha)) * (np.abs(af) @ np.abs(bf).transpose(0, 2, 1)) + abs(float(beta)) * np.abs(Cl)
    assert (np.abs(D - ref) <= util.gamma(16 * 21 + 3) * mag).all()
    first = util.tile_to_logical(o.mma(A, B, Cn, 0.0, dt))
    assert not np.array_equal(util.tile_to_logical(o.mma_scaled(A, B, Cn, 0.0, 1.0, 1.0, dt)), first)
    # one rounding for the final multiply-add (the fma page's test: the exact
    # alpha*acc + t lies between representable results)
    A, B, C, alpha = scaled_rounding_case(dt)
    D = util.tile_to_logical(o.mma_scaled(A, B, C, 0.0, alpha, 1.0, dt))
    assert D[0, 0, 0] == np.float32(2.0 ** -46), D[0, 0, 0]


def scaled_rounding_case(dt):
    """acc[0,0] = 1 + 2^-23 (from 1*1 + 2^-12 * 2^-11), alpha = 1 + 2^-23,
    beta*C = -(1 + 2^-22): fma gives 2^-46, a rounded multiply then add 0."""
    a = np.zeros((1, 16, 16), np.float32)
    b = np.zeros((1, 8, 16), np.float32)
    a[0, 0, 0], a[0, 0, 1] = 1.0, 2.0 ** -12
    b[0, 0, 0], b[0, 0, 1] = 1.0, 2.0 ** -11
    to_bits = workloads.f32_to_bf16_bits if dt == "bf16" else workloads.f32_to_f16_bits
    A = util.page_recipe_pack(to_bits(a), 16)
    B = util.page_recipe_pack(to_bits(b), 8)
    C = np.zeros((1, 1, 1, 16, 8), np.float32)
    C[0, 0, 0, 0, 0] = -(1.0 + 2.0 ** -22)
    return A, B, C, np.float32(1.0 + 2.0 ** -23)


def pin_normal_vs_float64(o):
    """Normal inputs: |D - D_f64| <= gamma_K * (|A||B|^T + |C|) elementwise,
    the worst-case bound of K sequential fp32 additions, against float64 numpy
    matmul of the same half values."""
    rng = np.random.default_rng(3)
    for dt, (batch, Mr, Nr, Kr) in (("bf16", (2, 2, 3, 37)), ("f16", (1, 3, 2, 21))):
        M, N, K = 16 * Mr, 8 * Nr, 16 * Kr
        a = workloads.draw_operand(rng, "normal", (batch, M, K), dt)
        b = workloads.draw_operand(rng, "normal", (batch, N, K), dt)
        C = rng.standard_normal((batch, Mr, Nr, 16, 8), dtype=np.float32)
        A, B = o.pack(a, 16), o.pack(b, 8)
        D = util.tile_to_logical(o.mma(A, B, C, 0.0, dt)).astype(np.float64)
        af, bf = util.decode(a, dt), util.decode(b, dt)
        Cl = util.tile_to_logical(C).astype(np.float64)
        ref = af @ bf.transpose(0, 2, 1) + Cl
        mag = np.abs(af) @ np.abs(bf).transpose(0, 2, 1) + np.abs(Cl)
        err = np.abs(D - ref)
        assert (err <= util.gamma(K) * mag).all(), (dt, float((err / mag).max()))
        # and the rounding is real: the fp32 result is not the fp64 sum cast once
        assert not np.array_equal(D, ref.astype(np.float32).astype(np.float64))


def pin_recurrence_chain(o):
    """C-then-D recurrence: one call over K equals calls chained over K chunks
    (C -> D -> D ...), bitwise, on normal data and with a scalar start."""
    rng = np.random.default_rng(4)
    dt, batch, Mr, Nr, Kr = "bf16", 1, 2, 3, 9
    M, N, K = 16 * Mr, 8 * Nr, 16 * Kr
    a = workloads.draw_operand(rng, "normal", (batch, M, K), dt)
    b = workloads.draw_operand(rng, "normal", (batch, N, K), dt)
    C = rng.standard_normal((batch, Mr, Nr, 16, 8), dtype=np.float32)
    A, B = o.pack(a, 16), o.pack(b, 8)
    full = o.mma(A, B, C, 0.0, dt)
    for cuts in ((4,), (1, 5), (2, 3, 7)):
        bounds = [0, *cuts, Kr]
        D = C
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            D = o.mma(A[:, :, lo:hi], B[:, :, lo:hi], D, 0.0, dt)
        assert np.array_equal(D, full), cuts
    full_s = o.mma(A, B, None, 0.5, dt)
    D = o.mma(A[:, :, :3], B[:, :, :3], None, 0.5, dt)
    D = o.mma(A[:, :, 3:], B[:, :, 3:], D, 0.0, dt)
    assert np.array_equal(D, full_s)


def pin_zero_a_and_scalar(o):
    """A = 0 gives D == C bitwise; a scalar c gives the same bits as a C tensor
    filled with c; K_repeat = 0 (empty sum) gives D == C."""
    rng = np.random.default_rng(5)
    dt, batch, Mr, Nr, Kr = "f16", 2, 2, 3, 4
    M, N, K = 16 * Mr, 8 * Nr, 16 * Kr
    b = workloads.draw_operand(rng, "normal", (batch, N, K), dt)
    C = rng.standard_normal((batch, Mr, Nr, 16, 8), dtype=np.float32)
    A0 = o.pack(np.zeros((batch, M, K), np.uint16), 16)
    B = o.pack(b, 8)
    assert np.array_equal(o.mma(A0, B, C, 0.0, dt), C)
    a = workloads.draw_operand(rng, "normal", (batch, M, K), dt)
    A = o.pack(a, 16)
    c = np.float32(0.7)
    assert np.array_equal(o.mma(A, B, None, c, dt), o.mma(A, B, np.full_like(C, c), 0.0, dt))
    assert np.array_equal(o.mma(A[:, :, :0], B[:, :, :0], C, 0.0, dt), C)


def pin_sampled_matches_full(o):
    """The sampled entry point returns exactly the full result's elements."""
    rng = np.random.default_rng(6)
    dt, batch, Mr, Nr, Kr = "bf16", 2, 3, 5, 6
    M, N, K = 16 * Mr, 8 * Nr, 16 * Kr
    A = o.pack(workloads.draw_operand(rng, "normal", (batch, M, K), dt), 16)
    B = o.pack(workloads.draw_operand(rng, "normal", (batch, N, K), dt), 8)
    C = rng.standard_normal((batch, Mr, Nr, 16, 8), dtype=np.float32)
    full = util.tile_to_logical(o.mma(A, B, C, 0.0, dt))
    idx = util.sample_indices(rng, batch, M, N, 200)
    got = o.mma_sampled(A, B, C, 0.0, dt, idx)
    assert np.array_equal(got, full[idx[:, 0], idx[:, 1], idx[:, 2]])


def pin_bound(o):
    """The tolerance scale of every normal-input parity test, |A|.|B|^T + |C|
    (absolute values elementwise), against float64 numpy on the decoded
    absolute values of the same halves: a sum of non-negative terms, so the
    oracle's fp32 recurrence lies within gamma_K of it relatively. Words whose
    two halves differ only in the sign bit, a C tensor of both signs and a
    negative scalar c are included; the sampled form equals the full form."""
    rng = np.random.default_rng(11)
    for dt, (batch, Mr, Nr, Kr) in (("bf16", (2, 2, 3, 5)), ("f16", (1, 3, 2, 4))):
        M, N, K = 16 * Mr, 8 * Nr, 16 * Kr
        a = workloads.draw_operand(rng, "normal", (batch, M, K), dt)
        b = workloads.draw_operand(rng, "normal", (batch, N, K), dt)
        # first atom row of A: each word holds x and -x (halves differing in sign only)
        a[:, :16, 1::2] = a[:, :16, 0::2] ^ np.uint16(0x8000)
        C = rng.standard_normal((batch, Mr, Nr, 16, 8), dtype=np.float32)
        A, B = o.pack(a, 16), o.pack(b, 8)
        af, bf = np.abs(util.decode(a, dt)), np.abs(util.decode(b, dt))
        prod = af @ bf.transpose(0, 2, 1)
        for Ct, c in ((C, 0.0), (None, -0.75)):
            ref = prod + (np.abs(util.tile_to_logical(Ct).astype(np.float64)) if Ct is not None
                          else abs(c))
            got = util.tile_to_logical(o.bound(A, B, Ct, c, dt)).astype(np.float64)
            assert (got >= 0).all(), dt
            assert (np.abs(got - ref) <= util.gamma(K) * ref).all(), \
                (dt, c, float((np.abs(got - ref) / ref).max()))
            idx = util.sample_indices(rng, batch, M, N, 100)
            assert np.array_equal(o.bound(A, B, Ct, c, dt, idx),
                                  util.tile_to_logical(o.bound(A, B, Ct, c, dt))[
                                      idx[:, 0], idx[:, 1], idx[:, 2]]), (dt, "sampled")


def pin_k8_sampled_matches_full(o):
    """The sampled entry of the k = 8 form (the reference of the full-size
    k = 8 tests) returns exactly the full k = 8 result's elements, with a C
    tensor and with a scalar c, for an odd number of k = 8 atoms."""
    rng = np.random.default_rng(12)
    dt, batch, Mr, Nr, K = "bf16", 2, 2, 3, 8 * 7
    M, N = 16 * Mr, 8 * Nr
    A = o.pack_k8(workloads.draw_operand(rng, "normal", (batch, M, K), dt), 16)
    B = o.pack_k8(workloads.draw_operand(rng, "normal", (batch, N, K), dt), 8)
    C = rng.standard_normal((batch, Mr, Nr, 16, 8), dtype=np.float32)
    idx = util.sample_indices(rng, batch, M, N, 150)
    for Ct, c in ((C, 0.0), (None, -0.5)):
        full = util.tile_to_logical(o.mma_k8(A, B, Ct, c, dt))
        got = o.mma_k8_sampled(A, B, Ct, c, dt, idx)
        assert np.array_equal(got, full[idx[:, 0], idx[:, 1], idx[:, 2]]), c


def pin_box_page_example(o):
    """The page's two-box example: the (2,8,16) image read back row by row is
    arange(256); 512 bytes per box, 1024 per barrier phase."""
    g = util.golden("tma_two_box_example.json")
    x = np.arange(256, dtype=np.uint32).reshape(16, 16)
    img, nbytes = o.box_copy(x, g["box"], g["coords"], g["n_repeat"], g["coord_steps"][0])
    assert img.shape == tuple(g["image_shape"])
    assert nbytes == g["bytes_per_barrier_phase"] == g["n_repeat"] * g["bytes_per_box"]
    assert np.array_equal(img.reshape(16, 16), x)


def pin_box_oob(o):
    """Boxes partly outside the tensor: inside elements are copied, the rest
    are zero (the default fill); checked against zero-padding + slicing, for
    ranks 1-3, several element sizes, negative starts and repeat steps."""
    rng = np.random.default_rng(7)
    cases = [
        (np.uint32, (16, 16), (8, 16), (-3, 5), 3, (6, -4)),
        (np.uint16, (5, 7, 9), (4, 4, 8), (3, -2, 4), 2, (-4, 3, 1)),
        (np.uint8, (37,), (32,), (20,), 2, (-25,)),
        (np.uint64, (9, 11), (3, 5), (0, 0), 4, (3, 3)),
    ]
    for dtype, shape, box, coords, rep, step in cases:
        x = rng.integers(1, 200, shape).astype(dtype)
        img, nbytes = o.box_copy(x, box, coords, rep, step)
        pad = 300
        xp = np.pad(x, [(pad, pad)] * len(shape))
        for t in range(rep):
            start = [pad + c + t * s for c, s in zip(coords, step)]
            ref = xp[tuple(slice(s0, s0 + bx) for s0, bx in zip(start, box))]
            assert np.array_equal(img[t], ref), (dtype, shape, t)
        assert nbytes == rep * int(np.prod(box)) * np.dtype(dtype).itemsize


# ---- box store and add reduction (cp.async.bulk.tensor page, "Stores,
# reductions, and completion") ----

def _padded_store(G, img, box, coords, step, combine):
    """Brute force: pad G, apply each repeat's image to its slice with numpy
    in repeat order, crop."""
    pad = 300
    xp = np.pad(G, [(pad, pad)] * G.ndim)
    inside = np.pad(np.ones(G.shape, bool), [(pad, pad)] * G.ndim)
    for t in range(img.shape[0]):
        sl = tuple(slice(pad + c + t * st, pad + c + t * st + bx)
                   for c, st, bx in zip(coords, step, box))
        m = inside[sl]
        xp[sl] = np.where(m, combine(xp[sl], img[t]), xp[sl])
    return xp[tuple(slice(pad, pad + n) for n in G.shape)]


def pin_box_store_page_example(o):
    """The page's two-box example read backwards: storing the (2, 8, 16) image
    of arange(256) at (0, 0) with step (8, 0) rebuilds the 16x16 tensor, and a
    store after a load of the same boxes is the identity."""
    x = np.arange(256, dtype=np.uint32).reshape(16, 16)
    out, nbytes = o.box_store(np.zeros_like(x), x.reshape(2, 8, 16), (8, 16), (0, 0), 2, (8, 0))
    assert np.array_equal(out, x) and nbytes == 1024
    rng = np.random.default_rng(12)
    y = rng.integers(0, 1 << 16, (12, 40)).astype(np.uint16)
    img, _ = o.box_copy(y, (4, 16), (2, 8), 3, (3, 1))
    back, _ = o.box_store(np.zeros_like(y), img, (4, 16), (2, 8), 3, (3, 1))
    touched = np.zeros(y.shape, bool)
    for t in range(3):
        touched[2 + 3 * t: 6 + 3 * t, 8 + t: 24 + t] = True
    assert np.array_equal(back[touched], y[touched]) and not back[~touched].any()


def pin_box_store_oob(o):
    """Stores partly outside the tensor write only the inside elements, and
    overlapping repeats leave the last repeat's values; checked against numpy
    slice assignment on a padded copy, for ranks 1-3 and several element sizes."""
    rng = np.random.default_rng(13)
    cases = [
        (np.uint32, (16, 16), (8, 16), (-3, 5), 3, (6, -4)),
        (np.uint16, (5, 7, 9), (4, 4, 8), (3, -2, 4), 2, (-4, 3, 1)),
        (np.uint8, (37,), (32,), (20,), 2, (-25,)),
        (np.uint64, (9, 11), (3, 5), (0, 0), 4, (1, 2)),      # repeats overlap
        (np.uint32, (8, 8), (4, 4), (2, 2), 3, (0, 0)),        # same box three times
    ]
    for dtype, shape, box, coords, rep, step in cases:
        G = rng.integers(1, 200, shape).astype(dtype)
        img = rng.integers(1, 200, (rep, *box)).astype(dtype)
        got, nbytes = o.box_store(G, img, box, coords, rep, step)
        ref = _padded_store(G, img, box, coords, step, lambda old, new: new)
        assert np.array_equal(got, ref), (dtype, shape)
        assert nbytes == rep * int(np.prod(box)) * np.dtype(dtype).itemsize


def _finite_bits(rng, shape, dt):
    bits = rng.integers(0, 1 << 16, shape, dtype=np.uint32).astype(np.uint16)
    expo_all_ones = 0x7C00 if dt == "f16" else 0x7F80
    return np.where((bits & expo_all_ones) == expo_all_ones, bits & ~np.uint16(0x4000), bits)


def pin_box_reduce_library_adds(o):
    """The add reduction of one element is the library's own addition in the
    element type: numpy float32 / float16 (computed through float32 and rounded
    once more, which is exact rounding for these formats), torch bfloat16 on
    the CPU, and wrap-around int32 / int64. Operands are random finite bit
    patterns, so ties, subnormals and overflow to infinity all occur."""
    import torch
    rng = np.random.default_rng(14)
    shape, box, coords = (24, 40), (16, 32), (3, 5)
    sl = (slice(3, 19), slice(5, 37))
    G32 = rng.standard_normal(shape).astype(np.float32) * np.float32(1e3)
    I32 = rng.standard_normal((1, *box)).astype(np.float32)
    got, _ = o.box_store(G32, I32, box, coords, op="add", elem_type="f32")
    ref = G32.copy()
    ref[sl] = ref[sl] + I32[0]
    assert np.array_equal(got, ref)
    for dt in ("f16", "bf16"):
        G = _finite_bits(rng, shape, dt)
        img = _finite_bits(rng, (1, *box), dt)
        got, _ = o.box_store(G, img, box, coords, op="add", elem_type=dt)
        ref = G.copy()
        if dt == "f16":
            with np.errstate(over="ignore"):
                ref[sl] = (G[sl].view(np.float16) + img[0].view(np.float16)).view(np.uint16)
        else:
            tg = torch.from_numpy(G[sl].view(np.int16).copy()).view(torch.bfloat16)
            ti = torch.from_numpy(img[0].view(np.int16).copy()).view(torch.bfloat16)
            ref[sl] = (tg + ti).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, ref), dt
    for it, dt in ((np.int32, "i32"), (np.int64, "i64")):
        info = np.iinfo(it)
        G = rng.integers(info.min, info.max, shape, dtype=it)
        img = rng.integers(info.min, info.max, (1, *box), dtype=it)
        got, _ = o.box_store(G, img, box, coords, op="add", elem_type=dt)
        ref = G.copy()
        with np.errstate(over="ignore"):
            ref[sl] = G[sl] + img[0]
        assert np.array_equal(got, ref), dt


def pin_box_reduce_order(o):
    """Overlapping repeats are added one at a time in repeat order, each add
    rounded: 1 + 2^-24 + 2^-24 stays 1 (ties to even twice), where summing
    the images first would give 1 + 2^-23. Partly outside boxes add only
    inside elements; checked against numpy on a padded copy."""
    one = np.ones((4, 4), np.float32)
    img = np.full((2, 4, 4), 2.0 ** -24, np.float32)
    got, _ = o.box_store(one, img, (4, 4), (0, 0), 2, (0, 0), op="add", elem_type="f32")
    assert (got == 1.0).all()
    rng = np.random.default_rng(15)
    G = rng.standard_normal((9, 11)).astype(np.float32)
    img = rng.standard_normal((4, 3, 5)).astype(np.float32)
    got, _ = o.box_store(G, img, (3, 5), (-1, 7), 4, (2, -1), op="add", elem_type="f32")
    ref = _padded_store(G, img, (3, 5), (-1, 7), (2, -1), lambda old, new: old + new)
    assert np.array_equal(got, ref)


# ---- split-K form ----

def _splitk_bounds(K, S):
    steps = -(-K // 32)
    S = min(S, steps)
    return [(32 * (s * steps // S), min(32 * ((s + 1) * steps // S), K)) for s in range(S)]


def pin_splitk_exact_and_degenerate(o):
    """Quarter-integer data: every split count gives the same bits as the
    recurrence (all sums exact). One split with C = 0 is the recurrence itself
    on normal data. K = 0 leaves D = C bit for bit, -0 included."""
    rng = np.random.default_rng(16)
    for dt, (M, N, K) in (("bf16", (32, 24, 224)), ("f16", (16, 40, 96))):
        a = _quarter_bits(rng, (2, M, K), dt)
        b = _quarter_bits(rng, (2, N, K), dt)
        A, B = o.pack(a, 16), o.pack(b, 8)
        C = (rng.integers(-64, 65, (2, M // 16, N // 8, 16, 8)) / 4).astype(np.float32)
        ref = o.mma(A, B, C, 0.0, dt)
        for S in (1, 2, 3, 5, 7, 100):
            assert np.array_equal(o.mma_splitk(A, B, C, 0.0, dt, S), ref), (dt, S)
    a = workloads.f32_to_bf16_bits(rng.standard_normal((1, 32, 160)).astype(np.float32))
    b = workloads.f32_to_bf16_bits(rng.standard_normal((1, 16, 160)).astype(np.float32))
    A, B = o.pack(a, 16), o.pack(b, 8)
    assert np.array_equal(o.mma_splitk(A, B, None, 0.0, "bf16", 1), o.mma(A, B, None, 0.0, "bf16"))
    C = rng.standard_normal((1, 2, 2, 16, 8)).astype(np.float32)
    C[0, 0, 0, 0, :4] = -0.0
    A0 = np.zeros((1, 2, 0, 16, 8), np.uint32)
    B0 = np.zeros((1, 2, 0, 8, 8), np.uint32)
    D0 = o.mma_splitk(A0, B0, C, 0.0, "bf16", 4)
    assert np.array_equal(D0.view(np.uint32), C.view(np.uint32))


def pin_splitk_boundaries_and_order(o):
    """Where the K axis is cut and how the partial sums meet C, fixed by
    single-rounding cases. K = 160 is 5 steps of 32; two splits take steps
    [0, 2) and [2, 5). C = 1, each product 2^-12 * 2^-12 = 2^-24:
      column 0: products at k = 0, 1 (one split): 1 + 2^-23
      column 1: products at k = 40, 70 (steps 1 and 2, two splits): 1
      column 2: products at k = 100, 130 (steps 3, 4, one split): 1 + 2^-23
    With a single split every column is 1 + 2^-23 (C meets the whole partial
    sum once), while the C-first recurrence gives 1 everywhere."""
    K = 160
    assert _splitk_bounds(K, 2) == [(0, 64), (64, 160)]
    h = np.float32(2.0 ** -12)
    a = np.zeros((1, 16, K), np.float32)
    b = np.zeros((1, 8, K), np.float32)
    a[0, 0, [0, 1, 40, 70, 100, 130]] = h
    b[0, 0, [0, 1]] = h
    b[0, 1, [40, 70]] = h
    b[0, 2, [100, 130]] = h
    b[0, 3, [40, 70]] = h
    A = o.pack(workloads.f32_to_bf16_bits(a), 16)
    B = o.pack(workloads.f32_to_bf16_bits(b), 8)
    big = np.float32(1 + 2.0 ** -23)
    D2 = o.mma_splitk(A, B, None, 1.0, "bf16", 2)[0, 0, 0, 0, :4]
    assert list(D2[:3]) == [big, 1.0, big], D2
    D1 = o.mma_splitk(A, B, None, 1.0, "bf16", 1)[0, 0, 0, 0, :4]
    assert (D1 == big).all(), D1
    assert (o.mma(A, B, None, 1.0, "bf16")[0, 0, 0, 0, :4] == 1.0).all()


def pin_splitk_normal_and_layouts(o):
    """Normal bf16 data, C tensor: every split count stays within
    gamma_(K+S+1) (|A||B|^T + |C|) of the float64 product (at most K + S + 1
    roundings on any path); the k = 8 layout of the same operands gives the
    same bits; sampled outputs equal the full result."""
    rng = np.random.default_rng(17)
    M, N, K = 32, 24, 328
    a = workloads.f32_to_bf16_bits(rng.standard_normal((1, M, K)).astype(np.float32))
    b = workloads.f32_to_bf16_bits(rng.standard_normal((1, N, K)).astype(np.float32))
    C = rng.standard_normal((1, M // 16, N // 8, 16, 8)).astype(np.float32)
    Kp = K + (-K) % 16
    a16 = np.pad(a, ((0, 0), (0, 0), (0, Kp - K)))
    b16 = np.pad(b, ((0, 0), (0, 0), (0, Kp - K)))
    A16, B16 = o.pack(a16, 16), o.pack(b16, 8)
    A8, B8 = o.pack_k8(a, 16), o.pack_k8(b, 8)
    af, bf = util.decode(a[0], "bf16"), util.decode(b[0], "bf16")
    exact = af @ bf.T + util.tile_to_logical(C)[0].astype(np.float64)
    mag = np.abs(af) @ np.abs(bf).T + np.abs(util.tile_to_logical(C)[0])
    for S in (1, 2, 3, 11):
        D8 = o.mma_splitk(A8, B8, C, 0.0, "bf16", S)
        err = np.abs(util.tile_to_logical(D8)[0] - exact)
        assert (err <= util.gamma(K + S + 1) * mag).all(), S
        # k = 16 holds the same values plus zero padding: same bits where the
        # padding does not move a split boundary
        if _splitk_bounds(K, S) == [(lo, min(hi, K)) for lo, hi in _splitk_bounds(Kp, S)]:
            assert np.array_equal(o.mma_splitk(A16, B16, C, 0.0, "bf16", S), D8), S
        idx = util.sample_indices(rng, 1, M, N, 40)
        got = o.mma_splitk_sampled(A8, B8, C, 0.0, "bf16", S, idx)
        assert np.array_equal(got, util.tile_to_logical(D8)[idx[:, 0], idx[:, 1], idx[:, 2]])


ALL_PINS = {name: fn for name, fn in globals().items() if name.startswith("pin_")}
