"""GPU parity of bmm_pack_operand and bmm_box_copy against the oracle:
bit-exact (these move bits, never values)."""
import numpy as np
import pytest
import torch

import bf16_matrix_multiply_amd as bmm
import oracle
import workloads
from tests import gpu_util as gu
from tests import util

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("R", [16, 8])
def test_pack_all_bit_patterns(R):
    """Every 16-bit pattern (NaN and Inf encodings included) lands bit-exactly
    where the oracle packer puts it, for several batches."""
    x = np.arange(1 << 17, dtype=np.uint32).astype(np.uint16).reshape(2, 256, 256)
    got = gu.host_u32(bmm.pack_operand(gu.dev_u16(x), R))
    assert np.array_equal(got, oracle.pack(x, R))


@pytest.mark.parametrize("R,rows,K,ld", [(16, 16, 16, 16), (8, 8, 32, 40), (16, 48, 80, 96),
                                         (8, 40, 2064, 2072), (16, 272, 336, 336),
                                         (16, 32, 1040, 1048)])
def test_pack_shapes_and_row_padding(R, rows, K, ld):
    rng = np.random.default_rng(rows + K)
    x = util.random_bits(rng, (3, rows, ld))
    got = gu.host_u32(bmm.pack_operand(gu.dev_u16(x), R, K=K))
    assert np.array_equal(got, oracle.pack(x, R, K=K))


def test_pack_full_size_operands():
    """The 8192x8192 and 16384x16384 operands of the large workloads."""
    rng = np.random.default_rng(0)
    for rows, K, R in ((8192, 8192, 16), (16384, 16384, 8)):
        x = workloads.draw_operand(rng, "normal", (1, rows, K), "bf16")
        got = gu.host_u32(bmm.pack_operand(gu.dev_u16(x), R))
        assert np.array_equal(got, oracle.pack(x, R)), (rows, K, R)
        del got, x


def test_pack_empty_and_errors():
    x = torch.zeros((1, 16, 32), dtype=torch.int16, device="cuda")
    assert bmm.pack_operand(x[:, :0], 16).numel() == 0
    # a host-side rejection writes nothing
    bad = torch.zeros((1, 24, 32), dtype=torch.int16, device="cuda")
    sentinel = torch.full((1, 1, 2, 16, 8), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(bmm.BmmError, match="multiple of atom_rows"):
        bmm.pack_operand(bad, 16, out=sentinel)
    torch.cuda.synchronize()
    assert (sentinel == 7).all()


@pytest.mark.parametrize("R", [16, 8])
def test_pack_kmajor_all_bit_patterns(R):
    """K-major source: every bit pattern lands where the oracle puts it."""
    xt = np.arange(1 << 17, dtype=np.uint32).astype(np.uint16).reshape(2, 256, 256)
    got = gu.host_u32(bmm.pack_operand_kmajor(gu.dev_u16(xt), R))
    assert np.array_equal(got, oracle.pack_kmajor(xt, R))


@pytest.mark.parametrize("R,rows,K,ld", [(16, 16, 16, 16), (8, 8, 32, 40), (16, 48, 80, 96),
                                         (8, 200, 336, 208), (16, 272, 1040, 272),
                                         (16, 64, 64, 64), (8, 72, 144, 80)])
def test_pack_kmajor_shapes(R, rows, K, ld):
    """Ragged 64x64 tiles in both directions, ld > rows, batch 3."""
    rng = np.random.default_rng(rows * 7 + K)
    xt = util.random_bits(rng, (3, K, ld))
    got = gu.host_u32(bmm.pack_operand_kmajor(gu.dev_u16(xt), R, rows=rows))
    assert np.array_equal(got, oracle.pack_kmajor(xt, R, rows))


@pytest.mark.parametrize("R", [16, 8])
def test_pack_kmajor_k8_all_bit_patterns(R):
    """K-major source into the m16n8k8 layout: every bit pattern lands where
    the oracle's k = 8 packer puts it for the row-major matrix."""
    xt = np.arange(1 << 17, dtype=np.uint32).astype(np.uint16).reshape(2, 256, 256)
    got = gu.host_u32(bmm.pack_operand_kmajor(gu.dev_u16(xt), R, atom_k=8))
    assert np.array_equal(got, oracle.pack_k8(np.swapaxes(xt, 1, 2), R))


@pytest.mark.parametrize("R,rows,K,ld", [(16, 16, 8, 16), (8, 8, 24, 40), (16, 48, 72, 96),
                                         (8, 200, 328, 208), (16, 272, 1032, 272),
                                         (16, 64, 64, 64), (8, 72, 136, 80)])
def test_pack_kmajor_k8_shapes(R, rows, K, ld):
    """k = 8 from K-major sources: ragged 64x64 tiles, K an odd number of
    8-deep atoms, ld > rows, batch 3; equal to the row-major k = 8 packer's
    words on the logical matrix."""
    rng = np.random.default_rng(rows * 11 + K)
    xt = util.random_bits(rng, (3, K, ld))
    got = gu.host_u32(bmm.pack_operand_kmajor(gu.dev_u16(xt), R, rows=rows, atom_k=8))
    x = np.ascontiguousarray(np.swapaxes(xt, 1, 2)[:, :rows, :])
    assert np.array_equal(got, oracle.pack_k8(x, R))


def test_pack_kmajor_equals_rowmajor_pack_full_size():
    """At 8192x8192 (A) and 16384x16384 (B): packing the K-major copy gives
    the same words as packing the row-major matrix, and the oracle's words."""
    rng = np.random.default_rng(3)
    for rows, K, R in ((8192, 8192, 16), (16384, 16384, 8)):
        x = workloads.draw_operand(rng, "normal", (1, rows, K), "bf16")
        xd = gu.dev_u16(x)
        xtd = xd.transpose(1, 2).contiguous()
        got = bmm.pack_operand_kmajor(xtd, R)
        ref = bmm.pack_operand(xd, R)
        assert torch.equal(got, ref), (rows, K)
        assert torch.equal(bmm.pack_operand_kmajor(xtd, R, atom_k=8),
                           bmm.pack_operand(xd, R, atom_k=8)), (rows, K, 8)
        if rows == 8192:
            assert np.array_equal(gu.host_u32(got), oracle.pack(x, R))
        del x, xd, xtd, got, ref


def test_box_page_example():
    """Two 8x16 uint32 boxes at (0,0) and (8,0): the image read back is the
    16x16 input, 1024 bytes for the two boxes."""
    g = util.golden("tma_two_box_example.json")
    x = np.arange(256, dtype=np.uint32).reshape(16, 16)
    xd = torch.from_numpy(x.view(np.int32)).cuda()
    for swz in range(4):
        img, nbytes = bmm.box_copy(xd, g["box"], g["coords"], g["n_repeat"], g["coord_steps"][0],
                                   swizzle=swz)
        torch.cuda.synchronize()
        assert tuple(img.shape) == tuple(g["image_shape"])
        assert nbytes == g["bytes_per_barrier_phase"]
        assert np.array_equal(img.cpu().numpy().view(np.uint32).reshape(16, 16), x)


BOX_CASES = [
    (np.uint32, (16, 16), (8, 16), (-3, 5), 3, (6, -4)),
    (np.uint16, (5, 7, 64), (4, 4, 40), (3, -2, 4), 2, (-4, 3, 1)),
    (np.uint8, (3, 112), (2, 128), (0, -20), 2, (1, 25)),
    (np.int64, (9, 12), (3, 5), (0, 0), 4, (3, 3)),
    (np.uint16, (2, 3, 4, 5, 16), (2, 2, 3, 4, 16), (0, 1, -1, 2, 0), 3, (1, 0, 1, -1, 8)),
    (np.uint32, (300, 64), (256, 64), (20, 0), 1, (0, 0)),
]


@pytest.mark.parametrize("swizzle", [0, 1, 2, 3])
@pytest.mark.parametrize("case", range(len(BOX_CASES)))
def test_box_matches_oracle(case, swizzle):
    dtype, shape, box, coords, rep, step = BOX_CASES[case]
    rng = np.random.default_rng(case)
    x = rng.integers(1, 120, shape).astype(dtype)
    ref, ref_bytes = oracle.box_copy(x, box, coords, rep, step)
    tdt = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[x.itemsize]
    xd = torch.from_numpy(x.view({1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}[x.itemsize])).cuda()
    assert xd.dtype == tdt
    img, nbytes = bmm.box_copy(xd, box, coords, rep, step, swizzle=swizzle)
    torch.cuda.synchronize()
    assert nbytes == ref_bytes
    assert np.array_equal(img.cpu().numpy().view(x.dtype), ref)


# 16-byte-path descriptors (every chunk wholly inside or outside), partly
# outside the tensor in every dimension, inner dimension included
CHUNK_BOX_CASES = [
    (np.uint32, (20, 48), (8, 16), (-4, -8), 4, (6, 12)),
    (np.uint16, (6, 5, 40), (3, 4, 16), (4, -2, -8), 3, (-2, 3, 24)),
    (np.uint8, (3, 80), (2, 48), (1, -16), 3, (1, 48)),
    (np.int64, (9, 12), (3, 4), (-1, -2), 3, (4, 6)),
    (np.uint32, (2, 130, 64), (1, 64, 64), (0, -32, 0), 5, (1, 64, 0)),
    # 64 KiB boxes (the limit: 1024 lanes, four chunks each)
    (np.uint32, (300, 300), (64, 256), (-16, 64), 3, (100, 16)),
    (np.uint8, (400, 304), (256, 256), (-8, 16), 2, (150, 32)),
]


def chunk_path(itemsize, shape, box, coords, step):
    """Whether the library takes its 16-byte box path for this descriptor:
    innermost box row, start, step and extent all whole 16-byte chunks."""
    return all((v * itemsize) % 16 == 0 for v in (box[-1], coords[-1], step[-1], shape[-1]))


@pytest.mark.parametrize("swizzle", [0, 1, 3])
@pytest.mark.parametrize("case", range(len(CHUNK_BOX_CASES)))
def test_box_chunk_path_matches_oracle(case, swizzle):
    dtype, shape, box, coords, rep, step = CHUNK_BOX_CASES[case]
    assert chunk_path(np.dtype(dtype).itemsize, shape, box, coords, step)
    rng = np.random.default_rng(100 + case)
    x = rng.integers(1, 120, shape).astype(dtype)
    ref, ref_bytes = oracle.box_copy(x, box, coords, rep, step)
    xd = torch.from_numpy(x.view({1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}[x.itemsize])).cuda()
    img, nbytes = bmm.box_copy(xd, box, coords, rep, step, swizzle=swizzle)
    torch.cuda.synchronize()
    assert nbytes == ref_bytes
    assert np.array_equal(img.cpu().numpy().view(x.dtype), ref)


def test_box_errors_leave_output():
    x = torch.arange(256, dtype=torch.int32, device="cuda").reshape(16, 16)
    out = torch.full((1, 8, 16), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(bmm.BmmError, match="swizzle"):
        bmm.box_copy(x, (8, 16), (0, 0), 1, swizzle=5, out=out)
    with pytest.raises(bmm.BmmError, match="box"):
        bmm.box_copy(x, (8, 300), (0, 0), 1, out=out)
    torch.cuda.synchronize()
    assert (out == -1).all()
