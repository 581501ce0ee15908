"""The C-ABI library on the CPU: it loads, exports every symbol include/bmm.h
declares, and rejects every invalid argument on the host before any HIP call
(so no GPU is needed; nothing valid is ever launched here)."""
import ctypes
import os
import re

import pytest

import bf16_matrix_multiply_amd as bmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bmm.h")

EINVAL, EALIGN, EOVERLAP, ERANGE = -1, -2, -3, -4

# Fake device addresses: only compared and range-checked by the validator,
# never dereferenced (every call below fails validation first).
P0, P1, P2, P3 = 0x7F0000000000, 0x7F1000000000, 0x7F2000000000, 0x7F3000000000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bmm.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return bmm.lib()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bmm_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert set(syms) >= {"bmm_pack_operand", "bmm_box_copy", "bmm_mma_tile", "bmm_last_error"}
    for s in syms:
        assert hasattr(L, s), f"libbmm.so does not export {s}"
    assert L.bmm_abi_version() == 1


def err(L):
    return L.bmm_last_error().decode()


def pack(L, dst=P0, src=P1, batch=1, rows=16, K=32, ld=32, R=16):
    return L.bmm_pack_operand(dst, src, batch, rows, K, ld, R, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(R=4), EINVAL, "atom_rows"),
    (dict(rows=24, R=16), EINVAL, "multiple of atom_rows"),
    (dict(K=40, ld=48), EINVAL, "multiple of 16"),
    (dict(ld=16), EINVAL, "ld_src"),
    (dict(batch=-1), EINVAL, "negative"),
    (dict(K=-16), EINVAL, "negative"),
    (dict(ld=36), EALIGN, "multiple of 8"),
    (dict(dst=P0 + 4), EALIGN, "aligned"),
    (dict(src=P1 + 2), EALIGN, "aligned"),
    (dict(dst=0), EINVAL, "null"),
    (dict(dst=P1 + 64), EOVERLAP, "overlaps"),
])
def test_pack_rejects(L, kw, code, needle):
    assert pack(L, **kw) == code
    assert needle in err(L)


def test_pack_empty_is_noop(L):
    # zero extents never reach HIP and need no pointers
    assert pack(L, dst=0, src=0, batch=0) == 0
    assert pack(L, dst=0, src=0, rows=0) == 0
    assert pack(L, dst=0, src=0, K=0, ld=0) == 0


def box_desc(**kw):
    d = bmm.BoxDesc()
    d.rank, d.elem_bytes = 2, 4
    d.dims[0], d.dims[1] = 16, 16
    d.strides[0], d.strides[1] = 64, 4
    d.box[0], d.box[1] = 8, 16
    d.n_repeat = 2
    d.coord_step[0] = 8
    for k, v in kw.items():
        if isinstance(v, tuple):
            getattr(d, k)[v[0]] = v[1]
        else:
            setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,code,needle", [
    (dict(rank=0), EINVAL, "rank"),
    (dict(rank=6), EINVAL, "rank"),
    (dict(elem_bytes=3), EINVAL, "elem_bytes"),
    (dict(box=(0, 0)), EINVAL, "box[0]"),
    (dict(box=(1, 257)), EINVAL, "box[1]"),
    (dict(swizzle=4), EINVAL, "swizzle"),
    (dict(swizzle=-1), EINVAL, "swizzle"),
    (dict(oob_fill=1), EINVAL, "oob_fill"),
    (dict(n_repeat=0), EINVAL, "n_repeat"),
    (dict(dims=(0, 0)), EINVAL, "dims[0]"),
    (dict(strides=(1, 8)), EINVAL, "innermost stride"),
    (dict(strides=(0, 72)), EALIGN, "multiple of 16"),
    (dict(strides=(0, -64)), EINVAL, "positive"),
    (dict(box=(0, 256), elem_bytes=8, strides=(1, 8)), ERANGE, "limit"),
])
def test_box_rejects(L, kw, code, needle):
    if "box" in kw and kw.get("elem_bytes") == 8:
        d = box_desc(elem_bytes=8)
        d.box[0], d.box[1] = 256, 256
        d.strides[1] = 8
    else:
        d = box_desc(**kw)
    n = ctypes.c_int64(-7)
    assert L.bmm_box_copy(P0, P1, ctypes.byref(d), ctypes.byref(n), None) == code
    assert needle in err(L)
    assert n.value == -7  # untouched on failure


def test_box_rejects_pointers(L):
    d = box_desc()
    assert L.bmm_box_copy(P0 + 8, P1, ctypes.byref(d), None, None) == EALIGN
    assert L.bmm_box_copy(0, P1, ctypes.byref(d), None, None) == EINVAL
    assert L.bmm_box_copy(P1 + 512, P1, ctypes.byref(d), None, None) == EOVERLAP
    assert L.bmm_box_copy(P0, P1, None, None, None) == EINVAL


def mma(L, D=P0, A=P1, B=P2, C=None, batch=1, M=2, N=3, K=4, dtype=1, kernel=0):
    return L.bmm_mma_tile_with(D, A, B, C, 0.0, batch, M, N, K, dtype, kernel, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(dtype=2), EINVAL, "dtype"),
    (dict(kernel=7), EINVAL, "kernel"),
    (dict(M=-1), EINVAL, "negative"),
    (dict(K=-1), EINVAL, "negative"),
    (dict(D=0), EINVAL, "D is null"),
    (dict(A=0), EINVAL, "null"),
    (dict(D=P0 + 4), EALIGN, "aligned"),
    (dict(A=P1 + 8), EALIGN, "aligned"),
    (dict(C=P3 + 4), EALIGN, "aligned"),
    (dict(D=P1 + 512), EOVERLAP, "overlaps A"),
    (dict(D=P2), EOVERLAP, "overlaps B"),
    (dict(C=P0 + 512), EOVERLAP, "partially overlaps C"),
    (dict(M=1 << 41), EINVAL, "too large"),
])
def test_mma_rejects(L, kw, code, needle):
    assert mma(L, **kw) == code
    assert needle in err(L)


def test_mma_empty_is_noop(L):
    assert mma(L, D=0, A=0, B=0, batch=0) == 0
    assert mma(L, D=0, A=0, B=0, M=0) == 0
    assert mma(L, D=0, A=0, B=0, N=0) == 0


def test_plain_entry_point_validates(L):
    assert L.bmm_mma_tile(P0 + 4, P1, P2, None, 0.0, 1, 1, 1, 1, 1, None) == EALIGN


def test_select_kernel(L):
    assert L.bmm_select_kernel(-1, 1, 1, 1) == EINVAL
    # 256 x 256 tiles only above 128 of them: 3072^3 (144 tiles) and 8192^3
    # take the large ones; 8192 x 1024 (128 of them) takes 256 x 128 tiles (256
    # of those), as do 2560^2 (200) and 2304 x 2048 (144); 2048^2 (128 of
    # those) takes 128 x 128
    assert L.bmm_select_kernel(1, 512, 128, 512) == 5
    assert L.bmm_select_kernel(1, 64, 1024, 512) == 5
    assert L.bmm_select_kernel(1, 160, 320, 256) == 5
    assert L.bmm_select_kernel(1, 144, 256, 256) == 5
    assert L.bmm_select_kernel(1, 128, 256, 512) == 4
    assert L.bmm_select_kernel(1, 192, 384, 192) == 2
    assert L.bmm_select_kernel(1, 512, 1024, 512) == 2
    for shape in [(1, 1, 1, 2), (1, 8, 16, 16), (1, 256, 512, 256), (1, 1, 2048, 1024),
                  (1, 512, 1024, 512)]:
        assert L.bmm_select_kernel(*shape) in (1, 2, 3, 4, 5)


def pack_km(L, dst=P0, src=P1, batch=1, rows=16, K=32, ld=16, R=16):
    return L.bmm_pack_operand_kmajor(dst, src, batch, rows, K, ld, R, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(R=4), EINVAL, "atom_rows"),
    (dict(rows=24, ld=24, R=16), EINVAL, "multiple of atom_rows"),
    (dict(K=40), EINVAL, "multiple of 16"),
    (dict(ld=8), EINVAL, "ld_src"),
    (dict(ld=20), EALIGN, "multiple of 8"),
    (dict(batch=70000), EINVAL, "too large"),
    (dict(K=(1 << 22) + 16), EINVAL, "too large"),
    (dict(K=1 << 22), EINVAL, "too large"),         # K / 64 would exceed the grid's y limit
    (dict(dst=P0 + 4), EALIGN, "aligned"),
    (dict(dst=0), EINVAL, "null"),
    (dict(dst=P1 + 32), EOVERLAP, "overlaps"),
])
def test_pack_kmajor_rejects(L, kw, code, needle):
    assert pack_km(L, **kw) == code
    assert needle in err(L)


def test_pack_kmajor_empty_is_noop(L):
    assert pack_km(L, dst=0, src=0, batch=0) == 0
    assert pack_km(L, dst=0, src=0, K=0) == 0


def pack_km8(L, dst=P0, src=P1, batch=1, rows=16, K=24, ld=16, R=16):
    return L.bmm_pack_operand_kmajor_k8(dst, src, batch, rows, K, ld, R, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(R=4), EINVAL, "atom_rows"),
    (dict(rows=24, ld=24, R=16), EINVAL, "multiple of atom_rows"),
    (dict(K=20), EINVAL, "multiple of 8"),
    (dict(ld=8), EINVAL, "ld_src"),
    (dict(ld=20), EALIGN, "multiple of 8"),
    (dict(K=1 << 22), EINVAL, "too large"),
    (dict(dst=P0 + 4), EALIGN, "aligned"),
    (dict(dst=P1 + 32), EOVERLAP, "overlaps"),
])
def test_pack_kmajor_k8_rejects(L, kw, code, needle):
    assert pack_km8(L, **kw) == code
    assert needle in err(L)


def test_pack_kmajor_k8_takes_k_multiple_of_8(L):
    # K = 24 is a whole number of 8-deep atoms, which the k = 16 form rejects
    assert pack_km8(L, dst=0, src=0, batch=0, K=24) == 0
    assert pack_km(L, K=24) == EINVAL


def pack_k8(L, dst=P0, src=P1, batch=1, rows=16, K=24, ld=24, R=16):
    return L.bmm_pack_operand_k8(dst, src, batch, rows, K, ld, R, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(R=4), EINVAL, "atom_rows"),
    (dict(K=12, ld=16), EINVAL, "multiple of 8"),
    (dict(ld=16), EINVAL, "ld_src"),
    (dict(ld=28), EALIGN, "multiple of 8"),
    (dict(dst=P0 + 4), EALIGN, "aligned"),
    (dict(dst=P1 + 64), EOVERLAP, "overlaps"),
])
def test_pack_k8_rejects(L, kw, code, needle):
    assert pack_k8(L, **kw) == code
    assert needle in err(L)


def test_pack_k8_accepts_k_multiple_of_8_only_there(L):
    # K = 24 is valid for the k = 8 packer (rejected later, on alignment) but
    # not for the k = 16 one
    assert pack_k8(L, src=P1 + 2) == EALIGN
    assert pack(L, K=24, ld=24) == EINVAL and "multiple of 16" in err(L)
    assert pack_k8(L, dst=0, src=0, K=0, ld=0) == 0


def mma_opts(L, D=P0, A=P1, B=P2, C=None, batch=1, M=2, N=3, K=4, dtype=1, opts=None):
    ref = None if opts is None else ctypes.byref(opts)
    return L.bmm_mma_tile_opts(D, A, B, C, 0.0, batch, M, N, K, dtype, ref, None)


@pytest.mark.parametrize("fields,code,needle", [
    ((4, 0, 0, 1.0, 1.0), EINVAL, "atom_k"),
    ((16, 9, 0, 1.0, 1.0), EINVAL, "kernel"),
    ((8, 0, 2, 1.0, 1.0), EINVAL, "scaled"),
])
def test_mma_opts_rejects_fields(L, fields, code, needle):
    assert mma_opts(L, opts=bmm.MmaOpts(*fields)) == code
    assert needle in err(L)


def test_mma_opts_null_is_plain_call(L):
    assert mma_opts(L, D=P0 + 4) == EALIGN
    assert mma_opts(L, D=0, A=0, B=0, M=0) == 0


def test_mma_opts_sizes_operands_by_atom_k(L):
    # A is (1, 2, 4, 16, atom_k/2) words: 4096 bytes with k = 16, 2048 with
    # k = 8. D placed 3072 bytes into A overlaps it only in the k = 16 layout;
    # C half-overlapping D then fails the k = 8 call before any launch.
    D = P1 + 3072
    k16 = bmm.MmaOpts(16, 1, 0, 1.0, 1.0)
    k8 = bmm.MmaOpts(8, 1, 0, 1.0, 1.0)
    assert mma_opts(L, D=D, C=D + 512, opts=k16) == EOVERLAP and "overlaps A" in err(L)
    assert mma_opts(L, D=D, C=D + 512, opts=k8) == EOVERLAP and "partially overlaps C" in err(L)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(rank=0), EINVAL, "rank"),
    (dict(box=(1, 300)), EINVAL, "box[1]"),
    (dict(oob_fill=2), EINVAL, "oob_fill"),
    (dict(strides=(0, 32)), EINVAL, "overlap itself"),     # 16 columns of 4 B need 64
    (dict(strides=(0, 72)), EALIGN, "multiple of 16"),
])
def test_box_store_rejects_desc(L, kw, code, needle):
    d = box_desc(**kw)
    n = ctypes.c_int64(-7)
    assert L.bmm_box_store(P0, P1, ctypes.byref(d), ctypes.byref(n), None) == code
    assert needle in err(L) and err(L).startswith("box_store")
    assert n.value == -7


def test_box_store_rejects_pointers(L):
    d = box_desc()
    assert L.bmm_box_store(P0 + 8, P1, ctypes.byref(d), None, None) == EALIGN
    assert L.bmm_box_store(0, P1, ctypes.byref(d), None, None) == EINVAL
    assert L.bmm_box_store(P1 + 512, P1, ctypes.byref(d), None, None) == EOVERLAP
    assert L.bmm_box_store(P0, P1, None, None, None) == EINVAL


@pytest.mark.parametrize("etype,eb,needle", [
    (0, 4, "not a bmm_elem_type"),
    (6, 4, "not a bmm_elem_type"),
    (2, 4, "does not match elem_bytes"),     # f16 over 4-byte elements
    (5, 4, "does not match elem_bytes"),
    (1, 8, "does not match elem_bytes"),
])
def test_box_reduce_rejects_types(L, etype, eb, needle):
    d = box_desc(elem_bytes=eb, strides=(1, eb))
    assert L.bmm_box_reduce_add(P0, P1, ctypes.byref(d), etype, None, None) == EINVAL
    assert needle in err(L) and err(L).startswith("box_reduce_add")


def splitk(L, D=P0, A=P1, B=P2, C=None, batch=1, M=2, N=3, K=4, dtype=1, atom_k=16, splits=2,
           ws=P3, ws_bytes=1 << 20):
    return L.bmm_mma_tile_splitk(D, A, B, C, 0.0, batch, M, N, K, dtype, atom_k, splits, ws,
                                 ws_bytes, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(splits=0), EINVAL, "splits"),
    (dict(splits=70000), EINVAL, "splits"),
    (dict(atom_k=4), EINVAL, "atom_k"),
    (dict(dtype=5), EINVAL, "dtype"),
    (dict(K=1 << 18), EINVAL, "K < 2^22"),
    (dict(ws_bytes=100), EINVAL, "workspace_bytes"),
    (dict(ws=0), EINVAL, "workspace is null"),
    (dict(ws=P3 + 8), EALIGN, "workspace"),
    (dict(ws=P1 + 256), EOVERLAP, "workspace overlaps"),
    (dict(ws=P0 + 512), EOVERLAP, "workspace overlaps"),
    (dict(D=P0 + 4), EALIGN, "aligned"),
])
def test_splitk_rejects(L, kw, code, needle):
    assert splitk(L, **kw) == code
    assert needle in err(L) and err(L).startswith("mma_tile_splitk")


def test_splitk_workspace_and_default(L):
    # S = min(splits, ceil(K / 32)): K = 64 values -> 2 steps
    assert L.bmm_mma_splitk_workspace_bytes(1, 2, 3, 4, 16, 5) == 2 * 2 * 3 * 512
    assert L.bmm_mma_splitk_workspace_bytes(1, 2, 3, 4, 8, 5) == 1 * 2 * 3 * 512
    assert L.bmm_mma_splitk_workspace_bytes(1, 2, 3, 0, 16, 5) == 0
    assert L.bmm_mma_splitk_workspace_bytes(1, 2, 3, 4, 16, 0) == EINVAL
    # 1024 x 1024 x 65536: 16 tiles -> 16 splits; 8192^3: 1024 tiles -> 1
    assert L.bmm_splitk_default(1, 64, 128, 4096, 16) == 16
    assert L.bmm_splitk_default(1, 512, 1024, 512, 16) == 1
    assert L.bmm_splitk_default(1, 1, 1, 10, 16) == 1
    # 2048 x 2048: 128 x 128 tiles below K = 16384 (256 tiles, no split), 256 x 256
    # tiles from K = 16384 (64 tiles, 4 splits)
    assert L.bmm_splitk_default(1, 128, 256, 1023, 16) == 1
    assert L.bmm_splitk_default(1, 128, 256, 1024, 16) == 4
    # 8192 x 1024 x 8192: 128 tiles of 256 x 256 below K = 16384 too, 2 splits
    assert L.bmm_splitk_default(1, 512, 128, 512, 16) == 2
    # 512 x 512 x 65536: only 4 tiles of 256 x 256, which 32 splits cannot spread
    # over the chip, so 128 x 128 tiles (16 of them, 16 splits); 1024 x 512 has 8
    # large tiles, and 32 splits of them
    assert L.bmm_splitk_default(1, 32, 64, 4096, 16) == 16
    assert L.bmm_splitk_default(1, 64, 64, 4096, 16) == 32
    # empty problems need no workspace and launch nothing
    assert splitk(L, D=0, A=0, B=0, M=0, ws=0, ws_bytes=0) == 0


def test_kernel_grid_limits(L):
    # AUTO passes over a kernel whose grid the shape would overflow: a skinny
    # shape with more than 65535 batches goes to another kernel
    assert L.bmm_select_kernel(1, 4, 2048, 1024) == 3
    assert L.bmm_select_kernel(70000, 4, 2048, 1024) != 3
    # forcing a kernel past its grid limit is a clear EINVAL, nothing launched
    assert mma(L, batch=70000, M=1, N=1, K=1, kernel=3) == EINVAL and "skinny" in err(L)


@pytest.mark.parametrize("fn", ["mma_tile", "mma_tile_splitk"])
def test_binding_requires_dtype(fn):
    """Packed words carry no element type, so the binding takes no default: a
    call without dtype, or with an unknown one, is refused before any library
    call (the tile operation changes no input type)."""
    import torch
    A = torch.zeros((1, 1, 2, 16, 8), dtype=torch.int32)
    B = torch.zeros((1, 1, 2, 8, 8), dtype=torch.int32)
    f = getattr(bmm, fn)
    with pytest.raises(ValueError, match="dtype is required"):
        f(A, B)
    with pytest.raises(ValueError, match="dtype is required"):
        f(A, B, None, 0.0)
    with pytest.raises(ValueError, match="unknown dtype"):
        f(A, B, None, 0.0, "fp8")


def test_noalloc_refuses_beyond_its_scratch(L):
    """The no-allocation split-K form refuses, before any HIP call, a request
    whose partial sums exceed its static scratch (BMM_ERANGE, a message with
    the sizes), and passes invalid fields to the regular validation."""
    assert bmm.NOALLOC_SCRATCH_BYTES == 64 << 20
    # 1024 x 1024 outputs (4 MiB of D) in 32 splits of 256 steps: 128 MiB of partials
    rc = L.bmm_mma_tile_splitk_noalloc(P0, P1, P2, None, 0.0, 1, 64, 128, 512, 1, 16, 32, None)
    assert rc == ERANGE
    assert "static scratch holds 67108864" in err(L) and "134217728" in err(L)
    # splits out of range: the regular message, no launch
    rc = L.bmm_mma_tile_splitk_noalloc(P0, P1, P2, None, 0.0, 1, 64, 128, 512, 1, 16, 0, None)
    assert rc == EINVAL and "splits" in err(L)
    rc = L.bmm_mma_tile_splitk_noalloc(P0, P1, P2, None, 0.0, 1, 64, 128, 512, 1, 12, 4, None)
    assert rc == EINVAL


def test_noalloc_binding_requires_out_and_dtype():
    import torch
    A = torch.zeros((1, 1, 2, 16, 8), dtype=torch.int32)
    B = torch.zeros((1, 1, 2, 8, 8), dtype=torch.int32)
    with pytest.raises(ValueError, match="dtype is required"):
        bmm.mma_tile_splitk_noalloc(A, B, out=torch.zeros((1, 1, 1, 16, 8)))
    with pytest.raises(ValueError, match="out is required"):
        bmm.mma_tile_splitk_noalloc(A, B, None, 0.0, "bf16")


# (M, N, K, default split-K us, plain entry point us): the sweeps of both forms on
# MI355X (bf16 normal operands, no C; profiles/kernel_choice_sweep.md), with the
# earlier ping-pong tiles and with the 4-wave tiles.
SWEEP_4WAVE = [(128, 128, 256, 16.0, 12.5), (512, 512, 512, 15.9, 12.4), (1024, 1024, 1024, 15.4, 12.6),
               (1536, 1536, 1536, 23.6, 18.4), (2048, 2048, 2048, 30.0, 22.8),
               (2560, 2560, 2560, 46.4, 34.7), (3072, 3072, 3072, 72.4, 59.0),
               (4096, 4096, 1024, 59.4, 36.1), (4096, 4096, 4096, 119.1, 95.6),
               (8192, 8192, 8192, 808.9, 758.1), (1024, 1024, 8192, 30.1, 41.0),
               (2048, 2048, 8192, 77.4, 70.7), (1024, 4096, 4096, 46.0, 39.0),
               (2048, 1024, 4096, 30.1, 36.5), (1024, 1024, 65536, 113.6, 337.1),
               (512, 512, 65536, 48.7, 270.4), (16, 1024, 1024, 17.3, 12.6), (64, 2048, 2048, 15.8, 13.7),
               (256, 4096, 4096, 22.4, 23.9), (512, 2048, 2048, 20.3, 13.3), (64, 8192, 8192, 27.5, 44.1),
               (32, 16384, 4096, 26.4, 28.9), (16, 16384, 16384, 105.7, 87.0),
               (8192, 1024, 8192, 113.9, 102.3), (1024, 8192, 8192, 114.5, 102.7),
               (2304, 2304, 4096, 60.1, 46.8), (3072, 2048, 4096, 63.6, 48.5),
               (2816, 2816, 4096, 71.3, 54.1)]
SWEEP = [(128, 128, 256, 16.9, 12.8), (512, 512, 512, 17.2, 13.5), (1024, 1024, 1024, 17.5, 13.5),
         (1536, 1536, 1536, 22.7, 18.2), (2048, 2048, 2048, 30.6, 24.2),
         (2560, 2560, 2560, 47.0, 35.9), (3072, 3072, 3072, 70.8, 59.6),
         (4096, 4096, 1024, 57.8, 38.4), (4096, 4096, 4096, 124.5, 103.9),
         (8192, 8192, 8192, 844.6, 777.7), (1024, 1024, 8192, 30.0, 39.7),
         (2048, 2048, 8192, 77.1, 71.0), (1024, 4096, 4096, 45.7, 39.2),
         (2048, 1024, 4096, 29.1, 34.0), (1024, 1024, 65536, 123.3, 335.1),
         (512, 512, 65536, 48.6, 272.4), (16, 1024, 1024, 14.7, 12.7), (64, 2048, 2048, 15.3, 13.6),
         (256, 4096, 4096, 22.0, 24.0), (512, 2048, 2048, 20.2, 13.1), (64, 8192, 8192, 27.4, 43.7),
         (32, 16384, 4096, 26.3, 28.8), (16, 16384, 16384, 106.8, 85.7),
         (8192, 1024, 8192, 121.4, 112.3), (1024, 8192, 8192, 121.8, 112.5),
         (2304, 2304, 4096, 59.9, 47.4), (3072, 2048, 4096, 64.1, 51.1),
         (2816, 2816, 4096, 73.6, 59.6), (2304, 2048, 4096, 61.6, 51.0),
         (2048, 2304, 4096, 59.9, 47.8), (2560, 2048, 4096, 61.8, 48.5),
         (2304, 2304, 2304, 41.6, 31.2), (2048, 2560, 8192, 109.0, 87.5)]


@pytest.mark.parametrize("M,N,K,split_us,plain_us", SWEEP + SWEEP_4WAVE)
def test_splitk_suggested_matches_the_sweep(L, M, N, K, split_us, plain_us):
    """bmm_splitk_suggested says to split exactly where the measured default
    split-K form beat the plain entry point, and then gives that split count."""
    s = L.bmm_splitk_suggested(1, M // 16, N // 8, K // 16, 16)
    assert (s > 1) == (split_us < plain_us), (M, N, K, s)
    if s > 1:
        assert s == L.bmm_splitk_default(1, M // 16, N // 8, K // 16, 16)
    assert bmm.splitk_suggested(1, M // 16, N // 8, K // 16) == s


def test_splitk_suggested_rejects_invalid(L):
    assert L.bmm_splitk_suggested(-1, 1, 1, 1, 16) == EINVAL
    assert L.bmm_splitk_suggested(1, 1, 1, 1, 12) == EINVAL
    assert L.bmm_splitk_suggested(1, 0, 0, 0, 16) == 1
