"""Python binding of libbmm.so: the tiled f16/bf16 multiply-accumulate
D = A * B^T + C on MI355X (gfx950).

Argument marshalling only. Each function takes torch tensors on the GPU, reads
their pointers, extents and the current torch stream, and calls the C ABI of
``include/bmm.h`` with the same name; every step of the computation runs in
the library's HIP kernels. If the library is not built, every call raises;
there is no other code path.

Layouts (mma.sync page of the TVM tirx tile-op documentation, "Operand
coordinates and ownership"):
    A packed: (batch, M/16, K/16, 16, 8) 32-bit words
    B packed: (batch, N/8,  K/16,  8, 8) 32-bit words
    C, D:     (batch, M/16, N/8,  16, 8) float32
or, with an atom K of 8 (the m16n8k8 form), A (batch, M/16, K/8, 16, 4) and
B (batch, N/8, K/8, 8, 4). Packed words are held in int32 tensors (bit
containers).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["BmmError", "pack_operand", "pack_operand_kmajor", "box_copy", "box_store",
           "box_reduce_add", "mma_tile", "mma_tile_splitk", "mma_tile_splitk_noalloc",
           "splitk_default", "splitk_suggested", "NOALLOC_SCRATCH_BYTES",
           "splitk_workspace_bytes", "select_kernel", "library_path", "KERNELS", "MmaOpts",
           "ELEM_TYPES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbmm.so")

BMM_F16, BMM_BF16 = 0, 1
_DTYPES = {"f16": BMM_F16, "float16": BMM_F16, torch.float16: BMM_F16,
           "bf16": BMM_BF16, "bfloat16": BMM_BF16, torch.bfloat16: BMM_BF16}
KERNELS = {"auto": 0, "direct": 1, "tiled": 2, "skinny": 3, "tiled128": 4, "tiled256x128": 5}
NOALLOC_SCRATCH_BYTES = 64 << 20   # BMM_NOALLOC_SCRATCH_BYTES
ELEM_TYPES = {"f32": 1, "f16": 2, "bf16": 3, "i32": 4, "i64": 5}
KERNEL_NAMES = {v: k for k, v in KERNELS.items()}


class BmmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"bmm error {code}: {msg}")
        self.code = code


class BoxDesc(ctypes.Structure):
    _fields_ = [
        ("rank", ctypes.c_int32),
        ("elem_bytes", ctypes.c_int32),
        ("dims", ctypes.c_int64 * 5),
        ("strides", ctypes.c_int64 * 5),
        ("box", ctypes.c_int32 * 5),
        ("coords", ctypes.c_int64 * 5),
        ("n_repeat", ctypes.c_int32),
        ("coord_step", ctypes.c_int64 * 5),
        ("swizzle", ctypes.c_int32),
        ("oob_fill", ctypes.c_int32),
    ]


class MmaOpts(ctypes.Structure):
    _fields_ = [
        ("atom_k", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
        ("scaled", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("beta", ctypes.c_float),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libbmm.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built: run `python -m bf16_matrix_multiply_amd.build` "
                "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(_LIB_PATH)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.bmm_abi_version.restype = ctypes.c_int
        L.bmm_last_error.restype = ctypes.c_char_p
        L.bmm_pack_operand.argtypes = [p, p, i64, i64, i64, i64, i32, p]
        L.bmm_pack_operand_kmajor.argtypes = [p, p, i64, i64, i64, i64, i32, p]
        L.bmm_pack_operand_k8.argtypes = [p, p, i64, i64, i64, i64, i32, p]
        L.bmm_pack_operand_kmajor_k8.argtypes = [p, p, i64, i64, i64, i64, i32, p]
        L.bmm_mma_tile_opts.argtypes = [p, p, p, p, ctypes.c_float, i64, i64, i64, i64,
                                        ctypes.c_int, ctypes.POINTER(MmaOpts), p]
        L.bmm_box_copy.argtypes = [p, p, ctypes.POINTER(BoxDesc), ctypes.POINTER(i64), p]
        L.bmm_mma_tile.argtypes = [p, p, p, p, ctypes.c_float, i64, i64, i64, i64, ctypes.c_int,
                                   p]
        L.bmm_mma_tile_with.argtypes = [p, p, p, p, ctypes.c_float, i64, i64, i64, i64,
                                        ctypes.c_int, i32, p]
        L.bmm_mma_tile_scaled.argtypes = [p, p, p, p, ctypes.c_float, ctypes.c_float,
                                          ctypes.c_float, i64, i64, i64, i64, ctypes.c_int, i32, p]
        L.bmm_select_kernel.argtypes = [i64, i64, i64, i64]
        L.bmm_box_store.argtypes = [p, p, ctypes.POINTER(BoxDesc), ctypes.POINTER(i64), p]
        L.bmm_box_reduce_add.argtypes = [p, p, ctypes.POINTER(BoxDesc), i32,
                                         ctypes.POINTER(i64), p]
        L.bmm_mma_tile_splitk.argtypes = [p, p, p, p, ctypes.c_float, i64, i64, i64, i64,
                                          ctypes.c_int, i32, i32, p, i64, p]
        L.bmm_mma_tile_splitk_noalloc.argtypes = [p, p, p, p, ctypes.c_float, i64, i64, i64,
                                                  i64, ctypes.c_int, i32, i32, p]
        L.bmm_mma_splitk_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32]
        L.bmm_mma_splitk_workspace_bytes.restype = i64
        L.bmm_splitk_default.argtypes = [i64, i64, i64, i64, i32]
        L.bmm_splitk_suggested.argtypes = [i64, i64, i64, i64, i32]
        for f in (L.bmm_pack_operand, L.bmm_pack_operand_kmajor, L.bmm_pack_operand_k8,
                  L.bmm_pack_operand_kmajor_k8,
                  L.bmm_box_copy, L.bmm_mma_tile, L.bmm_mma_tile_with, L.bmm_mma_tile_scaled,
                  L.bmm_mma_tile_opts, L.bmm_select_kernel, L.bmm_box_store,
                  L.bmm_box_reduce_add, L.bmm_mma_tile_splitk, L.bmm_mma_tile_splitk_noalloc,
                  L.bmm_splitk_default, L.bmm_splitk_suggested):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _dtype_code(dtype, fn: str) -> int:
    """The C ABI's element type for ``dtype``. Packed words carry no type, so the
    caller must name it: a missing or unknown dtype is an error, never a default
    (the tile operation changes no input type)."""
    if dtype is None:
        raise ValueError(f"{fn}: dtype is required ('f16' or 'bf16'): packed words carry no type")
    try:
        return _DTYPES[dtype]
    except (KeyError, TypeError):
        raise ValueError(f"{fn}: unknown dtype {dtype!r}; expected 'f16' or 'bf16'") from None


def _check(rc: int):
    if rc < 0:
        raise BmmError(rc, lib().bmm_last_error().decode())
    return rc


def _stream(t: torch.Tensor | None = None):
    if t is not None and not t.is_cuda:
        raise ValueError("bmm operates on GPU tensors only")
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("bmm operates on GPU tensors only")


def pack_operand(x: torch.Tensor, atom_rows: int, K: int | None = None,
                 out: torch.Tensor | None = None, atom_k: int = 16) -> torch.Tensor:
    """Row-major (batch, rows, ld) or (rows, ld) 16-bit tensor -> packed words
    (batch, rows/R, K/atom_k, R, atom_k/2) int32 (R = atom_rows: 16 for A, 8
    for B; atom_k 16, or 8 for bmm_pack_operand_k8).

    The source must have unit innermost stride and rows ``ld`` elements apart,
    with batches ``rows * ld`` apart; K (default ld) may be smaller than ld."""
    if atom_k not in (16, 8):
        raise ValueError("pack_operand: atom_k must be 16 or 8")
    _require_cuda(x)
    if x.element_size() != 2:
        raise ValueError("pack_operand takes 16-bit (f16/bf16 bit) tensors")
    if x.dim() == 2:
        x = x.unsqueeze(0)
    batch, rows, ld = x.shape
    # (an empty source has nothing to pack; torch gives it arbitrary strides)
    if x.numel() and (x.stride(2) != 1 or (rows > 1 and x.stride(1) != ld) or
                      (batch > 1 and x.stride(0) != rows * ld)):
        raise ValueError("pack_operand: source must be (batch, rows, ld) with dense strides")
    K = ld if K is None else K
    shape = (batch, rows // atom_rows, K // atom_k, atom_rows, atom_k // 2)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=x.device)
    elif tuple(out.shape) != shape or not out.is_contiguous() or out.element_size() != 4:
        raise ValueError(f"pack_operand: out must be a contiguous 32-bit tensor of shape {shape}")
    fn = lib().bmm_pack_operand if atom_k == 16 else lib().bmm_pack_operand_k8
    _check(fn(_ptr(out), _ptr(x), batch, rows, K, ld, atom_rows, _stream(x)))
    return out


def pack_operand_kmajor(xt: torch.Tensor, atom_rows: int, rows: int | None = None,
                        out: torch.Tensor | None = None, atom_k: int = 16) -> torch.Tensor:
    """K-major (batch, K, ld) or (K, ld) 16-bit tensor holding element (row, k)
    at [b, k, row] -> packed words (batch, rows/R, K/atom_k, R, atom_k/2) int32,
    the same words pack_operand gives for the row-major matrix (atom_k 16, or 8
    for bmm_pack_operand_kmajor_k8). rows defaults to ld."""
    if atom_k not in (16, 8):
        raise ValueError("pack_operand_kmajor: atom_k must be 16 or 8")
    _require_cuda(xt)
    if xt.element_size() != 2:
        raise ValueError("pack_operand_kmajor takes 16-bit (f16/bf16 bit) tensors")
    if xt.dim() == 2:
        xt = xt.unsqueeze(0)
    batch, K, ld = xt.shape
    if xt.numel() and (xt.stride(2) != 1 or (K > 1 and xt.stride(1) != ld) or
                       (batch > 1 and xt.stride(0) != K * ld)):
        raise ValueError("pack_operand_kmajor: source must be (batch, K, ld) with dense strides")
    rows = ld if rows is None else rows
    shape = (batch, rows // atom_rows, K // atom_k, atom_rows, atom_k // 2)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=xt.device)
    elif tuple(out.shape) != shape or not out.is_contiguous() or out.element_size() != 4:
        raise ValueError(f"pack_operand_kmajor: out must be a contiguous 32-bit tensor of shape {shape}")
    fn = lib().bmm_pack_operand_kmajor if atom_k == 16 else lib().bmm_pack_operand_kmajor_k8
    _check(fn(_ptr(out), _ptr(xt), batch, rows, K, ld, atom_rows, _stream(xt)))
    return out


def box_copy(src: torch.Tensor, box, coords, n_repeat: int = 1, coord_step=None,
             swizzle: int = 0, dims=None, strides=None, oob_fill: int = 0,
             out: torch.Tensor | None = None):
    """Stage boxes of ``src`` through LDS; return ((n_repeat, *box) image, bytes).

    dims/strides default to ``src``'s own extents and byte strides (outer to
    inner); strides are in bytes."""
    _require_cuda(src)
    d = _box_desc(src, box, coords, n_repeat, coord_step, swizzle, dims, strides, oob_fill)
    shape = (n_repeat, *box)
    if out is None:
        out = torch.empty(shape, dtype=src.dtype, device=src.device)
    nbytes = ctypes.c_int64(-1)
    _check(lib().bmm_box_copy(_ptr(out), _ptr(src), ctypes.byref(d), ctypes.byref(nbytes),
                              _stream(src)))
    return out, nbytes.value


def _box_desc(t: torch.Tensor, box, coords, n_repeat, coord_step, swizzle, dims, strides,
              oob_fill=0) -> BoxDesc:
    rank = len(box)
    dims = list(t.shape) if dims is None else list(dims)
    strides = [s * t.element_size() for s in t.stride()] if strides is None else list(strides)
    coord_step = [0] * rank if coord_step is None else list(coord_step)
    if not (len(dims) == len(strides) == len(coords) == len(coord_step) == rank):
        raise ValueError("box: box, coords, coord_step, dims and strides need one entry "
                         "per dimension")
    d = BoxDesc()
    d.rank, d.elem_bytes = rank, t.element_size()
    for i in range(rank):
        d.dims[i], d.strides[i], d.box[i] = dims[i], strides[i], box[i]
        d.coords[i], d.coord_step[i] = coords[i], coord_step[i]
    d.n_repeat, d.swizzle, d.oob_fill = n_repeat, swizzle, oob_fill
    return d


def box_store(dst: torch.Tensor, image: torch.Tensor, box, coords, n_repeat: int = 1,
              coord_step=None, swizzle: int = 0, dims=None, strides=None) -> int:
    """Write the compact (n_repeat, *box) ``image`` into ``dst``'s boxes (in place;
    elements outside the tensor are skipped). Returns the image bytes read."""
    _require_cuda(dst, image)
    if image.element_size() != dst.element_size() or not image.is_contiguous():
        raise ValueError("box_store: image must be contiguous with dst's element size")
    d = _box_desc(dst, box, coords, n_repeat, coord_step, swizzle, dims, strides)
    nbytes = ctypes.c_int64(-1)
    _check(lib().bmm_box_store(_ptr(dst), _ptr(image), ctypes.byref(d), ctypes.byref(nbytes),
                               _stream(dst)))
    return nbytes.value


def box_reduce_add(dst: torch.Tensor, image: torch.Tensor, box, coords, elem_type: str,
                   n_repeat: int = 1, coord_step=None, swizzle: int = 0, dims=None,
                   strides=None) -> int:
    """Add the compact (n_repeat, *box) ``image`` into ``dst``'s boxes (in place),
    one rounding per add in ``elem_type`` ("f32", "f16", "bf16", "i32", "i64")."""
    _require_cuda(dst, image)
    if image.element_size() != dst.element_size() or not image.is_contiguous():
        raise ValueError("box_reduce_add: image must be contiguous with dst's element size")
    d = _box_desc(dst, box, coords, n_repeat, coord_step, swizzle, dims, strides)
    nbytes = ctypes.c_int64(-1)
    _check(lib().bmm_box_reduce_add(_ptr(dst), _ptr(image), ctypes.byref(d), ELEM_TYPES[elem_type],
                                    ctypes.byref(nbytes), _stream(dst)))
    return nbytes.value


def splitk_workspace_bytes(batch, M_rep, N_rep, K_rep, atom_k, splits) -> int:
    return _check(lib().bmm_mma_splitk_workspace_bytes(batch, M_rep, N_rep, K_rep, atom_k,
                                                       splits))


def splitk_default(batch, M_rep, N_rep, K_rep, atom_k=16) -> int:
    return _check(lib().bmm_splitk_default(batch, M_rep, N_rep, K_rep, atom_k))


def splitk_suggested(batch, M_rep, N_rep, K_rep, atom_k=16) -> int:
    """bmm_splitk_suggested: the split count when mma_tile_splitk is expected
    to beat mma_tile for this shape, else 1."""
    return _check(lib().bmm_splitk_suggested(batch, M_rep, N_rep, K_rep, atom_k))


def mma_tile_splitk(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor | None = None,
                    c: float = 0.0, dtype=None, splits: int | None = None,
                    out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Split-K form: D = (((C + P_0) + P_1) + ...), P_s the partial sums of
    balanced ranges of 32-value K steps (bmm_mma_tile_splitk). ``splits``
    defaults to bmm_splitk_default; ``workspace`` (float32, at least
    bmm_mma_splitk_workspace_bytes) is allocated here when not given. ``dtype``
    ('f16' or 'bf16') is required."""
    dt = _dtype_code(dtype, "mma_tile_splitk")
    _require_cuda(A, B, C, out, workspace)
    if A.dim() != 5 or B.dim() != 5 or A.shape[3] != 16 or B.shape[3] != 8 or \
            A.shape[4] not in (8, 4) or B.shape[4] != A.shape[4]:
        raise ValueError("mma_tile_splitk: A must be (batch, M_rep, K_rep, 16, w) and B "
                         "(batch, N_rep, K_rep, 8, w) packed words, w = 8 or 4")
    atom_k = 2 * A.shape[4]
    batch, M_rep, K_rep = A.shape[:3]
    N_rep = B.shape[1]
    if B.shape[0] != batch or B.shape[2] != K_rep:
        raise ValueError("mma_tile_splitk: A and B disagree on batch or K_rep")
    for t, name in ((A, "A"), (B, "B")):
        if not t.is_contiguous() or t.element_size() != 4:
            raise ValueError(f"mma_tile_splitk: {name} must be a contiguous 32-bit tensor")
    shape = (batch, M_rep, N_rep, 16, 8)
    if C is not None and (tuple(C.shape) != shape or C.dtype != torch.float32
                          or not C.is_contiguous()):
        raise ValueError(f"mma_tile_splitk: C must be a contiguous float32 tensor of shape {shape}")
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=A.device)
    elif tuple(out.shape) != shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError(f"mma_tile_splitk: out must be a contiguous float32 tensor of shape {shape}")
    if splits is None:
        splits = splitk_default(batch, M_rep, N_rep, K_rep, atom_k)
    need = splitk_workspace_bytes(batch, M_rep, N_rep, K_rep, atom_k, splits)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=A.device)
    elif not workspace.is_contiguous():
        raise ValueError("mma_tile_splitk: workspace must be contiguous")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().bmm_mma_tile_splitk(_ptr(out), _ptr(A), _ptr(B), _ptr(C), float(c), batch, M_rep,
                                     N_rep, K_rep, dt, atom_k, splits,
                                     _ptr(workspace), ws_bytes, _stream(A)))
    return out


def mma_tile_splitk_noalloc(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor | None = None,
                            c: float = 0.0, dtype=None, splits: int | None = None,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """bmm_mma_tile_splitk_noalloc: the split-K form with its partial sums in
    the library's static per-device scratch (NOALLOC_SCRATCH_BYTES) instead of
    a workspace. ``out`` must be given: this call allocates nothing. Calls
    that overlap on one device race on the scratch."""
    dt = _dtype_code(dtype, "mma_tile_splitk_noalloc")
    if out is None:
        raise ValueError("mma_tile_splitk_noalloc: out is required (this form allocates nothing)")
    _require_cuda(A, B, C, out)
    if A.dim() != 5 or B.dim() != 5 or A.shape[3] != 16 or B.shape[3] != 8 or \
            A.shape[4] not in (8, 4) or B.shape[4] != A.shape[4]:
        raise ValueError("mma_tile_splitk_noalloc: A must be (batch, M_rep, K_rep, 16, w) and B "
                         "(batch, N_rep, K_rep, 8, w) packed words, w = 8 or 4")
    atom_k = 2 * A.shape[4]
    batch, M_rep, K_rep = A.shape[:3]
    N_rep = B.shape[1]
    if B.shape[0] != batch or B.shape[2] != K_rep:
        raise ValueError("mma_tile_splitk_noalloc: A and B disagree on batch or K_rep")
    for t, name in ((A, "A"), (B, "B")):
        if not t.is_contiguous() or t.element_size() != 4:
            raise ValueError(f"mma_tile_splitk_noalloc: {name} must be a contiguous 32-bit tensor")
    shape = (batch, M_rep, N_rep, 16, 8)
    for t, name in ((C, "C"), (out, "out")):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32
                              or not t.is_contiguous()):
            raise ValueError(f"mma_tile_splitk_noalloc: {name} must be a contiguous float32 "
                             f"tensor of shape {shape}")
    if splits is None:
        splits = splitk_default(batch, M_rep, N_rep, K_rep, atom_k)
    _check(lib().bmm_mma_tile_splitk_noalloc(_ptr(out), _ptr(A), _ptr(B), _ptr(C), float(c),
                                             batch, M_rep, N_rep, K_rep, dt, atom_k, splits,
                                             _stream(A)))
    return out


def mma_tile(A: torch.Tensor, B: torch.Tensor, C: torch.Tensor | None = None,
             c: float = 0.0, dtype=None, out: torch.Tensor | None = None,
             kernel: str = "auto", alpha: float | None = None,
             beta: float | None = None) -> torch.Tensor:
    """D = A * B^T + C over packed operands; returns D (batch, M/16, N/8, 16, 8).

    C is a float32 tensor in D's layout or None (then every element starts
    from the scalar ``c``). ``out`` may be C itself (in place). With alpha or
    beta given, the alpha/beta form runs instead (bmm_mma_tile_scaled):
    D = fma(alpha, A * B^T, beta * C), the product accumulated from zero.
    Operands packed with an atom K of 8 ((..., 16, 4) and (..., 8, 4) words)
    go through bmm_mma_tile_opts with atom_k = 8. ``dtype`` ('f16' or 'bf16',
    the type both operands were packed from) is required."""
    dt = _dtype_code(dtype, "mma_tile")
    _require_cuda(A, B, C, out)
    if A.dim() != 5 or B.dim() != 5 or A.shape[3] != 16 or B.shape[3] != 8 or \
            A.shape[4] not in (8, 4) or B.shape[4] != A.shape[4]:
        raise ValueError("mma_tile: A must be (batch, M_rep, K_rep, 16, w) and B "
                         "(batch, N_rep, K_rep, 8, w) packed words, w = 8 (k = 16) or 4 (k = 8)")
    atom_k = 2 * A.shape[4]
    batch, M_rep, K_rep = A.shape[:3]
    if B.shape[0] != batch or B.shape[2] != K_rep:
        raise ValueError("mma_tile: A and B disagree on batch or K_rep")
    N_rep = B.shape[1]
    shape = (batch, M_rep, N_rep, 16, 8)
    for t, name in ((A, "A"), (B, "B")):
        if not t.is_contiguous() or t.element_size() != 4:
            raise ValueError(f"mma_tile: {name} must be a contiguous 32-bit tensor")
    if C is not None and (tuple(C.shape) != shape or C.dtype != torch.float32
                          or not C.is_contiguous()):
        raise ValueError(f"mma_tile: C must be a contiguous float32 tensor of shape {shape}")
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=A.device)
    elif tuple(out.shape) != shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError(f"mma_tile: out must be a contiguous float32 tensor of shape {shape}")
    if atom_k == 8:
        scaled = not (alpha is None and beta is None)
        opts = MmaOpts(8, KERNELS[kernel], int(scaled), 1.0 if alpha is None else float(alpha),
                       1.0 if beta is None else float(beta))
        _check(lib().bmm_mma_tile_opts(_ptr(out), _ptr(A), _ptr(B), _ptr(C), float(c), batch,
                                       M_rep, N_rep, K_rep, dt, ctypes.byref(opts),
                                       _stream(A)))
    elif alpha is None and beta is None:
        _check(lib().bmm_mma_tile_with(_ptr(out), _ptr(A), _ptr(B), _ptr(C), float(c), batch,
                                       M_rep, N_rep, K_rep, dt, KERNELS[kernel],
                                       _stream(A)))
    else:
        _check(lib().bmm_mma_tile_scaled(
            _ptr(out), _ptr(A), _ptr(B), _ptr(C), float(c), 1.0 if alpha is None else float(alpha),
            1.0 if beta is None else float(beta), batch, M_rep, N_rep, K_rep, dt,
            KERNELS[kernel], _stream(A)))
    return out


def select_kernel(batch: int, M_rep: int, N_rep: int, K_rep: int) -> str:
    return KERNEL_NAMES[_check(lib().bmm_select_kernel(batch, M_rep, N_rep, K_rep))]
