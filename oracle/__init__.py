"""CPU oracle for D = A * B^T + C over the packed f16/bf16 layouts.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP product path
never imports, links or calls it, and it shares no code with that path.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc; see the header
of that file for the passages it follows). This module only compiles it and
marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, BF16 = 0, 1
_DTYPES = {"f16": F16, "bf16": BF16, F16: F16, BF16: BF16}

# -ffp-contract=off: every a*b and every + is its own IEEE operation, exactly
# as the C source reads. No -ffast-math.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile liboracle.so in place with gcc and return its path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = f"{_LIB_PATH}.{os.getpid()}.tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Oracle:
    """ctypes handle on one build of oracle.c (the default build, or a test's
    deliberately mutated copy)."""

    def __init__(self, path: str = _LIB_PATH):
        L = ctypes.CDLL(path)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_h2f.restype = ctypes.c_float
        L.oracle_h2f.argtypes = [ctypes.c_uint16, ctypes.c_int]
        L.oracle_h2f_array.argtypes = [p, p, i64, ctypes.c_int]
        L.oracle_pack.argtypes = [p, p, i64, i64, i64, i64, i64]
        L.oracle_unpack.argtypes = [p, p, i64, i64, i64, i64]
        L.oracle_pack_kmajor.argtypes = [p, p, i64, i64, i64, i64, i64]
        L.oracle_pack_k8.argtypes = [p, p, i64, i64, i64, i64, i64]
        L.oracle_mma_k.argtypes = [p, p, p, p, ctypes.c_float, i64, i64, i64, i64, i64,
                                   ctypes.c_int]
        L.oracle_mma_sampled_k.argtypes = [p, p, i64, p, p, p, ctypes.c_float, i64, i64, i64,
                                           i64, i64, ctypes.c_int]
        L.oracle_mma.argtypes = [p, p, p, p, ctypes.c_float, i64, i64, i64, i64, ctypes.c_int]
        L.oracle_mma_sampled.argtypes = [p, p, i64, p, p, p, ctypes.c_float, i64, i64, i64,
                                         i64, ctypes.c_int]
        L.oracle_mma_scaled.argtypes = [p, p, p, p, ctypes.c_float, ctypes.c_float,
                                        ctypes.c_float, i64, i64, i64, i64, ctypes.c_int]
        L.oracle_box_copy.restype = i64
        L.oracle_box_copy.argtypes = [p, p, i32, i32, p, p, p, p, i32, p]
        L.oracle_box_store.restype = i64
        L.oracle_box_store.argtypes = [p, p, i32, i32, p, p, p, p, i32, p, i32, i32]
        L.oracle_mma_splitk.argtypes = [p, p, p, p, ctypes.c_float, i64, i64, i64, i64, i64,
                                        i64, ctypes.c_int]
        L.oracle_mma_splitk_sampled.argtypes = [p, p, i64, p, p, p, ctypes.c_float, i64, i64,
                                                i64, i64, i64, i64, ctypes.c_int]
        self.L = L

    def threads(self) -> int:
        return int(self.L.oracle_threads())

    def h2f(self, bits: np.ndarray, dtype) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, np.float32)
        self.L.oracle_h2f_array(_ptr(out), _ptr(bits), bits.size, _DTYPES[dtype])
        return out

    def pack(self, x: np.ndarray, atom_rows: int, K: int | None = None) -> np.ndarray:
        """(batch, rows, ld) uint16 -> (batch, rows/R, K/16, R, 8) uint32 words.

        ``K`` defaults to the last extent; a smaller K packs a row-padded source.
        """
        x = np.ascontiguousarray(x, dtype=np.uint16)
        if x.ndim == 2:
            x = x[None]
        batch, rows, ld = x.shape
        K = ld if K is None else K
        out = np.empty((batch, rows // atom_rows, K // 16, atom_rows, 8), np.uint32)
        rc = self.L.oracle_pack(_ptr(out), _ptr(x), batch, rows, K, ld, atom_rows)
        if rc != 0:
            raise ValueError("oracle_pack rejected its arguments")
        return out

    def pack_kmajor(self, x: np.ndarray, atom_rows: int, rows: int | None = None) -> np.ndarray:
        """K-major (batch, K, ld) uint16 (element (row, k) at [b, k, row]) ->
        (batch, rows/R, K/16, R, 8) uint32 words; rows defaults to ld."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        if x.ndim == 2:
            x = x[None]
        batch, K, ld = x.shape
        rows = ld if rows is None else rows
        out = np.empty((batch, rows // atom_rows, K // 16, atom_rows, 8), np.uint32)
        rc = self.L.oracle_pack_kmajor(_ptr(out), _ptr(x), batch, rows, K, ld, atom_rows)
        if rc != 0:
            raise ValueError("oracle_pack_kmajor rejected its arguments")
        return out

    def pack_k8(self, x: np.ndarray, atom_rows: int) -> np.ndarray:
        """(batch, rows, K) uint16 -> (batch, rows/R, K/8, R, 4) uint32 words
        (atom K = 8, the m16n8k8 layout)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        if x.ndim == 2:
            x = x[None]
        batch, rows, K = x.shape
        out = np.empty((batch, rows // atom_rows, K // 8, atom_rows, 4), np.uint32)
        if self.L.oracle_pack_k8(_ptr(out), _ptr(x), batch, rows, K, K, atom_rows) != 0:
            raise ValueError("oracle_pack_k8 rejected its arguments")
        return out

    def mma_k8(self, A, B, C, c, dtype) -> np.ndarray:
        """D = A * B^T + C over k=8-atom operands (batch, M/16, K/8, 16, 4) and
        (batch, N/8, K/8, 8, 4)."""
        A = np.ascontiguousarray(A, np.uint32)
        B = np.ascontiguousarray(B, np.uint32)
        C = None if C is None else np.ascontiguousarray(C, np.float32)
        batch, M_rep, K_rep, ra, wa = A.shape
        b2, N_rep, K2, rb, wb = B.shape
        assert (ra, wa, rb, wb) == (16, 4, 8, 4) and b2 == batch and K2 == K_rep
        D = np.empty((batch, M_rep, N_rep, 16, 8), np.float32)
        rc = self.L.oracle_mma_k(_ptr(D), _ptr(A), _ptr(B), _ptr(C), float(c), batch, M_rep,
                                 N_rep, K_rep, 8, _DTYPES[dtype])
        if rc != 0:
            raise ValueError("oracle_mma_k rejected its arguments")
        return D

    def mma_k8_sampled(self, A, B, C, c, dtype, idx) -> np.ndarray:
        A = np.ascontiguousarray(A, np.uint32)
        B = np.ascontiguousarray(B, np.uint32)
        C = None if C is None else np.ascontiguousarray(C, np.float32)
        batch, M_rep, K_rep = A.shape[:3]
        N_rep = B.shape[1]
        idx = np.ascontiguousarray(idx, np.int64).reshape(-1, 3)
        out = np.empty(len(idx), np.float32)
        rc = self.L.oracle_mma_sampled_k(_ptr(out), _ptr(idx), len(idx), _ptr(A), _ptr(B),
                                         _ptr(C), float(c), batch, M_rep, N_rep, K_rep, 8,
                                         _DTYPES[dtype])
        if rc != 0:
            raise ValueError("oracle_mma_sampled_k rejected its arguments")
        return out

    def unpack(self, p: np.ndarray, atom_rows: int) -> np.ndarray:
        p = np.ascontiguousarray(p, dtype=np.uint32)
        batch, rows_rep, K_rep, R, w = p.shape
        assert R == atom_rows and w == 8
        out = np.empty((batch, rows_rep * R, K_rep * 16), np.uint16)
        if self.L.oracle_unpack(_ptr(out), _ptr(p), batch, rows_rep * R, K_rep * 16, R) != 0:
            raise ValueError("oracle_unpack rejected its arguments")
        return out

    def mma(self, A: np.ndarray, B: np.ndarray, C: np.ndarray | None, c: float,
            dtype) -> np.ndarray:
        """Full D = A * B^T + C in the (batch, M_rep, N_rep, 16, 8) float32 layout."""
        A = np.ascontiguousarray(A, np.uint32)
        B = np.ascontiguousarray(B, np.uint32)
        C = None if C is None else np.ascontiguousarray(C, np.float32)
        batch, M_rep, N_rep, K_rep = _mma_shapes(A, B, C)
        D = np.empty((batch, M_rep, N_rep, 16, 8), np.float32)
        rc = self.L.oracle_mma(_ptr(D), _ptr(A), _ptr(B), _ptr(C), float(c), batch, M_rep,
                               N_rep, K_rep, _DTYPES[dtype])
        if rc != 0:
            raise ValueError("oracle_mma rejected its arguments")
        return D

    def mma_scaled(self, A, B, C, c, alpha, beta, dtype) -> np.ndarray:
        """D = fma(alpha, A * B^T (from zero), fl(beta * C)), full output."""
        A = np.ascontiguousarray(A, np.uint32)
        B = np.ascontiguousarray(B, np.uint32)
        C = None if C is None else np.ascontiguousarray(C, np.float32)
        batch, M_rep, N_rep, K_rep = _mma_shapes(A, B, C)
        D = np.empty((batch, M_rep, N_rep, 16, 8), np.float32)
        rc = self.L.oracle_mma_scaled(_ptr(D), _ptr(A), _ptr(B), _ptr(C), float(c), float(alpha),
                                      float(beta), batch, M_rep, N_rep, K_rep, _DTYPES[dtype])
        if rc != 0:
            raise ValueError("oracle_mma_scaled rejected its arguments")
        return D

    def mma_sampled(self, A, B, C, c, dtype, idx: np.ndarray) -> np.ndarray:
        """D[b, m, n] for each row (b, m, n) of ``idx`` (logical coordinates)."""
        A = np.ascontiguousarray(A, np.uint32)
        B = np.ascontiguousarray(B, np.uint32)
        C = None if C is None else np.ascontiguousarray(C, np.float32)
        batch, M_rep, N_rep, K_rep = _mma_shapes(A, B, C)
        idx = np.ascontiguousarray(idx, np.int64).reshape(-1, 3)
        out = np.empty(len(idx), np.float32)
        rc = self.L.oracle_mma_sampled(_ptr(out), _ptr(idx), len(idx), _ptr(A), _ptr(B),
                                       _ptr(C), float(c), batch, M_rep, N_rep, K_rep,
                                       _DTYPES[dtype])
        if rc != 0:
            raise ValueError("oracle_mma_sampled rejected its arguments")
        return out

    def bound(self, A, B, C, c, dtype, idx: np.ndarray | None = None) -> np.ndarray:
        """|A| * |B|^T + |C| (full, or at the sampled coordinates), via the same
        routine on sign-cleared inputs; scales the normal-input tolerance."""
        Aa, Ba = abs_packed(A), abs_packed(B)
        Ca = None if C is None else np.abs(C)
        if idx is None:
            return self.mma(Aa, Ba, Ca, abs(float(c)), dtype)
        return self.mma_sampled(Aa, Ba, Ca, abs(float(c)), dtype, idx)

    def box_copy(self, src: np.ndarray, box, coords, n_repeat: int = 1, coord_step=None,
                 dims=None, strides=None):
        """Compact (n_repeat, *box) image of ``src`` and the bytes it holds.

        ``src`` is a C-contiguous array; dims/strides default to its own shape
        and byte strides. Elements outside dims are zero.
        """
        src = np.ascontiguousarray(src)
        rank = src.ndim if dims is None else len(dims)
        dims = list(src.shape if dims is None else dims)
        strides = list(src.strides if strides is None else strides)
        coord_step = list(coord_step if coord_step is not None else [0] * rank)

        def arr(v, t):
            a = np.zeros(5, t)
            a[: len(v)] = v
            return a

        d5, s5, c5, st5 = (arr(dims, np.int64), arr(strides, np.int64),
                          arr(coords, np.int64), arr(coord_step, np.int64))
        b5 = arr(box, np.int32)
        img = np.empty((n_repeat, *box), src.dtype)
        nbytes = self.L.oracle_box_copy(_ptr(img), _ptr(src), rank, src.itemsize, _ptr(d5),
                                        _ptr(s5), _ptr(b5), _ptr(c5), n_repeat, _ptr(st5))
        if nbytes < 0:
            raise ValueError("oracle_box_copy rejected its arguments")
        return img, int(nbytes)


    def _box_args(self, G, box, coords, n_repeat, coord_step, dims, strides):
        rank = G.ndim if dims is None else len(dims)
        dims = list(G.shape if dims is None else dims)
        strides = list(G.strides if strides is None else strides)
        coord_step = list(coord_step if coord_step is not None else [0] * rank)

        def arr(v, t):
            a = np.zeros(5, t)
            a[: len(v)] = v
            return a

        return rank, (arr(dims, np.int64), arr(strides, np.int64), arr(box, np.int32),
                      arr(coords, np.int64), arr(coord_step, np.int64))

    def box_store(self, G: np.ndarray, img: np.ndarray, box, coords, n_repeat: int = 1,
                  coord_step=None, op: str = "store", elem_type: str | None = None,
                  dims=None, strides=None):
        """A copy of ``G`` after storing (op="store") or add-reducing (op="add")
        the (n_repeat, *box) image ``img`` into it; returns (G', bytes).

        elem_type for "add": "f32", "f16", "bf16", "i32" or "i64" (``img`` and
        ``G`` hold the raw elements: float32, uint16 bits, int32, int64)."""
        G = np.array(G, copy=True, order="C")
        img = np.ascontiguousarray(img, dtype=G.dtype)
        assert img.shape == (n_repeat, *box)
        rank, (d5, s5, b5, c5, st5) = self._box_args(G, box, coords, n_repeat, coord_step,
                                                     dims, strides)
        opc = {"store": 0, "add": 1}[op]
        et = {None: 0, "f32": 1, "f16": 2, "bf16": 3, "i32": 4, "i64": 5}[elem_type]
        nbytes = self.L.oracle_box_store(_ptr(G), _ptr(img), rank, G.itemsize, _ptr(d5),
                                         _ptr(s5), _ptr(b5), _ptr(c5), n_repeat, _ptr(st5),
                                         opc, et)
        if nbytes < 0:
            raise ValueError("oracle_box_store rejected its arguments")
        return G, int(nbytes)

    def mma_splitk(self, A, B, C, c, dtype, splits: int) -> np.ndarray:
        """Split-K form over k=16 (A (…,16,8)) or k=8 (A (…,16,4)) operands."""
        A = np.ascontiguousarray(A, np.uint32)
        B = np.ascontiguousarray(B, np.uint32)
        C = None if C is None else np.ascontiguousarray(C, np.float32)
        batch, M_rep, K_rep = A.shape[:3]
        N_rep, ka = B.shape[1], 2 * A.shape[4]
        D = np.empty((batch, M_rep, N_rep, 16, 8), np.float32)
        rc = self.L.oracle_mma_splitk(_ptr(D), _ptr(A), _ptr(B), _ptr(C), float(c), batch,
                                      M_rep, N_rep, K_rep, ka, splits, _DTYPES[dtype])
        if rc != 0:
            raise ValueError("oracle_mma_splitk rejected its arguments")
        return D

    def mma_splitk_sampled(self, A, B, C, c, dtype, splits: int, idx) -> np.ndarray:
        A = np.ascontiguousarray(A, np.uint32)
        B = np.ascontiguousarray(B, np.uint32)
        C = None if C is None else np.ascontiguousarray(C, np.float32)
        batch, M_rep, K_rep = A.shape[:3]
        N_rep, ka = B.shape[1], 2 * A.shape[4]
        idx = np.ascontiguousarray(idx, np.int64).reshape(-1, 3)
        out = np.empty(len(idx), np.float32)
        rc = self.L.oracle_mma_splitk_sampled(_ptr(out), _ptr(idx), len(idx), _ptr(A), _ptr(B),
                                              _ptr(C), float(c), batch, M_rep, N_rep, K_rep, ka,
                                              splits, _DTYPES[dtype])
        if rc != 0:
            raise ValueError("oracle_mma_splitk_sampled rejected its arguments")
        return out


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _mma_shapes(A, B, C):
    batch, M_rep, K_rep, ra, wa = A.shape
    b2, N_rep, K2, rb, wb = B.shape
    assert (ra, wa, rb, wb) == (16, 8, 8, 8) and b2 == batch and K2 == K_rep
    if C is not None:
        assert C.shape == (batch, M_rep, N_rep, 16, 8) and C.dtype == np.float32
    return batch, M_rep, N_rep, K_rep


def abs_packed(P: np.ndarray) -> np.ndarray:
    """Clear both sign bits of every packed word: |x| of each half, exactly."""
    return np.ascontiguousarray(P, np.uint32) & np.uint32(0x7FFF7FFF)


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def threads() -> int:
    return default().threads()


def h2f(bits, dtype):
    return default().h2f(bits, dtype)


def pack(x, atom_rows, K=None):
    return default().pack(x, atom_rows, K)


def unpack(p, atom_rows):
    return default().unpack(p, atom_rows)


def pack_kmajor(x, atom_rows, rows=None):
    return default().pack_kmajor(x, atom_rows, rows)


def pack_k8(x, atom_rows):
    return default().pack_k8(x, atom_rows)


def mma_k8(A, B, C, c, dtype):
    return default().mma_k8(A, B, C, c, dtype)


def mma_k8_sampled(A, B, C, c, dtype, idx):
    return default().mma_k8_sampled(A, B, C, c, dtype, idx)


def mma(A, B, C, c, dtype):
    return default().mma(A, B, C, c, dtype)


def mma_sampled(A, B, C, c, dtype, idx):
    return default().mma_sampled(A, B, C, c, dtype, idx)


def mma_scaled(A, B, C, c, alpha, beta, dtype):
    return default().mma_scaled(A, B, C, c, alpha, beta, dtype)


def bound(A, B, C, c, dtype, idx=None):
    return default().bound(A, B, C, c, dtype, idx)


def box_copy(src, box, coords, n_repeat=1, coord_step=None, dims=None, strides=None):
    return default().box_copy(src, box, coords, n_repeat, coord_step, dims, strides)


def box_store(G, img, box, coords, n_repeat=1, coord_step=None, op="store", elem_type=None,
              dims=None, strides=None):
    return default().box_store(G, img, box, coords, n_repeat, coord_step, op, elem_type, dims,
                               strides)


def mma_splitk(A, B, C, c, dtype, splits):
    return default().mma_splitk(A, B, C, c, dtype, splits)


def mma_splitk_sampled(A, B, C, c, dtype, splits, idx):
    return default().mma_splitk_sampled(A, B, C, c, dtype, splits, idx)


def build_variant(source_text: str, out_path: str) -> str:
    """Compile a (test-modified) copy of oracle.c to ``out_path``."""
    src_path = out_path + ".c"
    with open(src_path, "w") as f:
        f.write(source_text)
    subprocess.check_call(["gcc", *CFLAGS, src_path, "-o", out_path, "-lm"])
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()
