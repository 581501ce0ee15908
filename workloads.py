"""Seeded synthetic inputs for the tiled f16/bf16 multiply-accumulate.

This module only draws numbers and lays them out; it holds none of the
method's arithmetic (no packing, no products, no sums), so both the CPU
oracle and the HIP path can take their inputs from it without sharing any
computation.

Recipes (all from ``numpy.random.default_rng(seed)``, draws in the order A,
B, C):

* ``quarter``: integers uniform in [-4, 4] divided by 4, stored as f16 (the
  recipe of the worked 16x8 example on the mma.sync page, "Example: a 16x8
  result with two K16 issues"). These values are exact in f16 and bf16.
* ``normal``: ``standard_normal(float32) * scale``, rounded once to bf16 with
  round-to-nearest-even (or to f16 with numpy's own round-to-nearest-even).
* ``ternary``: -1/4, 0 or 1/4, uniformly (integers in [0, 2] mapped to those
  three values), for exact cases with a very long K: every product is 0 or
  1/16 in magnitude, so partial sums stay exact in fp32 up to K = 2^24.
* C, when it is a tensor, is standard normal float32 (or, for the exact
  quarter-integer cases, integers in [-64, 64] divided by 4) drawn directly in
  the atom-tiled accumulator layout (batch, M/16, N/8, 16, 8); the draws are
  i.i.d., so drawing in the stored layout changes no statistics.

Half-precision operands are returned as uint16 bit patterns, row-major
(batch, rows, K).
"""
from __future__ import annotations

import dataclasses

import numpy as np

F16, BF16 = "f16", "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits.

    Input quantisation only: NaN is not expected in the synthetic draws and is
    rejected.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if np.isnan(x).any():
        raise ValueError("NaN in bf16 quantisation input")
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    M: int
    N: int
    K: int
    dtype: str            # "f16" | "bf16"
    a_dist: str           # "quarter" | "normal"
    b_dist: str
    b_scale: float = 1.0
    c_tensor: bool = False
    c_scalar: float = 0.0
    exact: bool = False   # every product and partial sum is exact in fp32
    c_dist: str = "normal"  # "quarter" keeps C on the exact grid as well

    @property
    def M_rep(self) -> int:
        return self.M // 16

    @property
    def N_rep(self) -> int:
        return self.N // 8

    @property
    def K_rep(self) -> int:
        return self.K // 16

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """Compulsory HBM bytes of one multiply-accumulate call: packed A and
        B read once, C read once if it is a tensor, D written once."""
        a = self.batch * self.M * self.K * 2
        b = self.batch * self.N * self.K * 2
        d = self.batch * self.M * self.N * 4
        return a + b + d + (d if self.c_tensor else 0)


WORKLOADS = {
    w.name: w
    for w in [
        # The worked example: M_repeat = N_repeat = 1, K_repeat = 2, scalar C = 0.
        Workload("tile_16x8x32_f16", 1, 16, 8, 32, F16, "quarter", "quarter", exact=True),
        Workload("gemm_128x128x256_bf16_ctensor", 1, 128, 128, 256, BF16, "normal", "normal",
                 c_tensor=True),
        Workload("gemm_4096_f16_quarter", 1, 4096, 4096, 4096, F16, "quarter", "quarter",
                 exact=True),
        Workload("skinny_16x16384x16384_bf16", 1, 16, 16384, 16384, BF16, "normal", "normal",
                 b_scale=0.02),
        Workload("gemm_8192_bf16_ctensor", 1, 8192, 8192, 8192, BF16, "normal", "normal",
                 c_tensor=True),
    ]
}

# Beyond the five: a long-K problem with few output tiles (16 tiles of 256 x 256
# for 256 CUs), the shape the split-K form is for.
EXTRA_WORKLOADS = {
    w.name: w
    for w in [
        Workload("deep_k_1024x1024x65536_bf16_ctensor", 1, 1024, 1024, 65536, BF16, "normal",
                 "normal", c_tensor=True),
        # one GPU's share of the 8192^3 multiply split 8 ways along N (all of A, an
        # eighth of the columns of B, C and D), and along M
        Workload("shard_n8_8192x1024x8192_bf16_ctensor", 1, 8192, 1024, 8192, BF16, "normal",
                 "normal", c_tensor=True),
        Workload("shard_m8_1024x8192x8192_bf16_ctensor", 1, 1024, 8192, 8192, BF16, "normal",
                 "normal", c_tensor=True),
    ]
}

# The headline compute-bound workload that bench.py times.
HEADLINE = "gemm_8192_bf16_ctensor"
SKINNY = "skinny_16x16384x16384_bf16"


# bit patterns of -1/4, 0 and 1/4 in each format (exact in both)
_TERNARY_BITS = {F16: np.array([0xB400, 0x0000, 0x3400], np.uint16),
                 BF16: np.array([0xBE80, 0x0000, 0x3E80], np.uint16)}


def draw_operand(rng: np.random.Generator, dist: str, shape, dtype: str, scale: float = 1.0):
    if dist == "ternary":
        # -1/4, 0 or 1/4 uniformly: every product is 0 or +-1/16, so sums of up
        # to 2^24 products are exact in fp32 (long-K exact cases)
        return _TERNARY_BITS[dtype][rng.integers(0, 3, shape, dtype=np.int8)]
    if dist == "quarter":
        vals = rng.integers(-4, 5, shape) / 4
        if dtype == F16:
            return vals.astype(np.float16).view(np.uint16)
        return f32_to_bf16_bits(vals.astype(np.float32))
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
        if scale != 1.0:
            x = x * np.float32(scale)
        return f32_to_bf16_bits(x) if dtype == BF16 else f32_to_f16_bits(x)
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(w: Workload, seed: int = 0, a_dist: str | None = None,
                b_dist: str | None = None):
    """Return dict(a, b, c_tensor, c_scalar) for workload ``w``.

    ``a``/``b`` are uint16 (batch, M, K) / (batch, N, K) row-major bits; the
    optional distribution overrides build quantised variants of a shape.
    """
    rng = np.random.default_rng(seed)
    a = draw_operand(rng, a_dist or w.a_dist, (w.batch, w.M, w.K), w.dtype)
    b = draw_operand(rng, b_dist or w.b_dist, (w.batch, w.N, w.K), w.dtype, w.b_scale)
    c = None
    if w.c_tensor:
        shape = (w.batch, w.M_rep, w.N_rep, 16, 8)
        if w.c_dist == "quarter":
            c = (rng.integers(-64, 65, shape) / 4).astype(np.float32)
        else:
            c = rng.standard_normal(shape, dtype=np.float32)
    return dict(a=a, b=b, c_tensor=c, c_scalar=np.float32(w.c_scalar))


def custom(batch, M, N, K, dtype=BF16, a_dist="normal", b_dist="normal", c_tensor=False,
           c_scalar=0.0, b_scale=1.0, name="custom") -> Workload:
    exact = a_dist in ("quarter", "ternary") and b_dist in ("quarter", "ternary")
    return Workload(name, batch, M, N, K, dtype, a_dist, b_dist, b_scale, c_tensor, c_scalar,
                    exact=exact, c_dist="quarter" if exact else "normal")


# ---- box transfers (cp.async.bulk.tensor page: box, coordinates, per-repeat
# coordinate step, repeat count; "Stores, reductions, and completion" for the
# store and add directions) ----

@dataclasses.dataclass(frozen=True)
class BoxWorkload:
    """A float32 tensor of (rows, cols) moved through rows / box_rows boxes of
    box_rows x cols, starting at (0, 0) and stepping box_rows rows per repeat:
    every element of the tensor is in exactly one box."""
    name: str
    rows: int
    cols: int
    box_rows: int

    @property
    def n_repeat(self) -> int:
        return self.rows // self.box_rows

    @property
    def box(self):
        return (self.box_rows, self.cols)

    @property
    def coords(self):
        return (0, 0)

    @property
    def step(self):
        return (self.box_rows, 0)

    @property
    def image_bytes(self) -> int:
        return self.n_repeat * self.box_rows * self.cols * 4

    def algorithmic_bytes(self, op: str) -> int:
        """Each byte touched once: the image and the box region read or written
        (copy and store: one read, one write; add: two reads, one write)."""
        return (3 if op == "box_reduce_add" else 2) * self.image_bytes


BOX_OPS = ("box_copy", "box_store", "box_reduce_add")

BOX_WORKLOADS = {
    bw.name: bw
    for bw in [
        # 512 MiB in 8192 boxes of 64 x 256 (64 KiB each, the staging limit)
        BoxWorkload("box_f32_524288x256_64x256", 524288, 256, 64),
    ]
}


def make_box_inputs(bw: BoxWorkload, seed: int = 0):
    """Return dict(tensor, image): standard normal float32, drawn in that order;
    ``image`` is the compact (n_repeat, box_rows, cols) image that the store
    and add directions write."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((bw.rows, bw.cols), dtype=np.float32)
    img = rng.standard_normal((bw.n_repeat, bw.box_rows, bw.cols), dtype=np.float32)
    return dict(tensor=g, image=img)
