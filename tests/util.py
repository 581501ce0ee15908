"""Test-side helpers: layout plumbing and independent decoders.

Nothing here computes the method: the decoders use numpy's float16 and
torch's bfloat16 conversions (library routines, independent of the oracle's
hand-written decoder), and the layout helpers only reshape.
"""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

U32 = 2.0 ** -24   # unit roundoff of float32


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def tile_to_logical(D):
    """(batch, M_rep, N_rep, 16, 8) -> (batch, M, N)."""
    b, mr, nr, i, j = D.shape
    return np.ascontiguousarray(np.asarray(D).transpose(0, 1, 3, 2, 4)).reshape(b, mr * i, nr * j)


def logical_to_tile(X):
    """(batch, M, N) -> (batch, M/16, N/8, 16, 8)."""
    b, M, N = X.shape
    return np.ascontiguousarray(np.asarray(X).reshape(b, M // 16, 16, N // 8, 8)
                                .transpose(0, 1, 3, 2, 4))


def decode(bits, dtype):
    """uint16 bit patterns -> float64 values, via numpy (f16) or torch (bf16)."""
    bits = np.ascontiguousarray(bits, np.uint16)
    if dtype in ("f16", 0):
        return bits.view(np.float16).astype(np.float64)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def gamma(n):
    return n * U32 / (1 - n * U32)


def page_recipe_pack(x, R):
    """The mma.sync page's host packing (reshape, transpose, view as uint32),
    written for any number of row atoms and K atoms: (batch, rows, K) uint16
    -> (batch, rows/R, K/16, R, 8) uint32."""
    b, rows, K = x.shape
    y = np.ascontiguousarray(x.reshape(b, rows // R, R, K // 16, 16).transpose(0, 1, 3, 2, 4))
    return y.view(np.uint32).reshape(b, rows // R, K // 16, R, 8)


def page_recipe_pack_k8(x, R):
    """The same recipe with an atom K of 8 (the m16n8k8 form): (batch, rows, K)
    uint16 -> (batch, rows/R, K/8, R, 4) uint32."""
    b, rows, K = x.shape
    y = np.ascontiguousarray(x.reshape(b, rows // R, R, K // 8, 8).transpose(0, 1, 3, 2, 4))
    return y.view(np.uint32).reshape(b, rows // R, K // 8, R, 4)


def random_bits(rng, shape):
    return rng.integers(0, 1 << 16, shape, dtype=np.uint32).astype(np.uint16)


def sample_indices(rng, batch, M, N, count, corners=True):
    """(count, 3) int64 (b, m, n) samples, plus the four corners of each batch."""
    idx = np.stack([rng.integers(0, batch, count), rng.integers(0, M, count),
                    rng.integers(0, N, count)], axis=1)
    if corners:
        extra = [(b, m, n) for b in range(batch) for m in (0, M - 1) for n in (0, N - 1)]
        idx = np.concatenate([idx, np.array(extra, np.int64)])
    return idx.astype(np.int64)
