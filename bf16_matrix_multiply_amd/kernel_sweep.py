"""Time every kernel of the multiply, and the split-K form, over a list of
shapes: the measurement behind the AUTO kernel rule and bmm_splitk_default.

    python3 -m bf16_matrix_multiply_amd.kernel_sweep [MxNxK ...]

Prints one line per shape (bf16 normal operands, no C): the median time of
each forced kernel and of split-K at several split counts, AUTO's choice and
the default split count.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import bf16_matrix_multiply_amd as bmm

DEFAULT_SHAPES = [(128, 128, 256), (512, 512, 512), (1024, 1024, 1024), (1536, 1536, 1536),
                  (2048, 2048, 2048), (2560, 2560, 2560), (3072, 3072, 3072), (4096, 4096, 1024),
                  (4096, 4096, 4096), (8192, 8192, 8192), (1024, 1024, 8192), (2048, 2048, 8192),
                  (1024, 4096, 4096), (2048, 1024, 4096), (1024, 1024, 65536), (512, 512, 65536),
                  (16, 1024, 1024), (64, 2048, 2048), (256, 4096, 4096), (512, 2048, 2048),
                  (64, 8192, 8192), (32, 16384, 4096), (16, 16384, 16384),
                  (8192, 1024, 8192), (1024, 8192, 8192), (2304, 2304, 4096), (3072, 2048, 4096),
                  (2816, 2816, 4096)]


def _median_us(fn, reps=8):
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]))


def sweep(shapes):
    dev = "cuda"
    for M, N, K in shapes:
        a = torch.randn(1, M, K, device=dev).to(torch.bfloat16).view(torch.int16)
        b = torch.randn(1, N, K, device=dev).to(torch.bfloat16).view(torch.int16)
        A, B = bmm.pack_operand(a, 16), bmm.pack_operand(b, 8)
        D = torch.empty(1, M // 16, N // 8, 16, 8, device=dev)
        times = {}
        for k in ("direct", "tiled", "tiled256x128", "tiled128", "skinny"):
            times[k] = _median_us(lambda: bmm.mma_tile(A, B, None, 0.0, "bf16", out=D, kernel=k))
        auto = bmm.select_kernel(1, M // 16, N // 8, K // 16)
        default = bmm.splitk_default(1, M // 16, N // 8, K // 16)
        for s in sorted({2, 4, 8, 16, 32, default}):
            nbytes = bmm.splitk_workspace_bytes(1, M // 16, N // 8, K // 16, 16, s)
            ws = torch.empty(max(nbytes // 4, 1), device=dev)
            times[f"split{s}"] = _median_us(
                lambda: bmm.mma_tile_splitk(A, B, None, 0.0, "bf16", s, out=D, workspace=ws))
            del ws
        best = min(times, key=times.get)
        flops = 2.0 * M * N * K
        print(f"{M}x{N}x{K} auto={auto} split_default={default} best={best} " +
              " ".join(f"{k}={v:.1f}us/{flops / v / 1e6:.0f}TF" for k, v in times.items()),
              flush=True)


def main():
    shapes = [tuple(int(x) for x in s.split("x")) for s in sys.argv[1:]] or DEFAULT_SHAPES
    sweep(shapes)


if __name__ == "__main__":
    main()
