"""Throughput of the box transfers (bmm_box_copy, bmm_box_store,
bmm_box_reduce_add) on one MI355X.

Each operation streams a 512 MiB float32 tensor, seen as (rows, 256), through
8192 boxes of 64 x 256 elements (64 KiB, the staging limit), stepping down
the rows: one workgroup per box, through an LDS image in each swizzle mode.
Prints one JSON line per operation: time per call (HIP events), the bytes it
moves (copy and store: read + write of the image; add: image + destination
read, destination write) and the fraction of the 8 TB/s HBM peak. Two
context lines time torch's own elementwise copy and in-place add over the
same bytes, the practical streaming rate on the same box.

    python3 -m bf16_matrix_multiply_amd.microbench.box_bench [--reps 10]
"""
from __future__ import annotations

import argparse
import json

import numpy as np
import torch

import bf16_matrix_multiply_amd as bmm

PEAK_GBS = 8000.0


def timed(fn, reps):
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
    return float(t.mean()), float(np.median(t)), float(t.min())


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    rows, cols, box_rows, n = 64 * 8192, 256, 64, 8192
    g = torch.randn((rows, cols), device="cuda")
    img = torch.empty((n, box_rows, cols), device="cuda")
    image_bytes = n * box_rows * cols * 4
    box, coords, step = (box_rows, cols), (0, 0), (box_rows, 0)
    flat = g.view(n, box_rows, cols)
    for name, fn, nbytes in (("torch_copy", lambda: img.copy_(flat), 2 * image_bytes),
                             ("torch_add_", lambda: flat.add_(img), 3 * image_bytes)):
        mean, med, mn = timed(fn, args.reps)
        gbs = nbytes / (mean * 1e-6) / 1e9
        print(json.dumps({"op": name, "bytes_per_call": nbytes, "us_mean": round(mean, 1),
                          "us_median": round(med, 1), "us_min": round(mn, 1),
                          "gbs": round(gbs, 1), "frac_of_8tbs": round(gbs / PEAK_GBS, 4)}),
              flush=True)
    for swz in (0, 3):
        ops = {
            "box_copy": (lambda: bmm.box_copy(g, box, coords, n, step, swizzle=swz, out=img),
                         2 * image_bytes),
            "box_store": (lambda: bmm.box_store(g, img, box, coords, n, step, swizzle=swz),
                          2 * image_bytes),
            "box_reduce_add_f32": (lambda: bmm.box_reduce_add(g, img, box, coords, "f32", n, step,
                                                              swizzle=swz),
                                   3 * image_bytes),
        }
        for name, (fn, nbytes) in ops.items():
            mean, med, mn = timed(fn, args.reps)
            gbs = nbytes / (mean * 1e-6) / 1e9
            print(json.dumps({"op": name, "swizzle": swz, "boxes": n, "box": list(box),
                              "elem": "f32", "bytes_per_call": nbytes,
                              "us_mean": round(mean, 1), "us_median": round(med, 1),
                              "us_min": round(mn, 1), "gbs": round(gbs, 1),
                              "frac_of_8tbs": round(gbs / PEAK_GBS, 4)}), flush=True)


if __name__ == "__main__":
    main()
