"""Profiling driver and counter summariser for rocprofv3.

Run under the profiler (one counter pass per run):

    rocprofv3 --pmc FETCH_SIZE -d OUT -o run -- python3 -m bf16_matrix_multiply_amd.profile_run \
        --workload gemm_8192_bf16_ctensor

The driver first runs a plain device-to-device copy of a known size (the
calibration dispatch: what the counter reads for bytes that are known), then
``--reps`` passes of the path (pack A, pack B, multiply-accumulate) on the
workload's synthetic inputs; for a box workload, ``--reps`` passes of
box_copy, box_store and box_reduce_add over it (summarised one at a time with
``--which box_copy`` and so on).

    python3 -m bf16_matrix_multiply_amd.profile_run --summarize FETCH.csv WRITE.csv \
        --workload gemm_8192_bf16_ctensor --kernel mma_tile

turns the counter CSVs of a FETCH_SIZE and a WRITE_SIZE pass into the
per-launch HBM byte record that bench.py reports as ``traffic`` (for packing:
per step, the A and B launches together).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30   # calibration copy: 1 GiB read + 1 GiB written
KERNEL_SOURCES = {
    "mma_tile": ["mma_direct.hip", "mma_tiled.hip", "mma_skinny.hip", "common.h", "launch.h"],
    "pack_operand": ["pack.hip", "common.h"],
    "pack_operand_kmajor": ["pack.hip", "common.h"],
    "box_copy": ["box.hip", "common.h"],
    "box_store": ["box.hip", "common.h"],
    "box_reduce_add": ["box.hip", "common.h"],
}
# Dispatch-name pieces of each kernel family (inside the bmm namespace). The
# box workloads take the 16-byte path; the add is the float32 one.
KERNEL_MATCH = {"mma_tile": ("mma_",), "pack_operand": ("pack_kernel<", "pack_staged_kernel<"),
                "pack_operand_kmajor": ("pack_kmajor_kernel<",),
                "box_copy": ("::box_kernel",), "box_store": ("box_store_kernel_v<0>",),
                "box_reduce_add": ("box_store_kernel_v<1>",)}


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed, so that a
    comment edit does not mark counter records stale (the kernels' sources
    hold no string literal containing a comment marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        p = os.path.join(ROOT, "bf16_matrix_multiply_amd", "csrc", f)
        if os.path.exists(p):
            h.update(_code_only(open(p).read()).encode())
    return h.hexdigest()[:16]


def run(workload: str, reps: int, kernel: str, kmajor: bool = False):
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import bf16_matrix_multiply_amd as bmm
    import workloads

    dev = torch.device("cuda:0")
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)                     # the calibration dispatch
    torch.cuda.synchronize()
    del src, dst

    if workload in workloads.BOX_WORKLOADS:
        bw = workloads.BOX_WORKLOADS[workload]
        inp = workloads.make_box_inputs(bw, seed=0)
        G = torch.from_numpy(inp["tensor"]).to(dev)
        img = torch.from_numpy(inp["image"]).to(dev)
        out = torch.empty_like(img)
        torch.cuda.synchronize()
        for _ in range(reps):
            bmm.box_copy(G, bw.box, bw.coords, bw.n_repeat, bw.step, out=out)
            bmm.box_store(G, img, bw.box, bw.coords, bw.n_repeat, bw.step)
            bmm.box_reduce_add(G, img, bw.box, bw.coords, "f32", bw.n_repeat, bw.step)
        torch.cuda.synchronize()
        print(f"profile_run: copy {COPY_BYTES} B, then {reps} x (box_copy, box_store, "
              f"box_reduce_add) on {bw.name}", flush=True)
        return

    w = {**workloads.WORKLOADS, **workloads.EXTRA_WORKLOADS}[workload]
    inp = workloads.make_inputs(w, seed=0)
    a = torch.from_numpy(inp["a"].view(np.int16)).to(dev)
    b = torch.from_numpy(inp["b"].view(np.int16)).to(dev)
    if kmajor:   # the operands stored transposed: element (row, k) at [b, k, row]
        a = a.transpose(1, 2).contiguous()
        b = b.transpose(1, 2).contiguous()
    pack = bmm.pack_operand_kmajor if kmajor else bmm.pack_operand
    C = None if inp["c_tensor"] is None else torch.from_numpy(inp["c_tensor"]).to(dev)
    A = pack(a, 16)
    B = pack(b, 8)
    D = torch.empty((w.batch, w.M_rep, w.N_rep, 16, 8), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for _ in range(reps):
        pack(a, 16, out=A)
        pack(b, 8, out=B)
        bmm.mma_tile(A, B, C, float(inp["c_scalar"]), w.dtype, out=D, kernel=kernel)
    torch.cuda.synchronize()
    kind = "K-major " if kmajor else ""
    print(f"profile_run: copy {COPY_BYTES} B, then {reps} x ({kind}pack A, {kind}pack B, "
          f"mma_tile[{kernel}]) on {w.name}", flush=True)


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _per_dispatch(rows, counter):
    """{dispatch_id: (kernel_name, value)} for one counter of a counter CSV."""
    out = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        did = int(r["Dispatch_Id"])
        name = r["Kernel_Name"]
        val = float(r["Counter_Value"])
        prev = out.get(did, (name, 0.0))[1]
        out[did] = (name, prev + val)
    return out


def summarize(fetch_csv, write_csv, workload, kernel):
    sys.path.insert(0, ROOT)
    import workloads

    box = workload in workloads.BOX_WORKLOADS
    w = workloads.BOX_WORKLOADS[workload] if box else {**workloads.WORKLOADS, **workloads.EXTRA_WORKLOADS}[workload]
    rec = {"workload": workload, "kernel": kernel, "source_sha": source_sha(kernel),
           "calibration_copy_bytes": COPY_BYTES}
    total = 0.0
    for path, counter, key in ((fetch_csv, "FETCH_SIZE", "fetch"), (write_csv, "WRITE_SIZE", "write")):
        d = _per_dispatch(_rows(path), counter)
        # the calibration dispatch is the device-to-device copy (its name says copy)
        copy_ids = [i for i, (n, _) in d.items() if "copy" in n.lower()]
        copy_kib = d[copy_ids[0]][1]
        scale = (COPY_BYTES / 1024) / copy_kib if copy_kib > 0 else float("nan")
        mine = [v for i, (n, v) in d.items() if any(m in n for m in KERNEL_MATCH[kernel])]
        # one launch of the multiply per step; packing is two launches per
        # step (A and B), counted together as bench.py's pack roofline does
        per_step = 2 if kernel.startswith("pack_operand") else 1
        kib = sum(mine) / (len(mine) / per_step)
        rec[f"{key}_kib_per_dispatch_raw"] = round(kib, 1)
        rec[f"{key}_copy_kib_raw"] = round(copy_kib, 1)
        rec[f"{key}_scale"] = round(scale, 4)
        rec[f"{key}_bytes_per_launch"] = round(kib * 1024 * scale)
        rec[f"{key}_dispatches"] = len(mine)
        total += kib * 1024 * scale
    rec["hbm_bytes_per_launch"] = round(total)
    if box:
        rec["algorithmic_bytes_per_launch"] = w.algorithmic_bytes(kernel)
    elif kernel == "mma_tile":
        rec["algorithmic_bytes_per_launch"] = w.algorithmic_bytes
        # the kernel AUTO ran (the run uses --kernel auto): a record holds for it only
        import bf16_matrix_multiply_amd as bmm
        rec["mma_kernel"] = bmm.select_kernel(w.batch, w.M_rep, w.N_rep, w.K_rep)
    else:
        rec["algorithmic_bytes_per_launch"] = 4 * w.batch * (w.M + w.N) * w.K
    rec["traffic_over_algorithmic"] = round(total / rec["algorithmic_bytes_per_launch"], 3)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="gemm_8192_bf16_ctensor")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--kernel", default="auto")
    ap.add_argument("--kmajor", action="store_true",
                    help="store the operands transposed and pack them with pack_operand_kmajor")
    ap.add_argument("--summarize", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--which", default="mma_tile", choices=sorted(KERNEL_SOURCES))
    args = ap.parse_args()
    if args.summarize:
        print(json.dumps(summarize(*args.summarize, args.workload, args.which), indent=1))
    else:
        run(args.workload, args.reps, args.kernel, args.kmajor)


if __name__ == "__main__":
    main()
