#!/usr/bin/env python3
"""Throughput of the packed f16/bf16 multiply-accumulate D = A * B^T + C on
one MI355X.

One step is the whole path over one batch of synthetic input already resident
in HBM: pack A (row-major halves -> packed words), pack B, and the
multiply-accumulate from C into D. Prints ONE JSON line on stdout.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--kernel auto]

``value`` is 2*M*N*K*batch / (time per step) in TFLOP/s, from K steps timed
as a whole. ``roofline`` is for the step's dominant kernel, timed with HIP
events on the stream it runs on in a second pass of K steps (an event after
each kernel: the events cost GPU time, so they stay out of the first pass);
``cpu_baseline`` is the CPU oracle timed on a bounded sample of the same
workload on this host's cores. The default (headline) run also adds
``extra_records``: the multiply alone on the 4096^3 f16 configuration against
the MFMA peak, and on the skinny 16 x 16384 x 16384 one against HBM (warm and
after a cache flush), each with its own traffic record; and ``power``: socket
power and per-XCD clocks (amd-smi) while the multiply runs back to back for
3 s, null where amd-smi is missing.

    python bench.py --op box_copy|box_store|box_reduce_add

times one box transfer instead (a step is one call over the whole box
workload; ``value`` in GB/s of algorithmic bytes), with the same roofline and
oracle legs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402
from bf16_matrix_multiply_amd.profile_run import source_sha  # noqa: E402

METRIC = "TFLOP/s for f16/bf16 A·Bᵀ+C (fp32 acc) and % of MFMA/HBM roofline"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # MI355X dense, published
PEAK_HBM_GBS = 8000.0                                  # MI355X HBM3E, published
RIDGE_FLOP_PER_BYTE = 2500e12 / 8000e9


def log(*a):
    print(*a, file=sys.stderr, flush=True)


MIN_WARMUP_S = 0.1


def warm_up(step, n: int, torch) -> int:
    """Run the n requested warm-up steps, then more until the GPU has been busy
    for MIN_WARMUP_S: the first few tens of milliseconds of a fresh burst of
    work run measurably slower (8192^3: 957 against 887-891 us per step after
    5 warm-up steps). Returns the number of warm-up steps run."""
    t0 = time.perf_counter()
    done = 0
    for _ in range(n):
        step()
        done += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < MIN_WARMUP_S:
        step()
        done += 1
        torch.cuda.synchronize()
    return done


def traffic_from_profiles(kernel: str, workload: str, variant: str = "", mma_kernel=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since it was taken.
    ``variant`` names what differs from the configuration the plain record
    was taken in (atom K, the alpha/beta form, split-K, a forced kernel); a
    variant reports only a record taken for that variant."""
    tag = f"{kernel}-{variant}" if variant else kernel
    p = os.path.join(ROOT, "profiles", f"traffic_{tag}_{workload}.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_sha") != source_sha(kernel):
        log(f"traffic record {p} is stale (kernel source changed); reporting null")
        return None
    if mma_kernel is not None and rec.get("mma_kernel") not in (None, mma_kernel):
        log(f"traffic record {p} was taken with {rec['mma_kernel']}, not {mma_kernel}; "
            "reporting null")
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, D_gpu, seconds: float, alpha=None, beta=None):
    """The oracle, as it stands, on the first rows of D (all N columns), sized
    to take about ``seconds`` of CPU time; also checks those rows against the
    GPU result (for the alpha/beta form: alpha * product + beta * C)."""
    import oracle
    from_rows = w.batch == 1
    A = oracle.pack(inp["a"], 16)
    B = oracle.pack(inp["b"], 8)
    C = inp["c_tensor"]

    def run(rows):
        idx = np.stack([np.zeros(rows * w.N, np.int64),
                        np.repeat(np.arange(rows, dtype=np.int64), w.N),
                        np.tile(np.arange(w.N, dtype=np.int64), rows)], axis=1)
        t0 = time.perf_counter()
        out = oracle.mma_sampled(A, B, C, inp["c_scalar"], w.dtype, idx)
        return time.perf_counter() - t0, out, idx

    probe_rows = min(w.M, 4)
    t_probe, _, _ = run(probe_rows)
    rows = int(max(probe_rows, min(w.M, seconds / max(t_probe, 1e-6) * probe_rows)))
    t, out, idx = run(rows)
    flops = 2.0 * rows * w.N * w.K
    Dl = D_gpu.transpose(0, 1, 3, 2, 4).reshape(w.batch, w.M, w.N)
    got = Dl[idx[:, 0], idx[:, 1], idx[:, 2]]
    if alpha is not None or beta is not None:
        al, be = (1.0 if alpha is None else alpha), (1.0 if beta is None else beta)
        P = oracle.mma_sampled(A, B, None, 0.0, w.dtype, idx).astype(np.float64)
        if C is None:
            cv = np.full(len(idx), float(inp["c_scalar"]))
        else:
            cv = C.transpose(0, 1, 3, 2, 4).reshape(w.batch, w.M, w.N)[idx[:, 0], idx[:, 1], idx[:, 2]]
        ref = al * P + be * cv
        bnd = abs(al) * oracle.bound(A, B, None, 0.0, w.dtype, idx) + abs(be) * np.abs(cv)
        ok = bool((np.abs(got.astype(np.float64) - ref) <= 1e-3 * bnd).all())
    elif w.exact:
        ok = bool(np.array_equal(got, out))
    else:
        bnd = oracle.bound(A, B, C, inp["c_scalar"], w.dtype, idx)
        ok = bool((np.abs(got.astype(np.float64) - out) <= 1e-3 * bnd).all())
    assert from_rows
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "seconds": round(t, 3),
            "sample": f"first {rows} rows of D x all {w.N} columns ({rows * w.N} outputs, "
                      f"K={w.K} each) of workload {w.name}",
            "sample_matches_gpu": ok}


def box_cpu_baseline(bw, op, inp, got, seconds: float):
    """The oracle's box routine, as it stands, on the first R repeats of the
    box workload (R sized for about ``seconds`` of CPU time), in GB/s of the
    same algorithmic bytes; also checks those repeats against the GPU result
    (``got``: the image for the copy, the tensor after one call from the
    initial one for the store and the add), bit for bit."""
    import oracle
    G0, img = inp["tensor"], inp["image"]

    def run(r):
        rows = r * bw.box_rows   # the first r boxes lie in these rows
        t0 = time.perf_counter()
        if op == "box_copy":
            out, _ = oracle.box_copy(G0[:rows], bw.box, bw.coords, r, bw.step)
        else:
            out, _ = oracle.box_store(G0[:rows], img[:r], bw.box, bw.coords, r, bw.step,
                                      op="store" if op == "box_store" else "add",
                                      elem_type=None if op == "box_store" else "f32")
        return time.perf_counter() - t0, out

    probe = min(8, bw.n_repeat)
    t_probe, _ = run(probe)
    r = int(max(probe, min(bw.n_repeat, seconds / max(t_probe, 1e-6) * probe)))
    t, out = run(r)
    mine = got[:r] if op == "box_copy" else got[:r * bw.box_rows]
    ok = bool(np.array_equal(mine.view(np.uint32), out.view(np.uint32)))
    nbytes = bw.algorithmic_bytes(op) * r / bw.n_repeat
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(t, 3),
            "sample": f"first {r} of {bw.n_repeat} repeats (boxes of {bw.box[0]}x{bw.box[1]} "
                      f"float32) of workload {bw.name}",
            "sample_matches_gpu": ok}


def run_box(args, torch, bmm):
    """One step = one box call over the whole workload (every repeat)."""
    op = args.op
    name = args.workload or next(iter(workloads.BOX_WORKLOADS))
    if name not in workloads.BOX_WORKLOADS:
        raise SystemExit(f"--op {op} needs a box workload: {sorted(workloads.BOX_WORKLOADS)}")
    bw = workloads.BOX_WORKLOADS[name]
    dev = torch.device("cuda:0")
    log(f"[bench] box workload {bw.name}: {bw.n_repeat} boxes of {bw.box} float32, op {op}")
    inp = workloads.make_box_inputs(bw, seed=0)
    G0 = torch.from_numpy(inp["tensor"]).to(dev)
    G = G0.clone()
    IMG = torch.from_numpy(inp["image"]).to(dev)
    OUT = torch.empty_like(IMG)
    stream = torch.cuda.current_stream()

    def call():
        if op == "box_copy":
            bmm.box_copy(G, bw.box, bw.coords, bw.n_repeat, bw.step, out=OUT)
        elif op == "box_store":
            bmm.box_store(G, IMG, bw.box, bw.coords, bw.n_repeat, bw.step)
        else:
            bmm.box_reduce_add(G, IMG, bw.box, bw.coords, "f32", bw.n_repeat, bw.step)

    warmup_run = warm_up(call, args.warmup, torch)
    # timed region: K calls back to back; then K more, each between two events
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream)
        call()
        e[1].record(stream)
    torch.cuda.synchronize()
    k = np.array([e[0].elapsed_time(e[1]) for e in evs])
    nbytes = bw.algorithmic_bytes(op)
    achieved = nbytes / (k.mean() * 1e-3) / 1e9
    log(f"[bench] {op}: {k.mean()*1e3:.1f} us per call (min {k.min()*1e3:.1f}), "
        f"{achieved:.0f} GB/s")

    # parity leg: one call from the initial tensor
    G.copy_(G0)
    call()
    torch.cuda.synchronize()
    got = (OUT if op == "box_copy" else G).cpu().numpy()
    line = {
        "metric": f"GB/s of the float32 {op} and % of HBM roofline",
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warmup_run,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": bw.name, "op": op, "rows": bw.rows, "cols": bw.cols,
                   "box": list(bw.box), "n_repeat": bw.n_repeat, "coord_step": list(bw.step),
                   "swizzle": 0},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_from_profiles(op, bw.name), "kernel": op,
                     "avg_launch_us": round(k.mean() * 1e3, 2),
                     "algorithmic_bytes_per_launch": nbytes},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample of the same workload")
        line["cpu_baseline"] = box_cpu_baseline(bw, op, inp, got, args.cpu_seconds)
    print(json.dumps(line), flush=True)


# The other two configurations with a roofline target, measured in the same
# run as extra records of the default (headline) line: 4096^3 f16 against the
# MFMA peak, and the skinny M = 16 shape against HBM (warm, and after a cache
# flush). Each times the multiply alone: warm calls back to back between one
# pair of events, flushed calls with an event pair each.
EXTRA_RECORDS = ("gemm_4096_f16_quarter", "skinny_16x16384x16384_bf16")


def parse_amd_smi_metric(text: str):
    """(socket power in W, [gfx clock in MHz of each XCD]) from the JSON that
    `amd-smi metric -p -c --json` prints for one GPU; (None, []) if absent."""
    import re
    pw = re.search(r'"socket_power":\s*\{\s*"value":\s*(\d+)', text)
    ck = [int(x) for x in re.findall(r'"gfx_\d+":\s*\{\s*"clk":\s*\{\s*"value":\s*(\d+)',
                                     text)]
    return (int(pw.group(1)) if pw else None), ck


def power_sample(call, torch, seconds=3.0, settle=1.0):
    """Socket power and per-XCD gfx clocks (amd-smi) while ``call`` runs back
    to back for ``seconds``; samples from the first ``settle`` seconds are
    dropped (the telemetry lags by about half a second). None without amd-smi."""
    import shutil
    import subprocess
    import threading
    if shutil.which("amd-smi") is None:
        return None
    samples, stop = [], [False]
    t0 = time.perf_counter()

    def sampler():
        while not stop[0]:
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"],
                                   capture_output=True, text=True, timeout=5)
            except (OSError, subprocess.SubprocessError):
                continue
            watts, clocks = parse_amd_smi_metric(r.stdout)
            if watts is not None:
                samples.append((time.perf_counter() - t0, watts, clocks))

    th = threading.Thread(target=sampler)
    th.start()
    calls = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            call()
        torch.cuda.synchronize()
        calls += 10
    elapsed = time.perf_counter() - t0
    stop[0] = True
    th.join()
    return summarize_power(samples, settle, elapsed / calls * 1e6)


def summarize_power(samples, settle, us_per_call):
    """The power object from (seconds since start, watts, [MHz per XCD]) samples:
    medians over the samples taken after ``settle`` seconds; the per-XCD clocks
    from the samples that list the usual number of XCDs. None without samples."""
    settled = [x for x in samples if x[0] >= settle]
    if not settled:
        return None
    watts = np.array([x[1] for x in settled])
    lengths = [len(x[2]) for x in settled if x[2]]
    n_xcd = max(set(lengths), key=lengths.count) if lengths else 0
    clocks = np.array([x[2] for x in settled if n_xcd and len(x[2]) == n_xcd], dtype=np.int64)
    return {"tool": "amd-smi metric -p -c", "samples": len(settled),
            "socket_w_median": float(np.median(watts)), "socket_w_max": int(watts.max()),
            "gfx_clock_mhz_median_per_xcd": [int(v) for v in np.median(clocks, axis=0)]
            if len(clocks) else None,
            "us_per_call_wall": round(us_per_call, 1)}


def multiply_record(name, torch, bmm, steps):
    w = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    inp = workloads.make_inputs(w, seed=0)
    a = torch.from_numpy(inp["a"].view(np.int16)).to(dev)
    b = torch.from_numpy(inp["b"].view(np.int16)).to(dev)
    A, B = bmm.pack_operand(a, 16), bmm.pack_operand(b, 8)
    del a, b
    C = None if inp["c_tensor"] is None else torch.from_numpy(inp["c_tensor"]).to(dev)
    c = float(inp["c_scalar"])
    D = torch.empty((w.batch, w.M_rep, w.N_rep, 16, 8), dtype=torch.float32, device=dev)
    kernel = bmm.select_kernel(w.batch, w.M_rep, w.N_rep, w.K_rep)
    stream = torch.cuda.current_stream()

    def call():
        bmm.mma_tile(A, B, C, c, w.dtype, out=D)

    warm_up(call, 5, torch)
    # back to back between one pair of events, as the calls run in a loop (an
    # event after every call would add its own few microseconds to each)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    hbm = w.flops / w.algorithmic_bytes < RIDGE_FLOP_PER_BYTE
    rec = {"workload": w.name, "kernel": f"mma_tile[{kernel}]", "dtype": w.dtype,
           "M": w.M, "N": w.N, "K": w.K, "c": "tensor" if w.c_tensor else "scalar",
           "avg_launch_us": round(us, 2), "tflops": round(w.flops / us / 1e6, 2),
           "gbs": round(w.algorithmic_bytes / us / 1e3, 1),
           "algorithmic_bytes_per_launch": w.algorithmic_bytes,
           "traffic": traffic_from_profiles("mma_tile", w.name, "", kernel)}
    if hbm:
        rec.update({"bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "achieved": rec["gbs"], "frac": round(rec["gbs"] / PEAK_HBM_GBS, 4)})
        # after a flush of L2 and the Infinity Cache: each call needs its own
        # flush, so each has its own event pair, whose cost it includes
        flush = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(10):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            cold.append((e0, e1))
        torch.cuda.synchronize()
        cold_us = float(np.mean([x.elapsed_time(y) * 1e3 for x, y in cold]))
        del flush
        rec.update({"cold_us": round(cold_us, 2),
                    "cold_achieved": round(w.algorithmic_bytes / cold_us / 1e3, 1),
                    "cold_frac": round(w.algorithmic_bytes / cold_us / 1e3 / PEAK_HBM_GBS, 4)})
    else:
        rec.update({"bound": "mfma", "peak": PEAK_MFMA_TFLOPS[w.dtype], "unit": "TFLOP/s",
                    "achieved": rec["tflops"],
                    "frac": round(rec["tflops"] / PEAK_MFMA_TFLOPS[w.dtype], 4)})
    log(f"[bench] extra record {w.name}: mma_tile[{kernel}] {us:.1f} us, "
        f"{rec['achieved']} {rec['unit']} ({rec['frac']:.3f} of peak)"
        + (f"; after a cache flush {rec['cold_us']} us ({rec['cold_frac']:.3f})" if hbm else ""))
    del A, B, C, D
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20,
                    help="warm-up steps; more run until the GPU has been busy for 100 ms")
    ap.add_argument("--workload", default=None,
                    choices=sorted(workloads.WORKLOADS) + sorted(workloads.EXTRA_WORKLOADS)
                    + sorted(workloads.BOX_WORKLOADS),
                    help=f"default {workloads.HEADLINE} (with --op, the box workload)")
    ap.add_argument("--op", default="mma", choices=("mma",) + workloads.BOX_OPS,
                    help="mma: the multiply path (pack A, pack B, mma_tile); box_*: one box "
                         "transfer over the box workload")
    ap.add_argument("--kernel", default="auto",
                    choices=["auto", "direct", "tiled", "skinny", "tiled128", "tiled256x128"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--alpha", type=float, default=None,
                    help="run the alpha/beta form D = alpha*A*B^T + beta*C (scaling in the epilogue)")
    ap.add_argument("--beta", type=float, default=None)
    ap.add_argument("--kmajor", action="store_true",
                    help="A and B are stored K-major (transposed) in HBM; the step packs them "
                         "with pack_operand_kmajor")
    ap.add_argument("--atom-k", type=int, default=16, choices=[16, 8],
                    help="K depth of a packed atom: 16, or 8 for the m16n8k8 layout "
                         "(pack_operand_k8 + mma_tile_opts)")
    ap.add_argument("--context", action="store_true",
                    help="also time torch.matmul (the vendor library) on the same logical operands, "
                         "for context only")
    ap.add_argument("--power", action="store_true",
                    help="also sample socket power and gfx clocks (amd-smi) while the multiply "
                         "runs back to back for 3 s (the default headline run always does)")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the power sample of the default (headline) run")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra records of the 4096^3 and skinny configurations that "
                         "the default (headline) run adds")
    ap.add_argument("--splitk", type=int, default=None,
                    help="run the split-K form with this many splits (0: the library's default)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        msg = ("bench.py measures one GPU only: this path has no multi-GPU leg "
               f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).")
        log(msg)
        print(json.dumps({"error": msg, "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import bf16_matrix_multiply_amd as bmm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.op != "mma":
        run_box(args, torch, bmm)
        return
    if args.workload in workloads.BOX_WORKLOADS:
        ap.error(f"{args.workload} is a box workload: pass --op box_copy|box_store|box_reduce_add")
    w = {**workloads.WORKLOADS, **workloads.EXTRA_WORKLOADS}[args.workload or workloads.HEADLINE]
    log(f"[bench] workload {w.name}: batch={w.batch} M={w.M} N={w.N} K={w.K} {w.dtype} "
        f"C={'tensor' if w.c_tensor else 'scalar'}")
    inp = workloads.make_inputs(w, seed=0)
    a = torch.from_numpy(inp["a"].view(np.int16)).to(dev)
    b = torch.from_numpy(inp["b"].view(np.int16)).to(dev)
    if args.kmajor:   # store the operands transposed: element (row, k) at [b, k, row]
        a = a.transpose(1, 2).contiguous()
        b = b.transpose(1, 2).contiguous()
    pack = bmm.pack_operand_kmajor if args.kmajor else bmm.pack_operand
    C = None if inp["c_tensor"] is None else torch.from_numpy(inp["c_tensor"]).to(dev)
    c = float(inp["c_scalar"])
    ka = args.atom_k
    A = torch.empty((w.batch, w.M_rep, w.K // ka, 16, ka // 2), dtype=torch.int32, device=dev)
    B = torch.empty((w.batch, w.N_rep, w.K // ka, 8, ka // 2), dtype=torch.int32, device=dev)
    pack_kw = {} if ka == 16 else {"atom_k": ka}
    D = torch.empty((w.batch, w.M_rep, w.N_rep, 16, 8), dtype=torch.float32, device=dev)
    kernel = bmm.select_kernel(w.batch, w.M_rep, w.N_rep, w.K_rep) if args.kernel == "auto" \
        else args.kernel
    splits, WS = None, None
    if args.splitk is not None:
        if args.alpha is not None or args.beta is not None:
            ap.error("--splitk computes the plain form only")
        splits = args.splitk or bmm.splitk_default(w.batch, w.M_rep, w.N_rep, w.K // ka, ka)
        ws_bytes = bmm.splitk_workspace_bytes(w.batch, w.M_rep, w.N_rep, w.K // ka, ka, splits)
        WS = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=dev)
        kernel = f"tiled+splitk{splits}"
    stream = torch.cuda.current_stream()

    def multiply():
        if splits is not None:
            bmm.mma_tile_splitk(A, B, C, c, w.dtype, splits, out=D, workspace=WS)
        else:
            bmm.mma_tile(A, B, C, c, w.dtype, out=D, kernel=kernel, alpha=args.alpha,
                         beta=args.beta)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pack(a, 16, out=A, **pack_kw)
        if ev is not None:
            ev[1].record(stream)
        pack(b, 8, out=B, **pack_kw)
        if ev is not None:
            ev[2].record(stream)
        multiply()
        if ev is not None:
            ev[3].record(stream)

    warmup_run = warm_up(step, args.warmup, torch)

    # The timed region: K whole steps with nothing recorded between the kernels
    # (a timing event costs the GPU about 3 us, which would land in the step).
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    # Per-kernel durations: K more steps with an event after each kernel, on the
    # stream the kernels run on. Each interval includes its closing event.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    pa = np.array([e[0].elapsed_time(e[1]) for e in evs])
    pb = np.array([e[1].elapsed_time(e[2]) for e in evs])
    mm = np.array([e[2].elapsed_time(e[3]) for e in evs])
    evented_ms = float(np.mean([e[0].elapsed_time(e[3]) for e in evs]))
    log(f"[bench] {args.steps} steps: {total_ms:.3f} ms on events, {wall_ms:.3f} ms wall; "
        f"with per-kernel events {evented_ms * 1e3:.1f} us per step: "
        f"pack A {pa.mean()*1e3:.1f} us, pack B {pb.mean()*1e3:.1f} us, "
        f"mma_tile[{kernel}] {mm.mean()*1e3:.1f} us (min {mm.min()*1e3:.1f})")

    # HBM-bound multiply: also time it with the caches flushed (a 2 GiB fill
    # between calls evicts L2 and the 256 MB Infinity Cache), so no part of B
    # is served from a cache the step's own pack just filled.
    cold_us = None
    if w.flops / w.algorithmic_bytes < RIDGE_FLOP_PER_BYTE:
        flush = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(10):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            multiply()
            e1.record(stream)
            cold.append((e0, e1))
        torch.cuda.synchronize()
        cold_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in cold]))
        del flush
        log(f"[bench] mma_tile after a cache flush: {cold_us:.1f} us "
            f"({w.algorithmic_bytes / cold_us / 1e3:.0f} GB/s)")

    context = None
    if args.context and w.dtype == "bf16" and w.batch == 1 and not args.kmajor:
        # Context, not a target: the vendor library on the same row-major
        # halves, D = A B^T (no C), bf16 output and float32 output.
        at, bt = a[0].view(torch.bfloat16), b[0].view(torch.bfloat16).t()
        context = {"note": "torch.matmul on the same operands (A B^T, no C); not this path"}
        forms = {"bf16_out": lambda: torch.matmul(at, bt),
                 "f32_out": lambda: torch.mm(at, bt, out_dtype=torch.float32)}
        for key, fn in forms.items():
            try:
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(10):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / 10
                context[key] = {"us": round(us, 1), "tflops": round(w.flops / us / 1e6, 1)}
                if args.power and key == "bf16_out":
                    context[key]["power"] = power_sample(fn, torch)
            except (RuntimeError, TypeError) as e:
                context[key] = f"unavailable: {str(e)[:80]}"
        log(f"[bench] context: {context}")

    value = w.flops / (ms_per_step * 1e-3) / 1e12
    op_bytes = 2 * (w.batch * w.M * w.K * 2)          # pack A: read + write
    op_bytes_b = 2 * (w.batch * w.N * w.K * 2)        # pack B: read + write
    mma_s = mm.mean() * 1e-3
    intensity = w.flops / w.algorithmic_bytes
    pack_key = "pack_operand_kmajor" if args.kmajor else "pack_operand"
    times = {"mma_tile": mm.mean(), pack_key: pa.mean() + pb.mean()}
    dominant = max(times, key=times.get)
    # what differs from the configuration each kernel's traffic record is taken in
    pack_variant = "k8" if ka != 16 else ""
    mma_variant = "+".join(v for v in (
        "k8" if ka != 16 else "",
        "scaled" if args.alpha is not None or args.beta is not None else "",
        f"splitk{splits}" if splits is not None else "",
        args.kernel if args.kernel != "auto" else "") if v)
    if dominant == "mma_tile":
        if intensity >= RIDGE_FLOP_PER_BYTE:
            achieved, peak, unit, bound = w.flops / mma_s / 1e12, PEAK_MFMA_TFLOPS[w.dtype], \
                "TFLOP/s", "mfma"
        else:
            achieved, peak, unit, bound = w.algorithmic_bytes / mma_s / 1e9, PEAK_HBM_GBS, \
                "GB/s", "hbm"
    else:
        pack_s = (pa.mean() + pb.mean()) * 1e-3
        achieved, peak, unit, bound = (op_bytes + op_bytes_b) / pack_s / 1e9, PEAK_HBM_GBS, \
            "GB/s", "hbm"
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4),
                "traffic": traffic_from_profiles(
                    dominant, w.name, mma_variant if dominant == "mma_tile" else pack_variant,
                    kernel if dominant == "mma_tile" else None),
                "kernel": dominant if dominant != "mma_tile" else f"mma_tile[{kernel}]",
                "avg_launch_us": round(times[dominant] * 1e3, 2),
                "algorithmic_bytes_per_launch": w.algorithmic_bytes if dominant == "mma_tile"
                else op_bytes + op_bytes_b}

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warmup_run,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "M": w.M, "N": w.N, "K": w.K,
                   "c": "tensor" if w.c_tensor else "scalar", "kernel": kernel,
                   "alpha": args.alpha, "beta": args.beta, "atom_k": ka, "splitk": splits,
                   "step": ("pack_kmajor A + pack_kmajor B + mma_tile" if args.kmajor
                            else "pack A + pack B + mma_tile")},
        "roofline": roofline,
        "kernels": {"timing": "second pass of the K steps, an event after each kernel",
                    "step_us_with_events": round(evented_ms * 1e3, 2),
                    "pack_a_us": round(pa.mean() * 1e3, 2), "pack_b_us": round(pb.mean() * 1e3, 2),
                    "mma_tile_us": round(mm.mean() * 1e3, 2),
                    "mma_tile_median_us": round(float(np.median(mm)) * 1e3, 2),
                    "mma_tile_min_us": round(float(mm.min()) * 1e3, 2),
                    "mma_tile_tflops": round(w.flops / mma_s / 1e12, 2),
                    "mma_tile_gbs": round(w.algorithmic_bytes / mma_s / 1e9, 1),
                    "pack_gbs": round((op_bytes + op_bytes_b) / ((pa.mean() + pb.mean()) * 1e-3)
                                      / 1e9, 1),
                    "mma_tile_cold_us": None if cold_us is None else round(cold_us, 2),
                    "mma_tile_cold_gbs": None if cold_us is None
                    else round(w.algorithmic_bytes / cold_us / 1e3, 1)},
        "cpu_baseline": None,
    }
    if context is not None:
        line["context"] = context
    default_run = (w.name == workloads.HEADLINE and args.kernel == "auto" and not args.kmajor
                   and ka == 16 and splits is None and args.alpha is None and args.beta is None)
    if args.power or (default_run and not args.no_power):
        try:
            line["power"] = power_sample(multiply, torch)
        except Exception as e:   # telemetry only: never lose the line to it
            log(f"[bench] power sample failed: {e!r}")
            line["power"] = None
        log(f"[bench] power while the multiply runs: {line['power']}")
    if default_run and not args.no_extra:
        line["extra_records"] = {n: multiply_record(n, torch, bmm, args.steps)
                                 for n in EXTRA_RECORDS}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample of the same workload")
        line["cpu_baseline"] = cpu_baseline(w, inp, D.cpu().numpy(), args.cpu_seconds, args.alpha,
                                            args.beta)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
