#!/usr/bin/env python3
"""Benchmark of the block-quantized GEMV/GEMM hot path on one MI355X.

Default workload (the headline metric): Q1_0.q8_0 GEMV at 8B-class decode
shapes, batch 1 -- weights 4096x4096 and 14336x4096 (K=4096), each applied to
32 seeded q8_0 activation vectors as separate batch-1 GEMVs. One step is those
64 GEMVs, run as two grouped launches (one per weight shape, 32 independent
problems each). Every problem reads its own copy of the repacked weight
planes, and successive steps rotate through a ring of copies totalling more
than 1 GiB, so no weight byte is served from cache (MI355X has a 256 MB
last-level cache): each step streams 342 MB of algorithmic bytes from HBM.

Printed: one JSON line with the metric, the roofline of the dominant kernel
(algorithmic bytes per launch / mean launch time from HIP events on the
launch stream) and the CPU oracle timed on a bounded sample of the same
workload on the host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload q1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth, decimal GB/s
MODEL_8B_Q1_BYTES = 8e9 * 18 / 128   # 8B weights at 18 bytes per 128 -> bytes per token
METRIC = "Q1_0·q8_0 GEMV effective HBM GB/s (% of peak) + equiv tok/s, batch 1"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def q1_gemv_bytes(rows: int, K: int) -> int:
    """Algorithmic bytes of one batch-1 GEMV: each weight byte once (18 bytes
    per 128 weights), the q8_0 activation once (34 per 32), the f32 output."""
    return rows * (K // 128) * 18 + (K // 32) * 34 + rows * 4


# ----------------------------------------------------------------- helpers

def measured_read_ceiling(gd, torch, gib: float = 2.0, passes: int = 8, reps: int = 5):
    """Streaming-read ceiling (page "roofline.html" method): fill a buffer far
    larger than the last-level cache with a non-zero pattern, then time
    repeated full read passes; best of `reps`."""
    nbytes = int(gib * (1 << 30))
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gd.gemm_decode_fill(buf, 12345)
    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    gd.gemm_decode_stream_read(buf, 2, sink)   # warm-up
    best = float("inf")
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        gd.gemm_decode_stream_read(buf, passes, sink)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3)
    del buf
    return nbytes * passes / best / 1e9


def cpu_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# --------------------------------------------------------- Q1 workload

def bench_q1(args, gd, torch):
    shapes = wl.Q1_DECODE
    K = shapes[0].K
    n_vec = len(shapes[0].act_seeds)
    log(f"[bench] q1: building inputs ({len(shapes)} weights, {n_vec} activation vectors)")
    Ws = [wl.q1_weights_aos(s.rows, s.K, s.weight_seed) for s in shapes]
    A = np.concatenate([wl.q8_acts_aos(K, sd) for sd in shapes[0].act_seeds])   # [n_vec, K/32, 34]
    a_dev = [torch.from_numpy(np.ascontiguousarray(A[c])).cuda() for c in range(n_vec)]

    step_bytes = sum(n_vec * q1_gemv_bytes(s.rows, s.K) for s in shapes)
    plane_bytes = [sum(gd.q1_planes_bytes(s.rows, s.K)) for s in shapes]
    set_bytes = n_vec * sum(plane_bytes)
    ring = max(2, int(np.ceil(args.ring_gib * (1 << 30) / set_bytes)))
    log(f"[bench] q1: step = {2 * n_vec} GEMVs, {step_bytes / 1e6:.1f} MB algorithmic; "
        f"ring of {ring} step sets = {ring * set_bytes / 2**30:.2f} GiB of planes")

    # planes: repack once per shape, then copy into every ring slot
    base = []
    for s, W in zip(shapes, Ws):
        b, sc = gd.q1_alloc_planes(s.rows, s.K)
        gd.q1_repack(torch.from_numpy(W.reshape(-1)).cuda(), s.rows, s.K, b, sc)
        base.append((b, sc))
    ys = [[torch.empty(s.rows, dtype=torch.float32, device="cuda") for _ in range(n_vec)] for s in shapes]
    slots = []     # slots[r][shape] = (problems tensor, keep-alive list)
    for r in range(ring):
        per_shape = []
        for si, s in enumerate(shapes):
            copies = [(base[si][0].clone(), base[si][1].clone()) for _ in range(n_vec)]
            probs = gd.make_q1_problems([(copies[c][0], copies[c][1], a_dev[c], ys[si][c])
                                         for c in range(n_vec)])
            per_shape.append((probs, copies))
        slots.append(per_shape)
    torch.cuda.synchronize()

    def step(r, events=None):
        for si, s in enumerate(shapes):
            if events is not None:
                events[si][0].record()
            gd.q1_q8_gemv_grouped(slots[r][si][0], n_vec, s.rows, s.K)
            if events is not None:
                events[si][1].record()

    # parity spot check (untimed): every output of the first ring slot
    step(0)
    torch.cuda.synchronize()
    mism = None
    if args.parity:
        import oracle
        mism = 0
        for si, (s, W) in enumerate(zip(shapes, Ws)):
            got = np.stack([ys[si][c].cpu().numpy() for c in range(n_vec)])
            want = oracle.q1_q8_gemv_aos(W, A, s.rows, s.K, n_act=n_vec, nthreads=cpu_cores())
            mism += int((got.view(np.uint32) != want.view(np.uint32)).sum())
        log(f"[bench] q1: parity vs oracle: {mism} mismatching outputs")

    for w in range(args.warmup):
        step(w % ring)
    torch.cuda.synchronize()

    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in shapes] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for k in range(args.steps):
        step((args.warmup + k) % ring, evs[k])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_s = t0.elapsed_time(t1) / 1e3
    per_launch = [[evs[k][si][0].elapsed_time(evs[k][si][1]) / 1e3 for k in range(args.steps)]
                  for si in range(len(shapes))]
    launch_bytes = [n_vec * q1_gemv_bytes(s.rows, s.K) for s in shapes]
    kern_s = sum(sum(p) for p in per_launch)
    kern_bytes = sum(launch_bytes[si] * args.steps for si in range(len(shapes)))
    achieved = kern_bytes / kern_s / 1e9

    gbps = step_bytes * args.steps / total_s / 1e9
    ms_per_step = total_s / args.steps * 1e3

    # serial mode: one launch per GEMV, back to back (decode-schedule figure)
    serial = None
    if args.serial_steps > 0:
        for r in range(min(2, ring)):     # warm
            for si, s in enumerate(shapes):
                for c in range(n_vec):
                    b, sc = slots[r][si][1][c]
                    gd.q1_q8_gemv(b, sc, a_dev[c], ys[si][c], s.rows, s.K, 1)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(args.serial_steps):
            r = k % ring
            for si, s in enumerate(shapes):
                for c in range(n_vec):
                    b, sc = slots[r][si][1][c]
                    gd.q1_q8_gemv(b, sc, a_dev[c], ys[si][c], s.rows, s.K, 1)
        e1.record()
        torch.cuda.synchronize()
        ser_s = e0.elapsed_time(e1) / 1e3
        serial = {"GBps": round(step_bytes * args.serial_steps / ser_s / 1e9, 1),
                  "us_per_gemv": round(ser_s / (args.serial_steps * 2 * n_vec) * 1e6, 3),
                  "launches": args.serial_steps * 2 * n_vec}

    ceiling = (measured_read_ceiling(gd, torch, gib=args.ceiling_gib, passes=args.ceiling_passes,
                                     reps=args.ceiling_reps) if args.ceiling else None)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_q1(Ws, A, shapes, budget_s=args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Q1_0.q8_0 GEMV batch 1: 32 activation vectors x {4096x4096, 14336x4096}, "
                        "K=4096, 64 independent GEMVs per step in 2 grouped launches, distinct weight "
                        "copies (ring > 1 GiB)",
            "rows": [s.rows for s in shapes], "K": K, "activation_vectors": n_vec,
            "step_bytes": step_bytes, "ring_sets": ring,
        },
        "pct_of_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "equiv_tok_s": round(gbps * 1e9 / MODEL_8B_Q1_BYTES, 1),
        "rows_K_per_s": round(sum(n_vec * s.rows * s.K for s in shapes) * args.steps / total_s, 1),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
            "kernel": "q1_gemv_grouped_kernel",
            "per_shape_us": {f"{s.rows}x{s.K}": round(float(np.mean(per_launch[si])) * 1e6, 2)
                             for si, s in enumerate(shapes)},
            "bytes_per_launch": {f"{s.rows}x{s.K}": launch_bytes[si] for si, s in enumerate(shapes)},
        },
        "parity_mismatches": mism,
        "serial_one_launch_per_gemv": serial,
        "measured_read_ceiling_GBps": None if ceiling is None else round(ceiling, 1),
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
    }
    return out


def cpu_baseline_q1(Ws, A, shapes, budget_s: float):
    """The oracle (form F1) on the host, on the same workload: the step's
    batch-1 GEMVs in order (vector c against each weight shape), cycling until
    about budget_s of CPU time has been spent."""
    import oracle
    threads = cpu_cores()
    oracle.lib()
    done_bytes, t_used, n_gemv = 0, 0.0, 0
    n_vec = A.shape[0]
    order = [(c, si) for c in range(n_vec) for si in range(len(shapes))]
    while t_used < budget_s:
        c, si = order[n_gemv % len(order)]
        s = shapes[si]
        t = time.perf_counter()
        oracle.q1_q8_gemv_aos(Ws[si], A[c], s.rows, s.K, 1, nthreads=threads)
        t_used += time.perf_counter() - t
        done_bytes += q1_gemv_bytes(s.rows, s.K)
        n_gemv += 1
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_gemv} batch-1 GEMVs of the step (vectors x {{4096x4096, 14336x4096}}, in order, "
                      f"cycling), {t_used:.2f} s of oracle time, OpenMP over rows, {cpu_model()}"}


# --------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="q1", choices=["q1"])
    ap.add_argument("--ring-gib", type=float, default=1.25)
    ap.add_argument("--serial-steps", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ceiling", dest="ceiling", action="store_false")
    ap.add_argument("--ceiling-gib", type=float, default=2.0)
    ap.add_argument("--ceiling-passes", type=int, default=8)
    ap.add_argument("--ceiling-reps", type=int, default=5)
    ap.add_argument("--no-parity", dest="parity", action="store_false",
                    help="skip the untimed oracle comparison (profiling runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (the kernels run on one MI355X; "
              "multi-GPU sharding is a design note, not built) -- run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no HIP device visible", file=sys.stderr)
        sys.exit(1)
    import gemm_decode_amd as gd
    torch.cuda.set_device(0)
    log(f"[bench] device: {torch.cuda.get_device_name(0)}")
    out = bench_q1(args, gd, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
