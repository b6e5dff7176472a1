#!/usr/bin/env python3
"""Benchmark of the block-quantized GEMV/GEMM hot path on one MI355X.

Default workload (the headline metric): Q1_0.q8_0 GEMV at 8B-class decode
shapes, batch 1 -- weights 4096x4096 and 14336x4096 (K=4096), each applied to
32 seeded q8_0 activation vectors as separate batch-1 GEMVs. One step is those
64 GEMVs, run as ONE grouped launch (64 independent problems, each with its
own row count). Every problem reads its own copy of the repacked weight
planes, and successive steps rotate through a ring of copies totalling more
than 1 GiB, so no weight byte is served from cache (MI355X has a 256 MB
last-level cache): each step streams 342 MB of algorithmic bytes from HBM.

Timing: after the warmup, R batches (--batches) of exactly K steps
(--steps), each batch between two HIP events on the launch stream with a
device synchronisation on both sides; the reported value and ms_per_step
come from the median batch (min and max are printed beside it). The other
paths are timed the same way: R batches of graph replays, median.

Printed: ONE compact JSON line on stdout (the metric, the roofline of the
dominant kernel, the CPU oracle timed on a bounded sample of the same
workload, and one short entry per other path under "workloads"); the full
record, with the samples' descriptions, goes to stderr and to --detail-out.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--batches R]
                       [--workload all|q1|...]
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
MFMA_F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 matrix peak
MODEL_8B_Q1_BYTES = 8e9 * 18 / 128   # 8B weights at 18 bytes per 128 -> bytes per token
METRIC = "Q1_0·q8_0 GEMV effective HBM GB/s (% of peak) + equiv tok/s, batch 1"
TRAFFIC_SOURCE = ("copied from profiles/hbm_traffic_all_paths.md: rocprofv3 --pmc FETCH_SIZE then WRITE_SIZE "
                  "on this kernel source, scaled by a streaming read and a fill of known size")
MIN_SPIN_S = 0.1       # sustained load before each short-kernel timing
MIN_BATCH_S = 0.02     # GPU time per timed batch of the other paths


# HBM bytes per launch from rocprofv3 counters (2 x FETCH_SIZE + WRITE_SIZE,
# in KiB, the factors read off a streaming read and a fill of known size),
# valid for the kernel source they were measured on: reported only while its
# hash matches, null after any change to it.
_TRAFFIC = {
    "q1": ("q1.hip", "6594bcff4a7b6f83", {"step": (170022.2, 2304.0)}),
    "q1_small": ("q1.hip", "6594bcff4a7b6f83", {"7646 x 256x1024": (138464.3, 7646.0)}),
    "q1mm": ("q1.hip", "6594bcff4a7b6f83", {"m2": (4307.5, 112.0), "m4": (4329.5, 224.0), "m8": (4397.5, 448.0)}),
    "ternary": ("ternary.hip", "126a8cf5dd046c1e",
                {"2560x2560": (101698.1, 1200.0), "6912x2560": (137148.8, 1620.0), "2560x6912": (65832.9, 300.0)}),
    "blockq8": ("blockq8.hip", "f40db311846149b4", {"m1": (26849.6, 192.5), "m16": (27505.1, 3072.0)}),
    # per call on the caller's words: prep (split + weight regroup) + gemm
    "sign": ("sign_gemm.hip", "65273486dc365ea0",
             {"prep": (6189.5, 12432.0), "gemm": (20668.0, 8192.0)}),
    "sign_lut": ("sign_lut.hip", "5495a8b23da9304f",
                 {"4096x4096": (2151.5, 16.0), "14336x4096": (7296.6, 56.0), "lut4": (35130.5, 8192.0)}),
    "quant": ("quantize.hip", "43e80662c6c5dcbe",
              {"q8_0_decode": (266.5, 136.0), "q8_0_batch_256MiB": (131082.9, 69632.0),
               "int8_planes_decode_step": (488.5 + 480.8, 227.8 + 203.4),
               "int8_planes_batch_256MiB": (131110.9, 66066.3)}),
    # per call: split kernel + merge kernel
    "attention": ("attention.hip", "849b98fd33aa133e",
                  {"kv4096": (16453.1 + 605.0, 1040.0 + 16.0),
                   "kv32768": (131141.2 + 605.0, 1040.0 + 16.0)}),
}

# Hardware MFMA busy fraction (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over the
# dispatch's duration x 1024 SIMDs at 2.4 GHz), for the kernel source measured.
_MFMA_BUSY = {
    "sign_gemm_kernel": ("sign_gemm.hip", "65273486dc365ea0", 0.474),
    "blockq8_mfma_kernel": ("blockq8.hip", "f40db311846149b4", 0.077),
}


def _src_sha(src: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, "gemm_decode_amd", "csrc", src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_mfma_busy(kernel: str):
    """The counter-measured MFMA busy fraction of a kernel, or None if its
    source has changed since."""
    src, sha, frac = _MFMA_BUSY[kernel]
    return frac if _src_sha(src) == sha else None


def measured_traffic(path: str):
    """{launch: HBM bytes} for one path, or None if its source has changed."""
    src, sha, launches = _TRAFFIC[path]
    if _src_sha(src) != sha:
        return None
    return {k: int(round((2.0 * fetch + write) * 1024)) for k, (fetch, write) in launches.items()}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def q1_gemv_bytes(rows: int, K: int) -> int:
    """Algorithmic bytes of one batch-1 GEMV: each weight byte once (18 bytes
    per 128 weights), the q8_0 activation once (34 per 32), the f32 output."""
    return rows * (K // 128) * 18 + (K // 32) * 34 + rows * 4


def _r(v, nd=2):
    return None if v is None else round(float(v), nd)


def roofline(achieved, peak, unit, bound, traffic=None, **extra):
    out = {"bound": bound, "achieved": _r(achieved, 2), "peak": peak, "unit": unit,
           "frac": _r(achieved / peak, 4), "traffic": traffic}
    out.update(extra)
    return out


def compact(full: dict) -> dict:
    """The short form of one path's record for the stdout line: value, unit,
    time, roofline fraction, traffic, parity, CPU baseline."""
    rf = full.get("roofline") or {}
    cpu = full.get("cpu_baseline") or {}
    out = {"value": full.get("value"), "unit": full.get("unit"), "us": full.get("us"),
           "bound": rf.get("bound"), "frac": rf.get("frac"), "traffic": rf.get("traffic")}
    if rf.get("mfma_busy_hw") is not None:
        out["mfma_busy_hw"] = rf["mfma_busy_hw"]
    for k in ("parity_mismatches", "parity_rel_err"):
        if k in full:
            out[k] = full[k]
    if cpu:
        out["cpu"] = {"value": cpu.get("value"), "unit": cpu.get("unit"), "cores": cpu.get("cores")}
    for k in ("spread_us", "extra"):
        if k in full:
            out[k] = full[k]
    return out


def with_floor(rec: dict, floor_us: float) -> dict:
    """A decode-size entry with its time as a multiple of the launch floor."""
    if rec.get("us") is not None and floor_us > 0:
        rec["x_launch_floor"] = _r(rec["us"] / floor_us, 2)
    return rec


# ----------------------------------------------------------------- timing

def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def spin_up(torch, run, n_min, min_s):
    """Runs run(n_min), then run(n_min) again until at least min_s seconds of
    GPU work have passed; returns the number of run() units done (untimed)."""
    done = 0
    t = time.perf_counter()
    while True:
        run(n_min)
        torch.cuda.synchronize()
        done += n_min
        if time.perf_counter() - t >= min_s:
            return done


def time_batches(torch, run_batch, units, batches):
    """Seconds per unit of `batches` timed batches: each batch is run_batch()
    (which enqueues `units` units of work on the current stream) between two
    HIP events on that stream, with a device synchronisation on both sides.
    Returns (median, min, max, all) in seconds per unit."""
    per = []
    for _ in range(batches):
        torch.cuda.synchronize()
        e0, e1 = _events(torch)
        e0.record()
        run_batch()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / 1e3 / units)
    arr = np.array(per)
    return float(np.median(arr)), float(arr.min()), float(arr.max()), per


def _time_launches(torch, launch, n, warmup, batches):
    """Per-launch time of n launches captured in one HIP graph (replayed on
    the launch stream, so the launches run back to back whatever the host's
    launch rate). The graph is replayed untimed for MIN_SPIN_S first (the
    clocks leave idle); then `batches` timed batches, each of as many
    replays as make up MIN_BATCH_S of GPU time. Returns (median s per launch,
    {"min_us", "max_us", "batches", "launches_per_batch"})."""
    for w in range(warmup):
        launch(w)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for k in range(n):
            launch(warmup + k)
    spin_up(torch, lambda _n: g.replay(), 1, MIN_SPIN_S)
    e0, e1 = _events(torch)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    one = e0.elapsed_time(e1) / 1e3
    reps = max(1, int(np.ceil(MIN_BATCH_S / max(one, 1e-7))))

    def batch():
        for _ in range(reps):
            g.replay()
    med, lo, hi, _ = time_batches(torch, batch, reps * n, batches)
    del g
    return med, {"min_us": _r(lo * 1e6, 3), "max_us": _r(hi * 1e6, 3), "batches": batches,
                 "launches_per_batch": reps * n}


def measured_launch_floor(gd, torch, batches: int):
    """Per-launch time of a trivial kernel (a 4 KiB fill) replayed 64 times in
    a HIP graph: the floor under any one launch on this machine, against which the
    latency-bound decode-size launches are read. Returns (us, timing)."""
    buf = torch.empty(4096, dtype=torch.uint8, device="cuda")
    per, st = _time_launches(torch, lambda k: gd.gemm_decode_fill(buf, k + 1), 64, 3, batches)
    return per * 1e6, st


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
        e0, e1 = _events(torch)
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

def q1_step_problems(gd, shapes, copies, a_dev, ys):
    """The decode step's problems in the order of its one grouped launch:
    shapes by increasing row count (the longer problems' work then fills the
    launch's tail), activation vector c against each. copies[si][c] are the
    (bits, scales) planes of problem (shape si, vector c), ys[si][c] its
    output; each problem carries its own row count."""
    order = sorted(range(len(shapes)), key=lambda si: shapes[si].rows)
    return gd.make_q1_problems([(copies[si][c][0], copies[si][c][1], a_dev[c], ys[si][c], shapes[si].rows)
                                for si in order for c in range(len(a_dev))])


def q1_step_launch(gd, problems, shapes, n_vec):
    """One decode step: its len(shapes) * n_vec problems in one grouped
    launch, the launch's rows the largest problem's."""
    gd.q1_q8_gemv_grouped(problems, len(shapes) * n_vec, max(s.rows for s in shapes), shapes[0].K)


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
    slots = []
    for r in range(ring):
        copies = [[(base[si][0].clone(), base[si][1].clone()) for _ in range(n_vec)] for si in range(len(shapes))]
        slots.append({"step": q1_step_problems(gd, shapes, copies, a_dev, ys), "copies": copies})
    torch.cuda.synchronize()

    def step(r):
        q1_step_launch(gd, slots[r]["step"], shapes, n_vec)

    # parity check (untimed): every output of the first ring slot
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

    # Timed steps: the launches are queued back to back from the host with
    # no event between them (the GPU runs them without gaps). --graph
    # replays HIP graphs instead: one graph per full ring cycle (`ring`
    # steps), one-step graphs per slot for a remainder.
    cap = torch.cuda.Stream()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            fn()
        return g

    if args.graph:
        ring_graph = capture(lambda: [step(r) for r in range(ring)])
        slot_graphs = [capture(lambda r=r: step(r)) for r in range(ring)]
        torch.cuda.synchronize()

    pos = [0]   # ring position, carried across batches

    def run_steps(n):
        if not args.graph:
            for _ in range(n):
                step(pos[0] % ring)
                pos[0] += 1
            return
        for _ in range(n // ring):
            ring_graph.replay()
        for _ in range(n % ring):
            slot_graphs[pos[0] % ring].replay()
            pos[0] += 1

    # Untimed warmup: at least W steps, and at least --min-warmup-s of
    # sustained load (the clocks take tens of milliseconds to ramp from idle;
    # a warmup of a few steps would time that ramp).
    warm_steps = spin_up(torch, run_steps, max(args.warmup, ring), args.min_warmup_s)

    # R batches of exactly K steps; the median batch is the result.
    wall0 = time.perf_counter()
    med, lo, hi, per_batch = time_batches(torch, lambda: run_steps(args.steps), args.steps, args.batches)
    wall = time.perf_counter() - wall0
    gbps = step_bytes / med / 1e9
    q1_traffic = measured_traffic("q1")

    # serial mode: one launch per GEMV (the decode schedule), the step's 64
    # launches captured in a HIP graph per ring slot and replayed back to back
    serial = None
    if args.serial_steps > 0:
        def one_step(r):
            for si, s in enumerate(shapes):
                for c in range(n_vec):
                    b, sc = slots[r]["copies"][si][c]
                    gd.q1_q8_gemv(b, sc, a_dev[c], ys[si][c], s.rows, s.K, 1)
        one_step(0)
        torch.cuda.synchronize()
        sgraphs = []
        for r in range(ring):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                one_step(r)
            sgraphs.append(g)
        spin_up(torch, lambda n: [sgraphs[k % ring].replay() for k in range(n)], ring, MIN_SPIN_S)
        spos = [0]

        def sbatch():
            for _ in range(args.serial_steps):
                sgraphs[spos[0] % ring].replay()
                spos[0] += 1
        smed, slo, shi, _ = time_batches(torch, sbatch, args.serial_steps, args.batches)
        serial = {"value": _r(step_bytes / smed / 1e9, 1), "unit": "GB/s",
                  "us_per_gemv": _r(smed / (2 * n_vec) * 1e6, 3),
                  "us_per_gemv_min_max": [_r(slo / (2 * n_vec) * 1e6, 3), _r(shi / (2 * n_vec) * 1e6, 3)],
                  "timing": f"one HIP graph of the step's 64 single-GEMV launches per ring slot; "
                            f"median of {args.batches} batches of {args.serial_steps} steps"}
        del sgraphs

    ceiling = (measured_read_ceiling(gd, torch, gib=args.ceiling_gib, passes=args.ceiling_passes,
                                     reps=args.ceiling_reps) if args.ceiling else None)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_q1(Ws, A, shapes, budget_s=args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": _r(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": _r(med * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Q1_0.q8_0 GEMV batch 1: 32 activation vectors x {4096x4096, 14336x4096}, "
                        "K=4096, 64 independent GEMVs per step in one grouped launch, "
                        "distinct weight copies (ring > 1 GiB)",
            "step_bytes": step_bytes, "ring_sets": ring,
            "timed_as": (f"HIP graph replays ({ring} steps per graph)" if args.graph
                         else "launches queued back to back, events only at a batch's ends"),
        },
        "batches": {"n": args.batches, "steps_each": args.steps, "ms_per_step_median": _r(med * 1e3, 5),
                    "ms_per_step_min": _r(lo * 1e3, 5), "ms_per_step_max": _r(hi * 1e3, 5),
                    "GBps_min_max": [_r(step_bytes / hi / 1e9, 1), _r(step_bytes / lo / 1e9, 1)]},
        "warmup_steps_run": warm_steps,
        "pct_of_peak": _r(100 * gbps / HBM_PEAK_GBPS, 2),
        "equiv_tok_s": _r(gbps * 1e9 / MODEL_8B_Q1_BYTES, 1),
        "rows_K_per_s": _r(sum(n_vec * s.rows * s.K for s in shapes) / med, 1),
        "roofline": roofline(gbps, HBM_PEAK_GBPS, "GB/s", "hbm",
                             None if q1_traffic is None else q1_traffic["step"],
                             traffic_source=TRAFFIC_SOURCE if q1_traffic else None,
                             kernel="q1_gemv_grouped2_kernel<4, 3>", us_per_launch=_r(med * 1e6, 2),
                             bytes_per_launch=step_bytes,
                             timing=f"HIP events on the launch stream around each batch of {args.steps} "
                                    f"back-to-back launches (one per step); median of {args.batches} batches"),
        "parity_mismatches": mism,
        "serial_one_launch_per_gemv": serial,
        "read_ceiling_GBps": _r(ceiling, 1),
        "cpu_baseline": cpu,
        "wall_s_timed": _r(wall, 4),
    }
    log(f"[bench] q1: {gbps:.1f} GB/s median ({step_bytes / hi / 1e9:.1f}-{step_bytes / lo / 1e9:.1f}), "
        f"{med * 1e6:.2f} us per step; batches (us/step): " + ", ".join(f"{p * 1e6:.2f}" for p in per_batch))
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
    # the same GEMVs on one thread, for a quarter of the budget
    one_bytes, one_used, n_one = 0, 0.0, 0
    while one_used < budget_s / 4:
        c, si = order[n_one % len(order)]
        s = shapes[si]
        t = time.perf_counter()
        oracle.q1_q8_gemv_aos(Ws[si], A[c], s.rows, s.K, 1, nthreads=1)
        one_used += time.perf_counter() - t
        one_bytes += q1_gemv_bytes(s.rows, s.K)
        n_one += 1
    return {"value": _r(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_gemv} batch-1 GEMVs of the step, {t_used:.1f} s, OpenMP over rows",
            "cpu_model": cpu_model(),
            "single_thread": {"value": _r(one_bytes / one_used / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{n_one} of the same GEMVs, {one_used:.1f} s"}}


# ---------------------------------------- Q1 correctness-sized (256 x 1024)

def bench_q1_small(args, gd, torch):
    """Q1_0.q8_0 GEMV rows=256, K=1024, batch 1 (the correctness-sized
    config; 38,976 algorithmic bytes per GEMV). (G): independent problems in
    grouped launches, each reading its own copy of the planes, the copies
    rotating over a ring > 1 GiB: the streaming figure; the problems share
    one activation vector, counted once per launch. (S): one launch per
    GEMV, back to back from a HIP graph: the latency figure."""
    import oracle
    cfg = wl.Q1_SMALL
    rows, K = cfg.rows, cfg.K
    W = wl.q1_weights_aos(rows, K, cfg.weight_seed)
    A = wl.q8_acts_aos(K, cfg.act_seeds[0])
    bb, sb = gd.q1_planes_bytes(rows, K)
    b0, s0 = gd.q1_alloc_planes(rows, K)
    gd.q1_repack(torch.from_numpy(W.reshape(-1)).cuda(), rows, K, b0, s0)
    a = torch.from_numpy(np.ascontiguousarray(A.reshape(-1))).cuda()
    gemv_bytes = q1_gemv_bytes(rows, K)
    sets = 4
    count = int(np.ceil(1.05 * (1 << 30) / (sets * (bb + sb))))      # problems per launch
    bits = [b0.repeat(count) for _ in range(sets)]
    scl = [s0.repeat(count) for _ in range(sets)]
    ys = [torch.empty(count * rows, device="cuda") for _ in range(sets)]
    probs = [gd.make_q1_problems([(bits[t][i * bb:(i + 1) * bb], scl[t][i * sb:(i + 1) * sb], a,
                                   ys[t][i * rows:(i + 1) * rows]) for i in range(count)]) for t in range(sets)]
    torch.cuda.synchronize()

    def grouped(kk):
        gd.q1_q8_gemv_grouped(probs[kk % sets], count, rows, K)
    per_g, st_g = _time_launches(torch, grouped, sets, sets, args.batches)
    # every output of every problem, bit for bit
    want = oracle.q1_q8_gemv_aos(W, A, rows, K).view(np.uint32).reshape(-1)
    mism = 0
    for t in range(sets):
        got = ys[t].cpu().numpy().view(np.uint32).reshape(count, rows)
        mism += int((got != want[None, :]).sum())
    ys1 = torch.empty(rows, device="cuda")
    stride = max(1, count // 64)

    def single(kk):
        t, i = kk % sets, (kk * stride) % count
        gd.q1_q8_gemv(bits[t][i * bb:(i + 1) * bb], scl[t][i * sb:(i + 1) * sb], a, ys1, rows, K, 1)
    per_s, st_s = _time_launches(torch, single, 64, 4, args.batches)
    mism += int((ys1.cpu().numpy().view(np.uint32) != want).sum())
    # the launch's algorithmic bytes: every problem's weights and output, and
    # the one activation vector all of them share, once
    act_bytes = (K // 32) * 34
    launch_bytes = count * (gemv_bytes - act_bytes) + act_bytes
    g_gbps = launch_bytes / per_g / 1e9
    small_traffic = measured_traffic("q1_small")
    threads = cpu_cores()
    t_used, n_g = 0.0, 0
    while t_used < args.aux_cpu_seconds:
        t = time.perf_counter()
        oracle.q1_q8_gemv_aos(W, A, rows, K, nthreads=threads)
        t_used += time.perf_counter() - t
        n_g += 1
    return {
        "workload": "Q1_0.q8_0 GEMV rows=256, K=1024, batch 1",
        "metric": "effective HBM GB/s (grouped: independent problems, ring > 1 GiB)",
        "value": _r(g_gbps, 1), "unit": "GB/s", "us": _r(per_g * 1e6, 2),
        "problems_per_launch": count, "ring_copies": sets * count, "timing": st_g,
        "extra": {"single_launch_us": _r(per_s * 1e6, 3)},
        "single_launch": {"us_per_gemv": _r(per_s * 1e6, 3), "GB_per_s": _r(gemv_bytes / per_s / 1e9, 1),
                          "timing": st_s, "note": "64 launches in a graph; latency-bound (a 39 KB GEMV)"},
        "roofline": roofline(g_gbps, HBM_PEAK_GBPS, "GB/s", "hbm",
                             (None if small_traffic is None or count != 7646
                              else small_traffic["7646 x 256x1024"]),
                             kernel="q1_gemv_grouped_small2_kernel<2>", bytes_per_launch=launch_bytes),
        "parity_mismatches": mism,
        "cpu_baseline": {"value": _r(n_g * gemv_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": threads,
                         "kind": "oracle", "sample": f"{n_g} GEMVs of 256x1024, {t_used:.2f} s"},
    }


# ------------------------------------------- Q1 small-M (several columns)

def bench_q1_mm(args, gd, torch):
    """Q1_0.q8_0 with several activation columns (P1's multi-column Q1_MM,
    the prompt side of the same method) on the 14336x4096 decode weight: one
    launch, each column its own GEMV with the bits of its batch-1 result.
    Weight copies rotate over a ring > 1 GiB (one graph of launches covers
    the whole ring, so no copy is read again from cache)."""
    import oracle
    cfg = wl.Q1_DECODE[1]
    rows, K = cfg.rows, cfg.K
    W = wl.q1_weights_aos(rows, K, cfg.weight_seed)
    b0, s0 = gd.q1_alloc_planes(rows, K)
    gd.q1_repack(torch.from_numpy(W.reshape(-1)).cuda(), rows, K, b0, s0)
    plane = sum(gd.q1_planes_bytes(rows, K))
    ring = max(2, int(np.ceil(1.05 * (1 << 30) / plane)))
    copies = [(b0.clone(), s0.clone()) for _ in range(ring)]
    w_bytes = rows * (K // 128) * 18
    threads = cpu_cores()
    mt = measured_traffic("q1mm")
    out = {}
    for M in (2, 4, 8):
        A = np.concatenate([wl.q8_acts_aos(K, sd) for sd in cfg.act_seeds[:M]])
        a = torch.from_numpy(np.ascontiguousarray(A.reshape(-1))).cuda()
        y = torch.empty(M * rows, device="cuda")

        def launch(k, a=a, y=y, M=M):
            bb, ss = copies[k % ring]
            gd.q1_q8_gemv(bb, ss, a, y, rows, K, M)
        per, st = _time_launches(torch, launch, ring, 3, args.batches)
        got = y.cpu().numpy().reshape(M, rows)
        t = time.perf_counter()
        want = oracle.q1_q8_gemv_aos(W, A, rows, K, n_act=M, nthreads=threads)   # every output
        t_cpu = time.perf_counter() - t
        mism = int((got.view(np.uint32) != want.reshape(M, -1).view(np.uint32)).sum())
        launch_bytes = w_bytes + M * ((K // 32) * 34 + rows * 4)
        out[f"m{M}"] = {
            "workload": f"Q1_0.q8_0 small-M: {M} activation columns x 14336x4096 weight",
            "metric": "HBM GB/s (weight bytes counted once)", "value": _r(launch_bytes / per / 1e9, 1), "unit": "GB/s",
            "us": _r(per * 1e6, 2), "timing": st,
            "gemv_equivalent_GBps": _r(M * q1_gemv_bytes(rows, K) / per / 1e9, 1),
            "roofline": roofline(launch_bytes / per / 1e9, HBM_PEAK_GBPS, "GB/s", "hbm",
                                 None if mt is None else mt[f"m{M}"],
                                 kernel=("q1_gemv_kernel<256> (128-row workgroups, one grid row per column)"
                                         if M == 2 else "q1_gemv_kernel<512> (one grid row per column)"),
                                 bytes_per_launch=launch_bytes),
            "parity_mismatches": mism,
            "cpu_baseline": {"value": _r(M * q1_gemv_bytes(rows, K) / t_cpu / 1e9, 4),
                             "unit": "GB/s (GEMV-equivalent)", "cores": threads, "kind": "oracle",
                             "sample": f"all {rows} rows x {M} columns, {t_cpu:.2f} s"},
        }
    return out


# ------------------------------------------------- sign-bit GEMM (prefill)

def bench_sign(args, gd, torch):
    """Sign-bit prefill GEMM y = x @ w^T, M=512 tokens, N=4096, K=4096: MFMA
    roofline on the useful 2MNK flops."""
    import oracle
    c = wl.SIGN_PREFILL
    M, N, K = c["M"], c["N"], c["K"]
    x, bits, scales = wl.sign_gemm_inputs(M, N, K, c["seed"])
    set_bytes = x.nbytes + bits.nbytes + scales.nbytes + M * N * 4
    ring = max(2, int(np.ceil(0.5 * (1 << 30) / set_bytes)))
    xs = torch.from_numpy(x).cuda()
    bs = torch.from_numpy(bits.view(np.int32)).cuda()
    ss = torch.from_numpy(scales).cuda()
    sets = [(xs.clone(), bs.clone(), ss.clone(), torch.empty(M * N, device="cuda")) for _ in range(ring)]

    def launch(k):
        a, b, s_, y = sets[k % ring]
        gd.q1_sign_gemm(a, b, s_, y, M, N, K)
    per, st = _time_launches(torch, launch, ring, 3, args.batches)
    flops = 2.0 * M * N * K
    tflops = flops / per / 1e12
    sg_traffic = measured_traffic("sign")
    # parity: every output of the last launched set against the f64 oracle
    y = sets[(3 + ring - 1) % ring][3].cpu().numpy().reshape(M, N)
    threads = cpu_cores()
    t = time.perf_counter()
    want = oracle.sign_gemm_f64(x, bits, scales, nthreads=threads)
    t_full = time.perf_counter() - t
    rel = float(np.max(np.abs(y - want)) / np.max(np.abs(want)))

    # the same GEMM on weights packed once (q1_sign_pack), and the LUT4
    # comparator on those packed weights
    packed = []
    for a, b, s_, yy in sets:
        wp = torch.empty(gd.q1_sign_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
        gd.q1_sign_pack(b, s_, N, K, wp)
        packed.append((a, wp, yy))

    def launch_packed(k):
        a, wp, yy = packed[k % ring]
        gd.q1_sign_gemm_packed(a, wp, yy, M, N, K)
    per_p, st_p = _time_launches(torch, launch_packed, ring, 3, args.batches)
    y_p = packed[(3 + ring - 1) % ring][2].cpu().numpy().reshape(M, N)
    rel_p = float(np.max(np.abs(y_p - want)) / np.max(np.abs(want)))

    def launch_lut(k):
        a, wp, yy = packed[k % ring]
        gd.q1_sign_gemm_lut4(a, wp, yy, M, N, K)
    per_l, st_l = _time_launches(torch, launch_lut, ring, 1, args.batches)
    y_l = packed[(1 + ring - 1) % ring][2].cpu().numpy().reshape(M, N)
    rel_l = float(np.max(np.abs(y_l - want)) / np.max(np.abs(want)))
    decode = bench_sign_gemv(args, gd, torch)
    busy = measured_mfma_busy("sign_gemm_kernel")
    return {
        "workload": "sign-bit prefill GEMM y=x@w^T, M=512, N=4096, K=4096, x f32 (fp16 hi+lo on MFMA)",
        "metric": "useful TFLOP/s (2MNK)", "value": _r(tflops, 2), "unit": "TFLOP/s",
        "us": _r(per * 1e6, 2), "timing": st, "prefill_tok_s": _r(M / per, 1),
        "roofline": roofline(tflops, MFMA_F16_PEAK_TFLOPS, "TFLOP/s", "mfma",
                             None if sg_traffic is None else sum(sg_traffic.values()),
                             traffic_per_kernel=sg_traffic,
                             kernel="q1_sign_gemm call (all its kernels)",
                             flops_per_launch=flops, mfma_busy_hw=busy,
                             mfma_issued_per_useful=3),
        "parity_rel_err": rel,
        "cpu_baseline": {"value": _r(flops / t_full / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
                         "kind": "oracle", "sample": f"all 512 x 4096 outputs (f64 oracle), {t_full:.2f} s"},
        "extra": {"packed_us": _r(per_p * 1e6, 2), "packed_frac": _r(flops / per_p / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                  "lut4_us": _r(per_l * 1e6, 2)},
        "packed_weights": {"note": "weights packed once by q1_sign_pack; per call: the remaining kernels",
                           "us_per_gemm": _r(per_p * 1e6, 2), "value": _r(flops / per_p / 1e12, 2),
                           "unit": "TFLOP/s", "frac": _r(flops / per_p / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                           "timing": st_p, "parity_rel_err": rel_p},
        "lut4_comparator": {"note": "the page's LUT4 prefill (table lookup, VALU + LDS), packed weights",
                            "us_per_gemm": _r(per_l * 1e6, 2), "value": _r(flops / per_l / 1e12, 2),
                            "unit": "TFLOP/s", "vs_mfma_packed": _r(per_l / per_p, 2), "timing": st_l,
                            "traffic": (None if measured_traffic("sign_lut") is None
                                        else measured_traffic("sign_lut")["lut4"]),
                            "parity_rel_err": rel_l},
        "decode_gemv": decode,
    }


def bench_sign_gemv(args, gd, torch):
    """Sign-bit decode GEMV (M=1) on packed weights at the 8B-class decode
    shapes, one launch per GEMV over a ring of weight copies > 1 GiB (one
    graph covers the ring); HBM roofline on the packed weight bytes + x + y."""
    import oracle
    out = {}
    lt = measured_traffic("sign_lut")
    for N, K in ((4096, 4096), (14336, 4096)):
        x, bits, scales = wl.sign_gemm_inputs(1, N, K, seed=N + K)
        wbytes = N * K // 4        # 1 bit + 1/32 of an f32 per weight
        ring = max(2, int(np.ceil(1.05 * (1 << 30) / wbytes)))
        bd = torch.from_numpy(bits.view(np.int32)).cuda()
        sd = torch.from_numpy(scales).cuda()
        wp0 = torch.empty(gd.q1_sign_packed_bytes(N, K), dtype=torch.uint8, device="cuda")
        gd.q1_sign_pack(bd, sd, N, K, wp0)
        copies = [wp0] + [wp0.clone() for _ in range(ring - 1)]
        xd = torch.from_numpy(x).cuda()
        y = torch.empty(N, device="cuda")

        def launch(k):
            gd.q1_sign_gemv(xd, copies[k % ring], y, 1, N, K)
        per, st = _time_launches(torch, launch, ring, 4, args.batches)
        bytes_ = wbytes + K * 4 + N * 4
        got = y.cpu().numpy()
        want = oracle.sign_gemm_f64(x, bits, scales, nthreads=cpu_cores())[0]
        out[f"{N}x{K}"] = {
            "us": _r(per * 1e6, 2), "value": _r(bytes_ / per / 1e9, 1), "unit": "GB/s", "timing": st,
            "roofline": roofline(bytes_ / per / 1e9, HBM_PEAK_GBPS, "GB/s", "hbm",
                                 None if lt is None else lt[f"{N}x{K}"], kernel="sign_gemv_narrow_kernel<16>" if N <= 8192 else "sign_gemv_kernel",
                                 bytes_per_launch=bytes_),
            "parity_rel_err": float(np.max(np.abs(got - want)) / np.max(np.abs(want))),
        }
        del copies
    return out


# ------------------------------------------------------ block-Q8 matmul_nt

def bench_blockq8(args, gd, torch):
    """Block-Q8 matmul_nt k=960, n=49152 at m=1 and m=16: HBM roofline on the
    algorithmic bytes (quants + scales once, x once, y once)."""
    import oracle
    c = wl.BLOCKQ8_LMHEAD
    k, n = c["k"], c["n"]
    out = {}
    x_all, quants, scales = wl.blockq8_inputs(16, k, n, c["seed"])
    w_bytes = quants.nbytes + scales.nbytes
    ring = max(2, int(np.ceil(1.05 * (1 << 30) / w_bytes)))
    qd = torch.from_numpy(quants.view(np.int32)).cuda()
    sd = torch.from_numpy(scales).cuda()
    copies = [(qd.clone(), sd.clone()) for _ in range(ring)]
    bq_traffic = measured_traffic("blockq8")
    threads = cpu_cores()
    for m in c["ms"]:
        x = np.ascontiguousarray(x_all[:m])
        xd = torch.from_numpy(x).cuda()
        y = torch.empty(m * n, device="cuda")

        def launch(kk):
            q_, s_ = copies[kk % ring]
            gd.blockq8_matmul_nt(xd, q_, s_, y, m, k, n)
        per, st = _time_launches(torch, launch, ring, 3, args.batches)
        bytes_ = w_bytes + x.nbytes + m * n * 4
        gbps = bytes_ / per / 1e9
        got = y.cpu().numpy().reshape(m, n)
        t = time.perf_counter()
        want = oracle.blockq8_f32(x, quants, scales, nthreads=threads)   # every output
        t_cpu = time.perf_counter() - t
        rel = float(np.max(np.abs(got - want)) / np.max(np.abs(want)))
        out[f"m{m}"] = {
            "workload": f"block-Q8 matmul_nt k=960 n=49152 m={m}",
            "metric": "effective HBM GB/s", "value": _r(gbps, 1), "unit": "GB/s",
            "us": _r(per * 1e6, 2), "timing": st,
            "roofline": roofline(gbps, HBM_PEAK_GBPS, "GB/s", "hbm",
                                 None if bq_traffic is None else bq_traffic[f"m{m}"],
                                 kernel="blockq8_gemv_kernel" if m == 1 else "blockq8_mfma_kernel<32>",
                                 bytes_per_launch=bytes_,
                                 mfma_busy_hw=None if m == 1 else measured_mfma_busy("blockq8_mfma_kernel")),
            "parity_rel_err": rel,
            "cpu_baseline": {"value": _r(bytes_ / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads,
                             "kind": "oracle", "sample": f"all 49152 output features, m={m}, {t_cpu:.2f} s"},
        }
    return out


# ------------------------------------------------- activation quantization

def bench_quant(args, gd, torch):
    """On-device activation quantization (the step before each GEMV): q8_0
    blocks for the Q1 path and per-token int8 bit planes for the ternary
    path, at decode sizes (launch latency) and at a 256 MiB batch (HBM
    roofline on 4 B read per element plus what is written)."""
    import oracle
    out = {}

    def measure(name, kind, shapes, copies_n):
        """shapes: list of (count, K) launched back to back as one step."""
        sets = []
        for ci in range(copies_n):
            entry = []
            for si, (cnt, K) in enumerate(shapes):
                rng = np.random.default_rng(1000 * ci + si)
                x = torch.from_numpy(rng.standard_normal(size=(cnt, K), dtype=np.float32)).cuda()
                if kind == "q8":
                    o = (torch.empty(cnt * (K // 32) * 34, dtype=torch.uint8, device="cuda"),)
                else:
                    o = (torch.empty(cnt * 8 * (K // 32), dtype=torch.int32, device="cuda"),
                         torch.empty(cnt, device="cuda"))
                entry.append((x, o))
            sets.append(entry)

        def launch(kk):
            for (cnt, K), (x, o) in zip(shapes, sets[kk % copies_n]):
                if kind == "q8":
                    gd.q8_0_quantize(x, o[0], cnt, K)
                else:
                    gd.ternary_quantize_act(x, cnt, K, o[0], o[1])
        per, st = _time_launches(torch, launch, max(args.aux_steps, copies_n), 2, args.batches)
        bytes_ = sum(cnt * K * 4 + (cnt * (K // 32) * 34 if kind == "q8" else cnt * (K + 4)) for cnt, K in shapes)
        gbps = bytes_ / per / 1e9
        # parity on the first rows of the first set (an oracle sample, also
        # timed as the CPU baseline)
        mism = 0
        t_used, done_bytes = 0.0, 0
        for (cnt, K), (x, o) in zip(shapes, sets[0]):
            r = min(cnt, 64)
            xs = x[:r].cpu().numpy()
            t = time.perf_counter()
            if kind == "q8":
                want = oracle.quantize_q8_0(xs)
                t_used += time.perf_counter() - t
                mism += int(np.count_nonzero(o[0][:r * (K // 32) * 34].cpu().numpy() != want))
                done_bytes += r * K * 4 + r * (K // 32) * 34
            else:
                q, sc = oracle.quantize_absmax_int8(xs)
                t_used += time.perf_counter() - t
                got_s = o[1][:r].cpu().numpy()
                u = q.view(np.uint8).astype(np.uint32).reshape(r, K // 32, 32)
                planes = np.stack([(((u >> b) & 1) << np.arange(32, dtype=np.uint32)).sum(axis=2)
                                   for b in range(8)], axis=1).astype(np.uint32)
                got_p = o[0][:r * 8 * (K // 32)].cpu().numpy().view(np.uint32).reshape(r, 8, K // 32)
                mism += int(np.count_nonzero(got_p != planes)) + int(np.count_nonzero(got_s != sc))
                done_bytes += r * K * 4 + r * (K + 4)
        out[name] = {
            "workload": " + ".join(f"{cnt}x{K}" for cnt, K in shapes) + (" f32 -> q8_0" if kind == "q8"
                                                                           else " f32 -> int8 planes"),
            "metric": "effective HBM GB/s", "value": _r(gbps, 1), "unit": "GB/s",
            "us": _r(per * 1e6, 2), "timing": st, "launches_per_step": len(shapes),
            "roofline": roofline(gbps, HBM_PEAK_GBPS, "GB/s", "hbm", None if qt is None else qt[name],
                                 kernel="q8_0_quantize_kernel" if kind == "q8" else "act_quant_kernel",
                                 bytes_per_step=bytes_),
            "parity_mismatches": mism,
            "cpu_baseline": {"value": _r(done_bytes / max(t_used, 1e-9) / 1e9, 4), "unit": "GB/s",
                             "cores": 1, "kind": "oracle",
                             "sample": "first <= 64 rows of each shape, single-threaded oracle"},
        }

    qt = measured_traffic("quant")
    measure("q8_0_decode", "q8", [(32, 4096)], 8)
    measure("q8_0_batch_256MiB", "q8", [(16384, 4096)], 2)
    measure("int8_planes_decode_step", "act", [(90, 2560), (30, 6912)], 8)
    measure("int8_planes_batch_256MiB", "act", [(16384, 4096)], 2)
    return out


# ------------------------------------------------------ decode attention

def bench_attention(args, gd, torch):
    """Split-K decode attention for one token at the 8B-class shape (32 query
    heads, 8 KV heads, head dim 128, f32 caches) at kv_len 4096 and 32768:
    HBM roofline on the K and V rows read once + q + out, over a ring of
    cache copies > 1 GiB."""
    import oracle
    Hq, Hkv, D = 32, 8, 128
    out = {}
    at = measured_traffic("attention")
    for L in (4096, 32768):
        rng = np.random.default_rng(L)
        q = rng.standard_normal((Hq, D), dtype=np.float32)
        k = rng.standard_normal((Hkv, L, D), dtype=np.float32)
        v = rng.standard_normal((Hkv, L, D), dtype=np.float32)
        set_bytes = 2 * k.nbytes
        ring = max(2, int(np.ceil(1.05 * (1 << 30) / set_bytes)))
        kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
        caches = [(kd, vd)] + [(kd.clone(), vd.clone()) for _ in range(ring - 1)]
        qd = torch.from_numpy(q).cuda()
        o = torch.empty(Hq * D, device="cuda")
        scale = 1.0 / np.sqrt(D)
        ws = torch.empty(gd.attn_decode_workspace_bytes(Hq, Hkv, D, L), dtype=torch.uint8, device="cuda")

        def launch(kk):
            kc, vc = caches[kk % ring]
            gd.attn_decode_splitk(qd, kc, vc, o, Hq, Hkv, D, L, L, scale, 0, ws)
        per, st = _time_launches(torch, launch, max(args.aux_steps, ring), 2, args.batches)
        bytes_ = set_bytes + 2 * Hq * D * 4
        got = o.cpu().numpy().reshape(Hq, D)
        t = time.perf_counter()
        want = oracle.attention_decode(q, k, v, scale)
        t_cpu = time.perf_counter() - t
        out[f"kv{L}"] = {
            "workload": f"decode attention, 1 token, {Hq} query / {Hkv} KV heads, d={D}, kv_len={L}, f32 KV",
            "metric": "effective HBM GB/s", "value": _r(bytes_ / per / 1e9, 1), "unit": "GB/s",
            "us": _r(per * 1e6, 2), "timing": st,
            "roofline": roofline(bytes_ / per / 1e9, HBM_PEAK_GBPS, "GB/s", "hbm",
                                 None if at is None else at[f"kv{L}"],
                                 kernel="attn_split_kernel<4> + attn_merge_kernel", bytes_per_call=bytes_),
            "parity_rel_err": float(np.max(np.abs(got - want)) / np.max(np.abs(want))),
            "cpu_baseline": {"value": _r(bytes_ / t_cpu / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                             "sample": "one whole call (f64 numpy, per head)"},
        }
        del caches
    return out


# ----------------------------------------------------------------- ternary

def bench_ternary(args, gd, torch):
    """BitNet-2B-like ternary decode step: 210 GEMVs (per layer 4 x 2560x2560,
    2 x 6912x2560, 1 x 2560x6912), each with its own activation vector (bit
    planes built on the device inside the step) and its own weight copy."""
    import oracle
    shapes = wl.bitnet_step_shapes()
    groups = {}
    for j, sh in enumerate(shapes):
        groups.setdefault(sh, []).append(j)
    # one weight per shape (copied to every GEMV slot), one activation per GEMV
    base = {}
    for sh in groups:
        P, N, ws, _, _ = wl.ternary_inputs(sh[0], sh[1], wl.TERNARY_SEED_BASE + 1000 + sh[0] + sh[1])
        base[sh] = (P, N, ws)
    xq, xsc = {}, {}
    for j, (rows, K) in enumerate(shapes):
        rng = np.random.default_rng(wl.TERNARY_SEED_BASE + j)
        q, s_ = wl.absmax_int8(rng.standard_normal(K))
        xq[j], xsc[j] = q, s_
    step_w_bytes = sum(2 * base[sh][0].nbytes * len(idx) for sh, idx in groups.items())
    n_sets = 2 if step_w_bytes * 2 > (1 << 30) else int(np.ceil((1 << 30) / step_w_bytes)) + 1
    keep, slots = [], []
    dev_base = {sh: (torch.from_numpy(base[sh][0].view(np.int32)).cuda(),
                     torch.from_numpy(base[sh][1].view(np.int32)).cuda()) for sh in groups}
    x_by_K, planes_by_K, xoff = {}, {}, {}
    for K in sorted({sh[1] for sh in shapes}):
        js = [j for j, sh in enumerate(shapes) if sh[1] == K]
        x_by_K[K] = torch.from_numpy(np.stack([xq[j] for j in js])).cuda()
        planes_by_K[K] = torch.empty(len(js) * 8 * (K // 32), dtype=torch.int32, device="cuda")
        for pos, j in enumerate(js):
            xoff[j] = (K, pos)
    ys = {j: torch.empty(shapes[j][0], device="cuda") for j in range(len(shapes))}
    for sset in range(n_sets):
        per = {}
        for sh, idx in groups.items():
            entries = []
            for j in idx:
                Pd, Nd = dev_base[sh][0].clone(), dev_base[sh][1].clone()
                keep.append((Pd, Nd))
                K, pos = xoff[j]
                W = K // 32
                xp = planes_by_K[K][pos * 8 * W:(pos + 1) * 8 * W]
                entries.append((Pd, Nd, xp, ys[j], None, base[sh][2], xsc[j]))
            per[sh] = gd.make_ternary_problems(entries)
        slots.append(per)
    torch.cuda.synchronize()
    step_bytes = step_w_bytes + sum(shapes[j][1] + shapes[j][0] * 4 + 8 for j in range(len(shapes)))
    pos_ = [0]

    def step():
        sset = slots[pos_[0] % n_sets]
        pos_[0] += 1
        for K, xd in x_by_K.items():
            gd.ternary_act_bitplanes(xd, xd.shape[0], K, planes_by_K[K])
        for sh, idx in groups.items():
            gd.ternary_gemv_grouped(sset[sh], len(idx), sh[0], sh[1])

    spin_up(torch, lambda n: [step() for _ in range(n)], 3, args.min_warmup_s)
    # R batches of steps queued back to back, events only at a batch's ends
    med, lo, hi, _ = time_batches(torch, lambda: [step() for _ in range(args.aux_steps)], args.aux_steps,
                                  args.batches)
    # GEMV kernels alone: each shape's grouped launch, `reps` back to back
    # over the weight sets between two events, median of the batches
    reps = 8
    gemv_s = 0.0
    for sh, idx in groups.items():
        for kk in range(2):
            gd.ternary_gemv_grouped(slots[kk % n_sets][sh], len(idx), sh[0], sh[1])

        def gb(sh=sh, idx=idx):
            for kk in range(reps):
                gd.ternary_gemv_grouped(slots[kk % n_sets][sh], len(idx), sh[0], sh[1])
        gemv_s += time_batches(torch, gb, reps, args.batches)[0]
    # GEMV bytes of a step: both weight planes, the activation planes, y
    gemv_bytes = step_w_bytes + sum(shapes[j][0] * 4 + 8 * (shapes[j][1] // 32) * 4 for j in range(len(shapes)))
    tern_traffic = measured_traffic("ternary")
    gbps = step_bytes / med / 1e9
    # parity: three GEMVs (one per shape), every row, against the oracle
    mism = 0
    for sh, idx in groups.items():
        j = idx[0]
        yo, _ = oracle.ternary_gemv(base[sh][0], base[sh][1], base[sh][2], xq[j], xsc[j], nthreads=cpu_cores())
        mism += int((ys[j].cpu().numpy().view(np.uint32) != yo.view(np.uint32)).sum())
    threads = cpu_cores()
    t_used, done_bytes, n_g = 0.0, 0, 0
    while t_used < args.aux_cpu_seconds:
        j = n_g % len(shapes)
        sh = shapes[j]
        rows = min(sh[0], 512)
        t = time.perf_counter()
        oracle.ternary_gemv(base[sh][0][:rows], base[sh][1][:rows], base[sh][2], xq[j], xsc[j], nthreads=threads)
        t_used += time.perf_counter() - t
        done_bytes += 2 * rows * sh[1] // 8
        n_g += 1
    return {
        "workload": "ternary bitplane decode step: 30 layers x {4x 2560x2560, 2x 6912x2560, 1x 2560x6912} = 210 "
                    "GEMVs, int8 activations as bit planes, P/N weight planes",
        "metric": "effective HBM GB/s (step)", "value": _r(gbps, 1), "unit": "GB/s",
        "us": _r(med * 1e6, 2), "spread_us": [_r(lo * 1e6, 2), _r(hi * 1e6, 2)],
        "equiv_tok_s": _r(1.0 / med, 1), "context_tok_s_at_0.69GB": _r(gbps / 0.69, 1),
        "extra": {"equiv_tok_s": _r(1.0 / med, 1), "gemv_us": _r(gemv_s * 1e6, 2)},
        "roofline": roofline(gemv_bytes / gemv_s / 1e9, HBM_PEAK_GBPS, "GB/s", "hbm",
                             None if tern_traffic is None else sum(tern_traffic.values()),
                             traffic_per_launch=tern_traffic,
                             kernel="ternary_held_grouped_kernel (3 launches per step, one per shape)",
                             bytes_per_step_gemv=gemv_bytes),
        "step_bytes": step_bytes, "ring_sets": n_sets,
        "parity_mismatches": mism,
        "cpu_baseline": {"value": _r(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": threads,
                         "kind": "oracle",
                         "sample": f"{n_g} GEMVs of the step (first 512 rows each), {t_used:.2f} s"},
    }


# --------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="steps per timed batch")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batches", type=int, default=15, help="timed batches (median reported), at least 10")
    ap.add_argument("--min-warmup-s", type=float, default=0.2,
                    help="untimed warmup continues until this much sustained load has run")
    ap.add_argument("--workload", default="all",
                    choices=["all", "q1", "q1small", "q1mm", "sign", "blockq8", "ternary", "quant", "attention"],
                    help="all (default): the Q1 metric line plus the other paths under 'workloads'")
    ap.add_argument("--aux-steps", type=int, default=20, help="launches per graph for the other paths (minimum)")
    ap.add_argument("--aux-cpu-seconds", type=float, default=4.0)
    ap.add_argument("--ring-gib", type=float, default=1.25)
    ap.add_argument("--serial-steps", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-ceiling", dest="ceiling", action="store_false")
    ap.add_argument("--graph", action="store_true",
                    help="time the Q1 steps as HIP graph replays instead of queued launches")
    ap.add_argument("--ceiling-gib", type=float, default=2.0)
    ap.add_argument("--ceiling-passes", type=int, default=8)
    ap.add_argument("--ceiling-reps", type=int, default=5)
    ap.add_argument("--no-parity", dest="parity", action="store_false",
                    help="skip the untimed oracle comparison (profiling runs)")
    ap.add_argument("--detail-out", default=None, help="also write the full record (JSON) to this file")
    ap.add_argument("--min-spin-s", type=float, default=MIN_SPIN_S,
                    help="sustained load before each short-kernel timing (counter runs set 0)")
    ap.add_argument("--min-batch-s", type=float, default=MIN_BATCH_S,
                    help="GPU time per timed batch of the other paths (counter runs set 0)")
    args = ap.parse_args()
    globals()["MIN_SPIN_S"] = args.min_spin_s
    globals()["MIN_BATCH_S"] = args.min_batch_s

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs each product on one MI355X, and sharding "
              "across GPUs is described, not implemented -- run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.batches < 10 or args.steps < 1:
        print("bench.py: --batches must be at least 10 and --steps at least 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no HIP device visible", file=sys.stderr)
        sys.exit(1)
    import gemm_decode_amd as gd
    torch.cuda.set_device(0)
    log(f"[bench] device: {torch.cuda.get_device_name(0)}")
    if args.workload in ("all", "q1"):
        out = bench_q1(args, gd, torch)
    else:
        out = {"metric": METRIC, "note": "Q1 workload skipped (--workload)"}
    floor_us, floor_st = measured_launch_floor(gd, torch, args.batches)
    out["launch_floor_us"] = _r(floor_us, 3)
    full = dict(out)
    full["launch_floor"] = {"us": _r(floor_us, 3), "timing": floor_st,
                            "kernel": "4 KiB fill, 64 launches per HIP graph"}
    if args.workload != "q1":
        extra = {}
        steps = [("cfg0_q1_256x1024", "q1small", bench_q1_small),
                 ("cfg2_sign_gemm", "sign", bench_sign),
                 ("cfg3_blockq8", "blockq8", bench_blockq8),
                 ("cfg4_ternary_step", "ternary", bench_ternary),
                 ("next1_q1_small_m", "q1mm", bench_q1_mm),
                 ("next2_act_quant", "quant", bench_quant),
                 ("next4_decode_attention", "attention", bench_attention)]
        for key, name, fn in steps:
            if args.workload in ("all", name):
                log(f"[bench] {key}")
                extra[key] = fn(args, gd, torch)
        full["workloads"] = extra
        short = {}
        for key, rec in extra.items():
            if key == "cfg3_blockq8":
                for m, r in rec.items():
                    short[f"cfg3_blockq8_{m}"] = compact(r)
            elif key in ("next1_q1_small_m", "next2_act_quant", "next4_decode_attention"):
                short[key] = {sub: with_floor(compact(r), floor_us) for sub, r in rec.items()}
            elif key == "cfg2_sign_gemm":
                short[key] = compact(rec)
                short["next3_sign_gemv"] = {sub: with_floor(compact(r), floor_us)
                                            for sub, r in rec["decode_gemv"].items()}
            else:
                short[key] = compact(rec)
        out["workloads"] = short
    if out.get("cpu_baseline"):
        cb = out["cpu_baseline"]
        out["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    log("[bench] detail " + json.dumps(full))
    if args.detail_out:
        with open(args.detail_out, "w") as f:
            json.dump(full, f, indent=1)
    print(json.dumps(out, separators=(",", ":")), flush=True)


if __name__ == "__main__":
    main()
