#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X.

Default workload: the fused dual-epsilon sandwich tail on 4096 rows x 6656
f32 (reads a and r, writes h and y: four row streams), with the gains and
epsilons of the model the Muser book describes (eps_post = 1e-8,
eps_pre = 1e-5). A step is one sandwich_tail call over the whole batch.

Prints ONE JSON line on stdout: achieved HBM GB/s from algorithmic bytes
(row streams plus each gain once per launch) over wall time, rows/s, the
dominant kernel's roofline (per-launch time from HIP events on the launch
stream; HBM traffic from the committed byte-counter summary), the attainable
floor on the same GPU (plain read, write and copy kernels of
bench_stream.hip, and the step's own row access pattern with no
arithmetic), and the f64 oracle's throughput on the host cores.

Inputs are resident in HBM before timing starts. Rotating sets of
input/output buffers (at least three, and together at least 1 GiB of step
traffic, four times the 256 MB Infinity Cache; at most 64) keep one launch's
inputs from being served by the cache the previous launches warmed.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("achieved HBM GB/s (% of peak) + rows/s, fused sandwich tail "
          "4096×6656 f32")
PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, published


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# row streams (reads + writes) and gains of each operation
STREAMS = {"plain": (2, 1), "tail": (4, 2), "norm_add": (3, 1),
           "add_norm": (4, 1), "multi": (2, 1)}
# row streams read, of those
READS = {"plain": 1, "tail": 2, "norm_add": 2, "add_norm": 2, "multi": 1}


def algorithmic_bytes(cfg) -> int:
    es = 4 if cfg.dtype == "f32" else 2
    if cfg.kind == "q8":
        # read x and gamma; write one 36-byte record per 32 elements
        return cfg.rows * cfg.n * es + cfg.n * es + cfg.rows * cfg.n // 32 * 36
    streams, gains = STREAMS[cfg.kind]
    if cfg.kind == "multi":
        gains = len(cfg.segments)
    return streams * cfg.rows * cfg.n * es + gains * cfg.n * es


def read_write_bytes(cfg):
    """(bytes read, bytes written) of one step; gains count as reads."""
    es = 4 if cfg.dtype == "f32" else 2
    total = algorithmic_bytes(cfg)
    if cfg.kind == "q8":
        written = cfg.rows * cfg.n // 32 * 36
    else:
        written = (STREAMS[cfg.kind][0] - READS[cfg.kind]) * cfg.rows * \
            cfg.n * es
    return total - written, written


# the streaming kernels of bench_stream.hip, by variant index
PROBE_READ, PROBE_WRITE, PROBE_WRITE_NT, PROBE_COPY = 0, 1, 2, 3
PROBE_MIB = 256          # per stream and buffer set
PROBE_GRIDS = (2048, 8192, 32768, 0)   # 0: one workgroup per trip's range


def stream_ceiling(cfg, torch, stream, achieved_gbs: float, sets=None,
                   shape: str = ""):
    """What plain streaming kernels (no arithmetic) sustain on this GPU, and
    the floor that sets for this workload's step.

    Reads alone and writes alone each stream faster than any mix of the two:
    an HBM channel turns its bus around between reads and writes. So the
    floor is a plain copy of the step's W written bytes (W bytes read, W
    written, in one launch) plus the step's remaining R - W read bytes at
    the read-only rate (R >= W for every workload here). The copy runs over
    rotating buffer sets of at least 1 GiB together, like the step; the
    read-only and write-only rates use 256 MiB buffers. Each figure is the
    best over a few grid sizes of a flat grid-stride loop, timed by one
    event pair around 30 back-to-back launches."""
    import ctypes
    # loaded after torch has initialised its own HIP runtime (the library
    # names the same runtime soname; a process keeps the first copy loaded)
    path = os.path.join(ROOT, "bench_stream.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.stream_probe.restype = ctypes.c_int
    lib.stream_probe.argtypes = [ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int64, ctypes.c_int,
                                 ctypes.c_void_p]
    lib.stream_probe_rows.restype = ctypes.c_int
    lib.stream_probe_rows.argtypes = [ctypes.c_void_p] * 4 + [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p]
    sink = torch.zeros(16, dtype=torch.int32, device="cuda:0")
    handle = stream.cuda_stream

    def buffers(nbytes):
        nsets = min(64, max(3, -(-(1 << 30) // (2 * nbytes))))
        return [(torch.ones(nbytes // 4, device="cuda:0"),
                 torch.empty(nbytes // 4, device="cuda:0"))
                for _ in range(nsets)]

    def best_us(variant, bufs, nbytes):
        def launch(i):
            src, dst = bufs[i % len(bufs)]
            rc = lib.stream_probe(variant, src.data_ptr(), dst.data_ptr(),
                                  sink.data_ptr(), nbytes, grid, handle)
            if rc != 0:
                raise RuntimeError(f"stream_probe({variant}, {grid}) -> {rc}")
        best = float("inf")
        for grid in PROBE_GRIDS:
            with torch.cuda.stream(stream):
                for i in range(5):
                    launch(i)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(30):
                    launch(i)
                e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / 30)
        return best

    big = PROBE_MIB << 20
    bufs = buffers(big)
    rd = big / best_us(PROBE_READ, bufs, big) * 1e-3
    wr = big / min(best_us(PROBE_WRITE, bufs, big),
                   best_us(PROBE_WRITE_NT, bufs, big)) * 1e-3
    del bufs
    r_bytes, w_bytes = read_write_bytes(cfg)
    w16 = w_bytes // 16 * 16
    copy_us = best_us(PROBE_COPY, buffers(w16), w16)
    floor_us = copy_us + (r_bytes - w_bytes) / rd * 1e-3
    floor_gbs = (r_bytes + w_bytes) / (floor_us * 1e-6) / 1e9
    pattern = row_pattern(cfg, torch, stream, lib, sets, shape)
    if pattern is not None:
        pattern["achieved_frac_of_pattern"] = round(
            achieved_gbs / ((r_bytes + w_bytes) / (pattern["us"] * 1e-6) /
                            1e9), 4)
    return {"read_gbs": round(rd, 1), "write_gbs": round(wr, 1),
            "copy_gbs": round(2 * w16 / copy_us * 1e-3, 1),
            "copy_us": round(copy_us, 3),
            "step_read_bytes": r_bytes, "step_write_bytes": w_bytes,
            "floor_us": round(floor_us, 3), "floor_gbs": round(floor_gbs, 1),
            "floor_frac_of_peak": round(floor_gbs / PEAK_HBM_GBS, 4),
            "achieved_frac_of_floor": round(achieved_gbs / floor_gbs, 4),
            "model": "copy of W bytes in one launch + (R - W) / read_gbs",
            "row_pattern": pattern,
            "probe": (f"plain read / write / copy kernels "
                      f"(bench_stream.hip); copy of the step's written "
                      f"bytes over rotating sets of >= 1 GiB; read and "
                      f"write over {PROBE_MIB} MiB buffers; best of grids "
                      f"{list(PROBE_GRIDS)} (0 = one trip)")}


ROW_PATTERN_SHAPES = {(1024, 1), (1024, 2), (512, 2), (512, 4), (256, 2),
                      (256, 4), (256, 8)}
# input row streams of each operation with a row pattern (outputs: out[...])
ROW_PATTERN_INPUTS = {"plain": ("x",), "norm_add": ("a", "b"),
                      "tail": ("a", "r"), "add_norm": ("a", "b")}


def row_pattern(cfg, torch, stream, lib, sets, shape: str):
    """The step's own access pattern with no arithmetic, on the step's own
    buffers: for an operation run by a one-row-per-workgroup tile, a kernel
    that loads its input rows and stores its output rows, one row per
    workgroup of the same lanes and vectors per lane. None for other
    workloads and shapes."""
    parts = shape.split(":")
    if (cfg.kind not in ROW_PATTERN_INPUTS or not sets or len(parts) != 4
            or parts[0] not in ("rowtile", "persist")):
        return None
    lanes, vpt, width = int(parts[1]), int(parts[2]), int(parts[3])
    if (lanes, vpt) not in ROW_PATTERN_SHAPES or cfg.n % width:
        return None
    keys = ROW_PATTERN_INPUTS[cfg.kind]
    handle = stream.cuda_stream

    def launch(i):
        st = sets[i % len(sets)]
        ins = [st[k].data_ptr() for k in keys] + [None]
        outs = [o.data_ptr() for o in st["out"]] + [None]
        rc = lib.stream_probe_rows(ins[0], ins[1], outs[0], outs[1],
                                   cfg.rows, cfg.n // width, lanes, vpt,
                                   handle)
        if rc != 0:
            raise RuntimeError(f"stream_probe_rows -> {rc}")
    with torch.cuda.stream(stream):
        for i in range(5):
            launch(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(200):
            launch(i)
        e1.record(stream)
    torch.cuda.synchronize()
    return {"us": round(e0.elapsed_time(e1) * 1e3 / 200, 3),
            "lanes": lanes, "vectors_per_lane": vpt,
            "what": f"{len(keys)} input row(s) loaded, {len(sets[0]['out'])} "
                    "output row(s) stored, one row per workgroup, no "
                    "arithmetic (bench_stream.hip)"}


def kernel_sources(cfg) -> list:
    """The source files the workload's kernels are built from."""
    csrc = os.path.join(ROOT, "sandwich_norm_residual_amd", "csrc")
    main = (("snr_q8.hip",) if cfg.kind == "q8"
            else ("snr_kernels.hip", "snr_persist.hip", "snr_split.hip"))
    return [os.path.join(csrc, f)
            for f in ("snr_internal.h", "snr_device.h") + main]


def kernel_source_digest(cfg) -> str:
    """sha256 over the workload's kernel sources; counters recorded for other
    sources are not reported."""
    import hashlib
    h = hashlib.sha256()
    for path in kernel_sources(cfg):
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(cfg, shape):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for
    a plain copy of known size), or None when there is no summary for this
    workload and dispatch shape or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"{cfg.name}.counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if (kv.get("kernel_source_sha256") != kernel_source_digest(cfg) or
            kv.get("dispatch_shape") != shape):
        return None
    return float(kv["traffic_bytes_per_launch"])


def to_device(arr, dtype, torch):
    """A storage array (float32, or uint16 bits of bf16/f16) on cuda:0."""
    import numpy as np
    dev = torch.device("cuda:0")
    if dtype == "f32":
        return torch.from_numpy(arr).to(dev)
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev)
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def make_device_sets(cfg, inp, sets, torch):
    """`sets` copies of the row inputs and their own outputs; gains shared."""
    st = cfg.dtype
    if cfg.kind == "multi":
        xs = [to_device(x, st, torch) for x in inp["xs"]]
        gs = [to_device(g, st, torch) for g in inp["gammas"]]
        return [{"xs": [x.clone() for x in xs], "gs": gs,
                 "out": [torch.empty_like(x) for x in xs]}
                for _ in range(sets)]
    if cfg.kind == "q8":
        x = to_device(inp["x"], st, torch)
        g = to_device(inp["gamma"], st, torch)
        blocks = (cfg.rows, cfg.n // 32, 36)
        return [{"x": x.clone(), "gamma": g,
                 "out": [torch.empty(blocks, dtype=torch.uint8,
                                     device=x.device)]}
                for _ in range(sets)]
    rows_keys = {"plain": ("x",), "tail": ("a", "r"),
                 "norm_add": ("a", "b"), "add_norm": ("a", "b")}[cfg.kind]
    gain_keys = ("gamma_post", "gamma_pre") if cfg.kind == "tail" else \
        ("gamma",)
    nout = {"plain": 1, "tail": 2, "norm_add": 1, "add_norm": 2}[cfg.kind]
    base = {k: to_device(inp[k], st, torch) for k in rows_keys + gain_keys}
    out = []
    for _ in range(sets):
        d = {k: base[k].clone() for k in rows_keys}
        d.update({k: base[k] for k in gain_keys})
        d["out"] = [torch.empty_like(base[rows_keys[0]]) for _ in range(nout)]
        out.append(d)
    return out


def make_step(cfg, inp, sets, snr, separate=False):
    kind = cfg.kind

    def step(i):
        s = sets[i % len(sets)]
        if kind == "tail":
            snr.sandwich_tail(s["a"], s["r"], s["gamma_post"],
                              inp["eps_post"], s["gamma_pre"], inp["eps_pre"],
                              h_out=s["out"][0], y_out=s["out"][1])
        elif kind == "plain":
            snr.rmsnorm_fwd(s["x"], s["gamma"], inp["eps"], out=s["out"][0])
        elif kind == "q8":
            snr.rmsnorm_q8_1(s["x"], s["gamma"], inp["eps"], out=s["out"][0])
        elif kind == "norm_add":
            snr.norm_then_add(s["a"], s["b"], s["gamma"], inp["eps"],
                              out=s["out"][0])
        elif kind == "multi" and separate:
            for x, g, y in zip(s["xs"], s["gs"], s["out"]):
                snr.rmsnorm_fwd(x, g, inp["eps"], out=y)
        elif kind == "multi":
            snr.rmsnorm_fwd_multi(
                [(x, g, inp["eps"]) for x, g in zip(s["xs"], s["gs"])],
                s["out"])
        else:
            snr.add_then_norm(s["a"], s["b"], s["gamma"], inp["eps"],
                              sum_out=s["out"][0], y_out=s["out"][1])
    return step


def capture_steps(step, count: int, torch):
    """A HIP graph (torch.cuda.CUDAGraph) of `count` consecutive steps,
    step(0) ... step(count - 1), captured after one eager pass of the same
    steps on the capture's side stream."""
    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(count):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(count):
            step(i)
    torch.cuda.synchronize()
    return graph


def host_cpus() -> dict:
    """The host's CPUs as this process sees them: the online count, the
    affinity mask, the CPU model, and the oracle's thread count (one thread
    per CPU in the affinity mask, unless OMP_NUM_THREADS states a smaller
    CPU share for this process)."""
    aff = sorted(os.sched_getaffinity(0))
    ranges, start = [], None
    for i, c in enumerate(aff):
        if start is None:
            start = c
        if i + 1 == len(aff) or aff[i + 1] != c + 1:
            ranges.append(f"{start}-{c}" if c > start else f"{c}")
            start = None
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cap = None
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "")) or None
    except ValueError:
        cap = None
    threads = len(aff) if not cap else max(1, min(len(aff), cap))
    return {"nproc": os.cpu_count(), "affinity": len(aff),
            "mask": ",".join(ranges), "model": model, "cap": cap,
            "threads": threads}


def cpu_baseline(cfg, inp, seconds: float) -> dict:
    """The f64 oracle as it stands, rows split across host threads (ctypes
    releases the GIL), repeated over the full workload for about `seconds`."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    O = oracle.load()
    hw = host_cpus()
    cores = hw["threads"]
    rows = cfg.rows
    bounds = [(rows * i // cores, rows * (i + 1) // cores)
              for i in range(cores)]
    bounds = [b for b in bounds if b[1] > b[0]]

    from sandwich_norm_residual_amd.inputs import from_storage
    st = cfg.dtype
    f = {k: from_storage(v, st) for k, v in inp.items()
         if isinstance(v, np.ndarray)}

    if cfg.kind == "multi":
        f = {"xs": [from_storage(x, st) for x in inp["xs"]],
             "gammas": [from_storage(g, st) for g in inp["gammas"]]}

    def one(b):
        lo, hi = b
        if cfg.kind == "multi":
            # rows of the concatenated segments [lo, hi)
            start = 0
            for x, g in zip(f["xs"], f["gammas"]):
                a, z = max(lo - start, 0), min(hi - start, x.shape[0])
                if a < z:
                    O.rmsnorm(x[a:z], g, inp["eps"])
                start += x.shape[0]
        elif cfg.kind == "tail":
            O.sandwich_tail(f["a"][lo:hi], f["r"][lo:hi], f["gamma_post"],
                            inp["eps_post"], f["gamma_pre"], inp["eps_pre"])
        elif cfg.kind == "plain":
            O.rmsnorm(f["x"][lo:hi], f["gamma"], inp["eps"])
        elif cfg.kind == "q8":
            O.rmsnorm_q8_1(f["x"][lo:hi], f["gamma"], inp["eps"])
        elif cfg.kind == "norm_add":
            O.norm_then_add(f["a"][lo:hi], f["b"][lo:hi], f["gamma"],
                            inp["eps"])
        else:
            O.add_then_norm(f["a"][lo:hi], f["b"][lo:hi], f["gamma"],
                            inp["eps"])

    # one core first (about a third of the budget, rows in slices), then
    # every core
    t1 = time.perf_counter()
    rows1 = 0
    while time.perf_counter() - t1 < seconds / 3:
        for b in bounds:
            one(b)
            rows1 += b[1] - b[0]
            if time.perf_counter() - t1 >= seconds / 3:
                break
    dt1 = time.perf_counter() - t1
    gbs1 = algorithmic_bytes(cfg) * rows1 / rows / dt1 / 1e9

    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(len(bounds)) as ex:
        while True:
            list(ex.map(one, bounds))
            passes += 1
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    gbs = algorithmic_bytes(cfg) * passes / dt / 1e9
    model = hw["model"]
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": len(bounds),
            "kind": "oracle",
            "single_core_value": round(gbs1, 3),
            "nproc": hw["nproc"], "affinity_cpus": hw["affinity"],
            "affinity_mask": hw["mask"], "cpu_model": model,
            "thread_cap": hw["cap"],
            "sample": (f"{passes} full passes over {cfg.name} "
                       f"({rows} rows) in {dt:.1f} s, scalar f64 C oracle, "
                       f"rows split over {len(bounds)} threads; "
                       f"rows/s {rows * passes / dt:.4g}; one core: "
                       f"{rows1} rows in {dt1:.1f} s, {gbs1:.3g} GB/s, "
                       f"rows/s {rows1 / dt1:.4g}; cpu: {model}; nproc "
                       f"{hw['nproc']}, {hw['affinity']} CPUs in the "
                       f"affinity mask ({hw['mask']})"
                       + (f", OMP_NUM_THREADS={hw['cap']}" if hw["cap"]
                          else ""))}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000,
                    help="timed steps (the headline's 2000 take about 0.15 s "
                         "of GPU time per pass)")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default=None,
                    help="workload name (default: the 4096x6656 f32 tail)")
    ap.add_argument("--sets", type=int, default=None,
                    help="rotating buffer sets (default: at least 3 and 1 GiB "
                         "of step traffic together, at most 64)")
    ap.add_argument("--prewarm-ms", type=float, default=500.0,
                    help="untimed steps back to back for this long before "
                         "the timed region (reported as prewarm_ms)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the oracle CPU baseline")
    ap.add_argument("--separate-launches", action="store_true",
                    help="several-norm workloads: one rmsnorm_fwd launch per "
                         "problem instead of one rmsnorm_fwd_multi launch")
    ap.add_argument("--graph", action="store_true",
                    help="replay the steps from HIP graphs (each graph holds "
                         "one step per buffer set, repeated to 64 or more "
                         "steps) instead of launching them from Python: the "
                         "decode-size steps are then bound by the GPU, not "
                         "by the host's call rate")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-rate kernels that state the "
                         "attainable HBM floor of the workload")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run 10 plain device copies of MIB MiB "
                         "(byte-counter calibration under rocprofv3)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(rows are independent, so a batch would shard across GPUs by "
              "rows with no communication). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    import sandwich_norm_residual_amd as snr
    from sandwich_norm_residual_amd import _lib
    from sandwich_norm_residual_amd import inputs as gen
    if not os.path.exists(_lib.LIBRARY):
        import __graft_entry__
        __graft_entry__.build()

    cfg = gen.CONFIGS[args.config or gen.HEADLINE]
    log(f"workload {cfg.name}: rows={cfg.rows} n={cfg.n} {cfg.dtype} "
        f"seed={cfg.seed}")
    inp = gen.make(cfg)
    nbytes = algorithmic_bytes(cfg)
    nsets = args.sets or min(64, max(3, -(-(1 << 30) // nbytes)))
    sets = make_device_sets(cfg, inp, nsets, torch)
    stream = torch.cuda.Stream()   # default priority

    step = make_step(cfg, inp, sets, snr, args.separate_launches)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        shape = snr.last_shape()
        torch.cuda.synchronize()

        # `unit` steps per call of run(): one step launched from Python, or
        # one replay of a graph holding `unit` steps
        unit = 1
        run = step
        if args.graph:
            unit = len(sets) * max(1, -(-64 // len(sets)))
            graph = capture_steps(step, unit, torch)
            run = lambda i: graph.replay()  # noqa: E731
        calls = max(1, args.steps // unit)
        steps = calls * unit

        # Pre-warm: steps back to back for a fixed stretch of wall time
        # before the timed region (untimed, beyond the W warm-up steps), so
        # that a short timed region meets the GPU's clocks at steady state
        # rather than ramping up from idle.
        # The host waits on the batch before last, so the GPU always has a
        # batch queued and never idles.
        prewarm_calls = 0
        prev = None
        tp = time.perf_counter()
        while time.perf_counter() - tp < args.prewarm_ms * 1e-3:
            for _ in range(16):
                run(prewarm_calls)
                prewarm_calls += 1
            ev_batch = torch.cuda.Event()
            ev_batch.record(stream)
            if prev is not None:
                prev.synchronize()
            prev = ev_batch
        torch.cuda.synchronize()
        prewarm_s = time.perf_counter() - tp

        # whole-job throughput: K back-to-back steps, synchronised both
        # sides. Inside the same region, one event pair on the launch stream
        # brackets calls 1 .. K-1 (the first call's host launch latency, when
        # the GPU has nothing queued, stays outside the pair): their average
        # is the per-launch duration.
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        for i in range(calls):
            run(i)
            if i == 0:
                e0.record(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if calls > 1:
            mean_us = e0.elapsed_time(e1) * 1e3 / ((calls - 1) * unit)
        else:
            mean_us = wall * 1e6 / steps

        # spread of single launches (each bracketed by its own events, which
        # adds the events' own overhead to every sample; with graphs, the
        # mean step of each replay)
        ev = [(torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True))
              for _ in range(max(2, min(calls, 200)))]
        for i in range(len(ev)):
            ev[i][0].record(stream)
            run(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        durs_us = [a.elapsed_time(b) * 1e3 / unit for a, b in ev]

        if args.copy_probe:
            n = args.copy_probe * (1 << 20) // 4
            src = torch.ones(n, device="cuda:0")
            dst = torch.empty_like(src)
            for _ in range(10):
                dst.copy_(src)
            torch.cuda.synchronize()
            log(f"copy probe: 10 x {args.copy_probe} MiB device copies")

    ms_per_step = wall / steps * 1e3
    value = nbytes * steps / wall / 1e9
    med_us = statistics.median(durs_us)
    q = statistics.quantiles(durs_us, n=10)
    achieved = nbytes / (mean_us * 1e-6) / 1e9
    log(f"shape {shape}; wall {ms_per_step * 1e3:.2f} us/step; events over "
        f"the timed region {mean_us:.2f} us/launch; single-launch events "
        f"median {med_us:.2f} p10 {q[0]:.2f} p90 {q[-1]:.2f}")
    traffic = measured_traffic(cfg, shape)

    # the floor needs an HBM-bound step: at least 64 MiB of traffic
    ceiling = None
    if not args.no_ceiling and nbytes >= (64 << 20):
        try:
            ceiling = stream_ceiling(cfg, torch, stream, achieved, sets, shape)
        except (OSError, RuntimeError) as e:
            # the step is measured already; the floor is context, so its
            # failure is reported and leaves "attainable" null
            log(f"attainable floor not measured: {e}")
    if ceiling:
        log(f"attainable: read {ceiling['read_gbs']} GB/s, write "
            f"{ceiling['write_gbs']} GB/s, copy of the step's written bytes "
            f"{ceiling['copy_us']} us = {ceiling['copy_gbs']} GB/s; "
            f"floor {ceiling['floor_us']} us/step = "
            f"{100 * ceiling['floor_frac_of_peak']:.1f}% of peak; this step "
            f"reaches {100 * ceiling['achieved_frac_of_floor']:.1f}% of it")
        if ceiling["row_pattern"]:
            pat = ceiling["row_pattern"]
            log(f"row pattern without arithmetic ({pat['lanes']} x "
                f"{pat['vectors_per_lane']}): {pat['us']} us; this step "
                f"reaches {100 * pat['achieved_frac_of_pattern']:.1f}% of it")

    cpu = None
    if not args.no_cpu:
        log(f"cpu baseline: oracle for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(cfg, inp, args.cpu_seconds)

    line = {
        "metric": METRIC if cfg.name == gen.HEADLINE else
        f"achieved HBM GB/s + rows/s, {cfg.name}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": (f"synthetic: seeded PCG64 (seed {cfg.seed}) Gaussian rows "
                 "with log-uniform per-row scales, gains 1+0.1*N(0,1)"),
        "config": {"workload": cfg.name, "rows": cfg.rows, "n": cfg.n,
                   "kind": cfg.kind, "eps": list(cfg.eps),
                   "launches_per_step": (len(cfg.segments)
                                         if args.separate_launches else 1),
                   "steps_per_graph": unit if args.graph else None,
                   "dispatch_shape": shape,
                   "rotating_buffer_sets": len(sets),
                   "algorithmic_bytes_per_step": nbytes},
        "rows_per_s": round(cfg.rows * steps / wall, 1),
        "pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        "prewarm_ms": round(prewarm_s * 1e3, 1),
        "prewarm_steps": prewarm_calls * unit,
        "kernel_us": {"mean_over_timed_region": round(mean_us, 3),
                      "single_launch_median": round(med_us, 3),
                      "single_launch_p10": round(q[0], 3),
                      "single_launch_p90": round(q[-1], 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "attainable": ceiling,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
