"""Benchmark of the key-only GLA forward (libgtrgla) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload img640]

A step is one pass of the hot path over one batch: the four scan-order calls
(left->right, right->left, top->bottom, bottom->top) that four consecutive GTR
blocks make, each on its own input tensors. Inputs are synthetic
(gla_synth, seeded) and already resident in HBM when timing starts. They are
rotated over at least 512 MiB of distinct buffers so that the 256 MB Infinity
Cache cannot serve them from a previous call (--rotate-mib: less, for counter
runs, where the profiler serialises every dispatch). Steps are captured into HIP
graphs and replayed (--no-graph: direct calls).

Prints ONE JSON line. `value` is tokens/s over the timed steps: calls x B x L
tokens divided by the time between two HIP events on the stream the graphs
(and so the kernels) run on. `roofline` covers the fused kernel (one launch
per call): algorithmic bytes per launch (inputs read once, outputs and final
state written once) divided by the mean launch duration, i.e. the same event
interval divided by the number of launches, against the 8 TB/s HBM peak.
`cpu_baseline` times the fp64 oracle on this host for a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 512 << 20     # 2x the Infinity Cache
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
DIRS = (0, 1, 2, 3)
DIR_NAMES = ("l2r", "r2l", "t2b", "b2t")


def lowrank_features(w) -> int:
    """Feature width C of the gate's input x: the model width H * d_v."""
    return w.H * w.d_v


def alg_bytes(w, gate: bool = False, init: bool = False, lowrank: bool = False) -> int:
    """Bytes the method must move per call: read q, k, v, log_gamma, write o and final_state
    (with the output gate also read the gate and the norm weight; with an initial state
    also read that; with the low-rank gate read x, W1, W2 and the bias instead of
    log_gamma)."""
    s = 2 if w.dtype == "fp16" else 4
    rows = w.B * w.L * w.H
    n = rows * (2 * w.d_k + 2 * w.d_v) * s + w.B * w.H * w.d_k * w.d_v * 4
    if lowrank:
        C = lowrank_features(w)
        K = w.H * w.d_k
        n += w.B * w.L * C * s + (C * 16 + 16 * K + K) * 4
    else:
        n += rows * w.d_k * s
    if gate:
        n += rows * w.d_v * s + w.d_v * 4
    if init:
        n += w.B * w.H * w.d_k * w.d_v * 4
    return n


def split_name(name: str):
    """'long2048+gate+init' -> ('long2048', {"gate": True, "init": True, "lowrank": False})."""
    parts = name.split("+")
    extra = set(parts[1:])
    bad = extra - {"gate", "init", "lowrank"}
    if bad:
        raise ValueError(f"unknown workload variant {sorted(bad)}")
    return parts[0], {k: k in extra for k in ("gate", "init", "lowrank")}


def mfma_flops(w) -> int:
    """Full-tile MFMA FLOPs per call: scores, A.V, Q.S and K^T.V per 64-token chunk."""
    C = w.chunk
    return w.B * w.H * w.L * (2 * C * (w.d_k + w.d_v) + 4 * w.d_k * w.d_v)


# sources of the fused token-mixer kernels, whose counters profiles/ holds
FUSED_SOURCES = ("gla_common.h", "gla_ws.h", "gla_fused.hip", "gla_span.hip")
# sources of the Spatial SwiGLU kernels and of the low-rank gate path (the
# projection kernel and the fused kernels' low-rank variant)
MIXER_SOURCES = ("gla_common.h", "gla_ws.h", "gla_fused.hip", "gla_gate.hip", "sswiglu.hip")


def kernel_hash(sources=FUSED_SOURCES) -> str:
    """Hash of the kernels' code (by default the fused token-mixer kernels):
    line comments, trailing blanks and empty lines are dropped first, so that a
    comment edit keeps the counter summaries taken on the same code valid."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunkwise_gated_recurrence_amd", "csrc")
    for f in sources:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            lines = (re.sub(r"//.*", "", l).rstrip() for l in fh)
            code = "\n".join(l for l in lines if l)
        h.update(f.encode() + code.encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic_<workload>.txt, lines "key: value"), or None when it was
    taken on a different kernel source."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{workload}.txt")
    try:
        with open(path) as fh:
            kv = dict(l.split(":", 1) for l in fh if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_hash") != kernel_hash():
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def rotation_groups(per_call: int, rotate: bool) -> int:
    """Input sets per scan order: enough that the sets of the four scan orders
    together span >= ROTATE_BYTES (2x the Infinity Cache), whatever the step count."""
    if not rotate:
        return 1
    return max(1, math.ceil(ROTATE_BYTES / (per_call * len(DIRS))))


def replay_plan(steps: int, n_groups: int):
    """(full replays of the n_groups-step graph, steps of the remainder graph):
    exactly `steps` steps in total."""
    return steps // n_groups, steps % n_groups


def run_workload(w, steps: int, warmup: int, rotate: bool, use_graph: bool = True,
                 gate: bool = False, init: bool = False, per_dir: bool = False,
                 lowrank: bool = False):
    """Time `steps` steps of the workload. A step is four calls (the four scan
    orders), each on its own input set; the sets rotate over >= 512 MiB. The
    steps are captured into HIP graphs (one graph per four sets) and replayed,
    so the timed region holds the kernels back to back, as the pages measure
    their operator (under CUDA Graph); --no-graph times direct calls. gate /
    init: calls through gtr_gla_fwd_ex with the RMSNorm + SiLU output gate and /
    or an initial state (each set has its own). lowrank: calls through
    gtr_gla_fwd_lowrank, the gate computed from x [B, L, H d_v] by the rank-16
    projection (each set has its own x; W1, W2 and the bias are shared)."""
    import numpy as np
    import torch

    import chunkwise_gated_recurrence_amd as gla
    import gla_synth

    arrays = gla_synth.generate(w)
    per_call = alg_bytes(w, gate, init, lowrank)
    nsets = len(DIRS) * rotation_groups(per_call, rotate)
    dev = torch.device("cuda:0")
    base = [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in arrays]
    rng = np.random.default_rng(w.seed + 1000)
    if gate:
        base.append(torch.from_numpy(rng.standard_normal((w.B, w.L, w.H, w.d_v)).astype(
            arrays[0].dtype)).to(dev))
    if init:
        base.append(torch.from_numpy(0.5 * rng.standard_normal(
            (w.B, w.H, w.d_k, w.d_v)).astype(np.float32)).to(dev))
    norm_w = torch.from_numpy(rng.uniform(0.5, 1.5, w.d_v).astype(np.float32)).to(dev)
    C = lowrank_features(w)
    if lowrank:
        x, w1, w2, gbias = [torch.from_numpy(np.ascontiguousarray(a)).to(dev)
                            for a in gla_synth.generate_lowrank(w, C, w.seed + 2000)]
        base[3] = x   # log_gamma is not read; x takes its place in each set
    sets = []
    for i in range(nsets):
        ins = base if i == 0 else [t.clone() for t in base]
        out = torch.empty((w.B, w.L, w.H, w.d_v), dtype=base[0].dtype, device=dev)
        fs = torch.empty((w.B, w.H, w.d_k, w.d_v), dtype=torch.float32, device=dev)
        sets.append((ins, out, fs))
    is_fp32 = w.dtype == "fp32"
    ws_fn = gla.gtr_gla_lowrank_workspace_bytes if lowrank else gla.gtr_gla_workspace_bytes
    ws_bytes = ws_fn(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, w.chunk, int(is_fp32))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    gla.gtr_gla_workspace_init(ws, ws.numel())
    fn = gla.gtr_gla_fwd_f32_ws if is_fp32 else gla.gtr_gla_fwd_ws

    def call(i, d):
        ins, out, fs = sets[i % nsets]
        q, k, v, lg = ins[:4]
        if lowrank:
            z = ins[4] if gate else None
            s0 = ins[-1] if init else None
            gla.gtr_gla_fwd_lowrank(q, k, v, lg, w1, w2, gbias, 1.0 / 16, C, s0, z,
                                    norm_w if gate else None, 1e-5, w.B, w.H, w.grid_h, w.grid_w,
                                    w.d_k, w.d_v, d, w.chunk, int(is_fp32), out, fs, ws,
                                    ws.numel())
        elif gate or init:
            z = ins[4] if gate else None
            s0 = ins[-1] if init else None
            gla.gtr_gla_fwd_ex(q, k, v, lg, s0, z, norm_w if gate else None, 1e-5, w.B, w.H,
                               w.grid_h, w.grid_w, w.d_k, w.d_v, d, w.chunk, int(is_fp32), out,
                               fs, ws, ws.numel())
        else:
            fn(q, k, v, lg, w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, d, w.chunk, out, fs, ws,
               ws.numel())

    n_groups = nsets // len(DIRS)
    for d in DIRS:   # eager calls first: plan caches, kernel attributes
        call(d, d)
    torch.cuda.synchronize()
    if use_graph:
        # One graph holds n_groups consecutive steps over every input set, as a model's
        # forward graph holds its blocks back to back; a second graph holds the first
        # `rem` groups, so that replays of the two run exactly the requested steps.
        def capture(groups):
            g_ = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_):
                for g in range(groups):
                    for d in DIRS:
                        call(len(DIRS) * g + d, d)
            return g_
        graph = capture(n_groups)
        rem_graphs = {}
        torch.cuda.synchronize()

        def run_steps(count):
            full, rem = replay_plan(count, n_groups)
            for _ in range(full):
                graph.replay()
            if rem:
                if rem not in rem_graphs:
                    rem_graphs[rem] = capture(rem)
                rem_graphs[rem].replay()
        # capture the remainder graphs outside the timed region
        for c in (warmup, steps):
            rem = replay_plan(c, n_groups)[1]
            if rem and rem not in rem_graphs:
                rem_graphs[rem] = capture(rem)
        torch.cuda.synchronize()
    else:
        def run_steps(count):
            for n in range(count):
                for d in DIRS:
                    call(len(DIRS) * (n % n_groups) + d, d)

    run_steps(warmup)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    run_steps(steps)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ncalls = steps * len(DIRS)
    dir_us = None
    dir_stats = None
    errors = None
    if per_dir and use_graph:
        # each scan order on its own: graphs of one direction's calls over the rotating sets
        dir_us = {}
        reps = max(5, steps // 8)
        for d in DIRS:
            graph_d = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph_d):
                for i in range(nsets):
                    call(i, d)
            graph_d.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                graph_d.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            dir_us[DIR_NAMES[d]] = 1e3 * e0.elapsed_time(e1) / (reps * nsets)
    if per_dir:
        # per-call distribution: direct calls, each bracketed by two events on the stream
        # the kernel runs on (inputs rotating as above); p10 / median / p90 per direction
        dir_stats = {}
        n_per = 100 if w.L * w.B <= 4096 else 50
        for d in DIRS:
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n_per)]
            for i, (a, b) in enumerate(evs):
                a.record(stream)
                call(len(DIRS) * (i % n_groups) + d, d)
                b.record(stream)
            torch.cuda.synchronize()
            us = np.sort([1e3 * a.elapsed_time(b) for a, b in evs])
            dir_stats[DIR_NAMES[d]] = {"p10_us": float(np.percentile(us, 10)),
                                       "median_us": float(np.median(us)),
                                       "p90_us": float(np.percentile(us, 90)), "calls": n_per}
        if not (gate or init or lowrank):
            # err_o / err_S of one call per direction on input set 0 against the fp64 oracle
            import oracle
            errors = {}
            ins, out, fs = sets[0]
            for d in DIRS:
                call(0, d)
                torch.cuda.synchronize()
                o_ref, s_ref = oracle.recurrent(*arrays, w.grid_h, w.grid_w, DIR_NAMES[d])
                errors[DIR_NAMES[d]] = {
                    "err_o": float(oracle.rel_err(out.float().cpu().numpy(), o_ref)),
                    "err_S": float(oracle.rel_err(fs.cpu().numpy(), s_ref))}
    kern, span, grid = gla.gtr_gla_plan(w.B, w.H, w.grid_h, w.grid_w, w.d_k, w.d_v, w.chunk,
                                        int(is_fp32), lowrank)
    return {
        "total_ms": total_ms,
        "ms_per_step": total_ms / steps,
        "tokens_per_s": ncalls * w.B * w.L / (total_ms * 1e-3),
        "call_us_mean": 1e3 * total_ms / ncalls,
        "alg_bytes_per_call": per_call,
        "rotating_sets": nsets,
        "graph": use_graph,
        "kernel": {1: "generic", 2: "fused", 3: "fused-rk", 4: "span"}.get(kern, str(kern)),
        "span": span,
        "grid": grid,
        "per_dir_us": dir_us,
        "per_dir_call_us": dir_stats,
        "errors": errors,
        "rotated_bytes": nsets * per_call,
    }


# Spatial SwiGLU workloads: (B, grid_h, grid_w, C, Hd) -- GTR-L's width (C = 384,
# Hd = 4 C) at 640x640 and 1024x1024 input
SSWIGLU_WORKLOADS = {
    "sswiglu640": (1, 40, 40, 384, 1536),
    "sswiglu1024": (1, 64, 64, 384, 1536),
}


def run_sswiglu(name: str, steps: int, warmup: int, rotate: bool = True):
    """Time the Spatial SwiGLU mixer like the token mixer: four calls per step (four
    blocks), each with its own input and weights, sets rotated over >= 512 MiB, all
    steps in one HIP graph. Returns a dict with us per call, TFLOP/s and MFMA fraction."""
    import numpy as np
    import torch

    import chunkwise_gated_recurrence_amd as gla
    import gla_synth

    B, gh, gw, C, Hd = SSWIGLU_WORKLOADS[name]
    L = gh * gw
    dev = torch.device("cuda:0")
    base = [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            for a in gla_synth.generate_sswiglu(B, gh, gw, C, Hd, seed=21)]
    per_call = (2 * B * L * C + 3 * Hd * C) * 2 + Hd * 40
    nsets = len(DIRS) * rotation_groups(per_call, rotate)
    sets = []
    for i in range(nsets):
        ins = base if i == 0 else [t.clone() for t in base]
        sets.append((ins, torch.empty((B, L, C), dtype=torch.float16, device=dev)))
    nws = gla.gtr_sswiglu_workspace_bytes(B, gh, gw, C, Hd)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)

    def call(i):
        ins, y = sets[i % nsets]
        gla.gtr_sswiglu_fwd(*ins, B, gh, gw, C, Hd, y, workspace=ws, workspace_bytes=nws)

    for i in range(len(DIRS)):
        call(i)
    torch.cuda.synchronize()
    n_groups = nsets // len(DIRS)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(nsets):
            call(i)
    torch.cuda.synchronize()
    reps_w = max(1, (warmup + n_groups - 1) // n_groups)
    reps = max(1, (steps + n_groups - 1) // n_groups)
    for _ in range(reps_w):
        graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / (reps * nsets)
    flops = 6 * B * L * C * Hd
    return {
        "workload": name, "B": B, "grid": f"{gh}x{gw}", "C": C, "Hd": Hd,
        "call_us_mean": us, "tokens_per_s": B * L / (us * 1e-6),
        "flop_per_call": flops, "TFLOPs": flops / (us * 1e-6) / 1e12,
        "mfma_frac": flops / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS,
        "alg_bytes_per_call": per_call,
        "kernels": "sswiglu_up_kernel + sswiglu_down_kernel",
    }


def run_ceiling(w, steps: int, warmup: int):
    """Practical ceiling: a plain streaming kernel (libgtrgla_ceiling.so) that reads four
    fp16 tensors and writes one, each of the workload's [B, L, H, 64] size, i.e. the
    operator's q, k, v, log_gamma and out bytes, timed like the operator (four calls per
    step, graph replay, sets rotated over >= 512 MiB). Each thread keeps 4 x unroll 16-byte
    loads in flight; the fastest of a few unroll / grid choices is reported. Returns
    (microseconds per call, the configuration)."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "chunkwise_gated_recurrence_amd", "libgtrgla_ceiling.so")
    lib = ctypes.CDLL(path)
    lib.gtr_stream_ceiling.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_int,
                                                                ctypes.c_int, ctypes.c_void_p]
    lib.gtr_stream_ceiling.restype = ctypes.c_int
    n = w.B * w.L * w.H * w.d_v
    per_call = 5 * n * 2
    n_groups = rotation_groups(per_call, True)
    nsets = len(DIRS) * n_groups
    dev = torch.device("cuda:0")
    sets = [[torch.full((n,), 0.01 * (i + 1), dtype=torch.float16, device=dev) for i in range(5)]
            for _ in range(nsets)]
    stream = torch.cuda.current_stream()
    best = None
    for unroll in (1, 2, 4):
        for blocks in (512, 1024, 2048, 4096):
            def call(i):
                a, b, c, d, o = sets[i % nsets]
                # the stream current at the call: under capture, the capturing one
                st = torch.cuda.current_stream().cuda_stream
                r = lib.gtr_stream_ceiling(a.data_ptr(), b.data_ptr(), c.data_ptr(), d.data_ptr(),
                                           o.data_ptr(), n, blocks, unroll, st)
                if r != 0:
                    raise RuntimeError(f"gtr_stream_ceiling failed ({r})")

            for i in range(len(DIRS)):
                call(i)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(nsets):
                    call(i)
            reps = max(1, steps // (4 * n_groups))
            for _ in range(max(1, warmup // n_groups)):
                graph.replay()
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            for _ in range(reps):
                graph.replay()
            t1.record(stream)
            torch.cuda.synchronize()
            us = 1e3 * t0.elapsed_time(t1) / (reps * nsets)
            if per_call / (us * 1e-6) / 1e9 > HBM_PEAK_GBS:
                raise RuntimeError("streaming ceiling above the HBM peak: the timed graph "
                                   "did not hold its kernels")
            if best is None or us < best[0]:
                best = (us, {"unroll": unroll, "blocks": blocks})
            del graph
    return best


def host_cpu() -> dict:
    """The host the oracle runs on: CPU model, logical CPUs, CPUs this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": affinity}


def _time_oracle(w, arrays, threads: int, budget_s: float):
    import oracle
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.recurrent(*arrays, w.grid_h, w.grid_w, DIRS[calls % 4], threads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / calls * (calls + 1) > 2.5 * budget_s:
            break
    return calls, el


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle as it stands, on this host, for as many single-direction
    calls of the workload as fit in about `budget_s` seconds (at least one), with
    one thread per (batch, head) sequence up to the CPUs available; then again on
    one thread for about a third of that budget."""
    import gla_synth
    import oracle

    arrays = gla_synth.generate(w)
    host = host_cpu()
    threads = min(oracle.default_threads(), w.B * w.H)
    calls, el = _time_oracle(w, arrays, threads, budget_s)
    calls1, el1 = _time_oracle(w, arrays, 1, budget_s / 3)
    return {
        "value": calls * w.B * w.L / el,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{calls} single-direction calls of {w.name} "
                  f"(B={w.B}, {w.grid_h}x{w.grid_w}, H={w.H}, d_k={w.d_k}, d_v={w.d_v}) "
                  f"in {el:.1f} s, fp64 token-by-token recurrence, one thread per (batch, head) "
                  f"sequence ({threads} threads)",
        "threads": threads,
        "host": host,
        "single_thread": {"value": calls1 * w.B * w.L / el1, "unit": "tokens/s", "cores": 1,
                          "sample": f"{calls1} calls in {el1:.1f} s on one thread"},
    }


def main() -> int:
    global ROTATE_BYTES
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="img640")
    ap.add_argument("--secondary",
                    default="img1024,long2048,batched640,img640_dk32,img640+gate,long2048+gate,"
                            "img640_dk32+lowrank,long2048+lowrank",
                    help="comma-separated extra workloads reported beside the main one "
                         "(NAME+gate: with the RMSNorm + SiLU output gate; NAME+init: from an "
                         "initial state)")
    ap.add_argument("--sswiglu", default="sswiglu640,sswiglu1024",
                    help="Spatial SwiGLU workloads to time as well (comma list, may be empty)")
    ap.add_argument("--warm", action="store_true", help="reuse one input set (cache-warm)")
    ap.add_argument("--rotate-mib", type=int, default=ROTATE_BYTES >> 20,
                    help="bytes (MiB) the rotating input sets span; counter runs use less, since a "
                         "profiler serialises every dispatch")
    ap.add_argument("--verbose", action="store_true", help="a line on stderr as each workload ends")
    ap.add_argument("--no-graph", action="store_true", help="time direct calls, not graph replays")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of COPY_BYTES (for counter calibration)")
    args = ap.parse_args()

    ROTATE_BYTES = args.rotate_mib << 20
    say = (lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)) if args.verbose else (
        lambda m: None)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): this build runs on "
              "one GPU; the B*H sequences shard across GPUs with no communication, so N GPUs run "
              "N independent copies of this measurement.", file=sys.stderr)
        return 2

    import torch

    import chunkwise_gated_recurrence_amd as gla
    import gla_synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        return copy_calibration()
    if not os.path.exists(gla.LIB_PATH):
        from chunkwise_gated_recurrence_amd import build as _b
        _b.build()
    gla.load_library()

    w = gla_synth.WORKLOADS[args.workload]
    graph = not args.no_graph
    r = run_workload(w, args.steps, args.warmup, rotate=not args.warm, use_graph=graph,
                     per_dir=True)
    say(f"{w.name} done")
    achieved = r["alg_bytes_per_call"] / (r["call_us_mean"] * 1e-6) / 1e9
    traffic = measured_traffic(w.name)
    secondary = []
    for name in [s for s in args.secondary.split(",") if s and s != w.name]:
        base_name, variant = split_name(name)
        ws = gla_synth.WORKLOADS[base_name]
        rs = run_workload(ws, max(20, args.steps // 4), args.warmup, rotate=not args.warm,
                          use_graph=graph, per_dir=not any(variant.values()), **variant)
        say(f"{name} done")
        gbs = rs["alg_bytes_per_call"] / (rs["call_us_mean"] * 1e-6) / 1e9
        ceil_us = run_ceiling(ws, max(20, args.steps // 4), args.warmup)[0] if not any(
            variant.values()) else None
        secondary.append({
            "workload": name, "tokens_per_s": rs["tokens_per_s"], "ms_per_step": rs["ms_per_step"],
            "ceiling_us": ceil_us,
            "call_us_mean": rs["call_us_mean"], "achieved_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "mfma_frac": mfma_flops(ws) / (rs["call_us_mean"] * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "kernel": rs["kernel"], "span": rs["span"], "grid": rs["grid"],
            "traffic": measured_traffic(name),
            "call_us_per_dir": rs["per_dir_call_us"], "errors_vs_oracle": rs["errors"],
        })

    mixer = []
    for name in [n for n in args.sswiglu.split(",") if n]:
        mixer.append(run_sswiglu(name, max(20, args.steps // 4), args.warmup, rotate=not args.warm))
        say(f"{name} done")

    ceil_us, ceil_cfg = run_ceiling(w, max(20, args.steps // 4), args.warmup)
    ceiling = {
        "kind": "plain streaming kernel: read 4 fp16 tensors, write 1 (the operator's q, k, v, "
                "log_gamma, out bytes), same timing; fastest of unroll x grid choices",
        "us_per_call": ceil_us,
        "config": ceil_cfg,
        "GBs": 5 * w.B * w.L * w.H * w.d_v * 2 / (ceil_us * 1e-6) / 1e9,
        "operator_over_ceiling": r["call_us_mean"] / ceil_us,
    }
    line = {
        "metric": "key-only GLA fwd tokens/s at 1.6K & 16.4K tokens; % of HBM/MFMA roofline",
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if w.dtype == "fp16" else "f32",
        "data": (f"synthetic (seeded gla_synth inputs, rotated over {r['rotated_bytes'] / 2**20:.0f} "
                 f"MiB of HBM buffers, >= {ROTATE_BYTES >> 20} MiB)"
                 if not args.warm else "synthetic (seeded gla_synth inputs, one warm set)"),
        "config": {
            "workload": w.name, "B": w.B, "grid": f"{w.grid_h}x{w.grid_w}", "L": w.L, "H": w.H,
            "d_k": w.d_k, "d_v": w.d_v, "chunk": w.chunk, "calls_per_step": len(DIRS),
            "input_dtype": w.dtype, "kernel": r["kernel"], "span": r["span"], "grid_wg": r["grid"],
            "timing": "HIP graph replay" if graph else "direct calls",
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": {"fused": "gla_fused_kernel", "fused-rk": "gla_fused_rk_kernel",
                       "span": "gla_span_kernel"}.get(r["kernel"], "generic (3 kernels)"),
            "alg_bytes_per_launch": r["alg_bytes_per_call"],
            "launch_us_mean": r["call_us_mean"],
            "launch_us_per_dir": r["per_dir_us"],
            "call_us_per_dir": r["per_dir_call_us"],
            "mfma_frac": mfma_flops(w) / (r["call_us_mean"] * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS,
        },
        "errors_vs_oracle": r["errors"],
        "ceiling": ceiling,
        "secondary": secondary,
        "spatial_swiglu": mixer,
        "kernel_hash": kernel_hash(),
        "mixer_kernel_hash": kernel_hash(MIXER_SOURCES),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


COPY_BYTES = 1 << 30


def copy_calibration() -> int:
    """A plain device-to-device copy of COPY_BYTES (read once, written once),
    run a few times: the FETCH_SIZE / WRITE_SIZE counters of this run, divided
    by COPY_BYTES, give the factor that turns counter readings into bytes."""
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "repeats": 3}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
