"""Benchmark of the block-sparse attention hot path on one MI355X.

Default (no ``--config``): every workload at full size, in one JSON line.

  1 tiny sparse decode             (B=1, H=4, D=64, Sk=1024; sets A, B and their combine)
  2 speculative + sparse decode    (B=32, Hq=32, Hkv=8, D=128, Sk=32768)      <- headline
  3 block-sparse causal prefill    (S=32768, Hq=32, Hkv=8, 128x128 tiles, 34-entry lists)
  4 BSFA gated causal prefill      (S=65536, Hq=32, Hkv=8, ~50% of off-diagonal tiles skipped)
  5 vertical-slash varlen prefill  (seqlens 65536 + 32768, H=32; conversion + attention)
  6 selected attention             (seqlens 65536 + 32768, 4 heads, top-16 of 64-key blocks)
  7 backward of workload 3         (dQ, dK, dV)

The headline ``value`` / ``ms_per_step`` is workload 2, a step being both attention passes and
the combine; ``config.per_config`` carries every workload's ms per call, rate, dominant kernel,
algorithmic work, roofline fraction and CPU baseline.  ``--config N`` prints workload N alone.

Phase 1 (CPU only, before anything touches the GPU): generate the seeded inputs and time the
float64 oracle on a bounded sample of each workload in a process pool (one worker per host
core, up to 16, each with one BLAS thread).  Phase 2: upload and time each workload on the
GPU with HIP events on the stream the library launches on.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "sparse-attn fwd: effective TFLOP/s (prefill), HBM GB/s (decode), ms/call"
ALL_CONFIGS = (1, 2, 3, 4, 5, 6, 7)
HEADLINE = 2


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=None, choices=list(ALL_CONFIGS),
                    help="one workload only (default: all of them in one line)")
    ap.add_argument("--cpu-seconds", type=float, default=3.0, help="wall-clock budget of each oracle sample")
    ap.add_argument("--settle", type=float, default=0.2,
                    help="seconds each workload runs untimed before its warm-up (GPU clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time decode steps as eager launches instead of HIP graph replays")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 4 device-to-device copies of 1 GiB (reference for HBM byte counters)")
    ap.add_argument("--markers", action="store_true",
                    help="wrap each workload's GPU phase in a roctx range (rocprofv3 --marker-trace shows them)")
    ap.add_argument("--results", default=None,
                    help="append each workload's result, as it completes, as one JSON line to this file")
    ap.add_argument("--resume", action="store_true",
                    help="with --results: reuse the workloads already in the file instead of running them again")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Results file (JSON lines, one per finished workload) and roctx ranges
# ---------------------------------------------------------------------------

def load_results(path):
    """Workload results stored by earlier runs: {workload number: result}; the last line of a
    workload wins, and lines that do not parse (a run cut off mid-write) are skipped."""
    out = {}
    if not path or not os.path.exists(path):
        return out
    with open(path) as f:
        for line in f:
            try:
                rec = json.loads(line)
                out[int(rec["workload_index"])] = rec["result"]
            except (ValueError, KeyError, TypeError):
                continue
    return out


def append_result(path, c, r):
    with open(path, "a") as f:
        f.write(json.dumps({"workload_index": c, "result": r}) + "\n")
        f.flush()


class _Markers:
    """roctx ranges through torch's range API (backed by roctx on ROCm); a no-op if unavailable."""

    def __init__(self, torch):
        self.api = None
        try:
            torch.cuda.nvtx.range_push("bench")
            torch.cuda.nvtx.range_pop()
            self.api = torch.cuda.nvtx
        except Exception as e:  # the profiler's marker library may be absent
            _log(f"markers unavailable ({e}); running without them")

    def push(self, name):
        if self.api:
            self.api.range_push(name)

    def pop(self):
        if self.api:
            self.api.range_pop()


def _log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Inputs (seeded, synthetic)
# ---------------------------------------------------------------------------

def generate(cfg):
    from synth.workloads import (block_sparse_prefill, gated_prefill, selected_prefill, spec_sparse_decode,
                                 tiny_decode, vs_varlen_prefill)
    from synth import normal_bf16

    t0 = time.perf_counter()
    if cfg == 1:
        w = tiny_decode()
    elif cfg == 2:
        w = spec_sparse_decode()
    elif cfg in (3, 7):
        w = block_sparse_prefill()
        if cfg == 7:
            w["do"] = normal_bf16(1007, "do", w["q"].shape)
    elif cfg == 4:
        w = gated_prefill()
    elif cfg == 5:
        w = vs_varlen_prefill()
    else:
        w = selected_prefill()
    _log(f"workload {cfg}: inputs generated in {time.perf_counter() - t0:.1f} s")
    return w


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample, in a process pool
# ---------------------------------------------------------------------------

_W = {}  # workloads, read by the forked workers (copy on write)


def cpu_cores():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _worker_init():
    from threadpoolctl import threadpool_limits

    global _LIMIT
    _LIMIT = threadpool_limits(limits=1)


def _unit_tiny(u):
    import oracle

    w = _W[1]
    t0 = time.perf_counter()
    B, H = w["B"], w["Hq"]
    parts = [oracle.block_sparse(w["q"], w["k"], w["v"], np.full((B, H, 1), w[s].shape[-1], np.int32),
                                 w[s][:, :, None, :], 1, 64) for s in ("set_a", "set_b")]
    oracle.combine(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    return time.perf_counter() - t0, 1.0


def _unit_decode(bh):
    import oracle

    w = _W[2]
    b, h = bh
    G = w["Hq"] // w["Hkv"]
    hs = slice(h * G, (h + 1) * G)
    s0, bs, n = w["spec_start"], w["block_size"], w["missed"].shape[-1]
    t0 = time.perf_counter()
    oracle.speculative_sparse(w["q"][b:b + 1, :, hs], w["k"][b:b + 1, s0:, h:h + 1], w["v"][b:b + 1, s0:, h:h + 1],
                              w["k"][b:b + 1, :, h:h + 1], w["v"][b:b + 1, :, h:h + 1],
                              np.full((1, 1, 1), n, np.int32), w["missed"][b:b + 1, h:h + 1, None, :], bs,
                              causal_spec=True)
    dt = time.perf_counter() - t0
    # algorithmic bytes of one (b, kv head) group: its K/V blocks, Q, O (bf16), LSE, list
    D = w["D"]
    byts = (n + (w["Sk"] - s0) // bs) * bs * D * 4 + G * D * 4 + G * 4 + n * 4 + 4
    return dt, float(byts)


def _unit_block(hi):
    import oracle

    w = _W[3]
    h, i = hi
    G = w["Hq"] // w["Hkv"]
    ents = w["index"][0, h, i, :w["count"][0, h, i]]
    keys = np.concatenate([np.arange(j * 128, (j + 1) * 128) for j in ents])
    rows = np.arange(i * 128, (i + 1) * 128)
    t0 = time.perf_counter()
    oracle.attend_rows(w["q"][0, rows, h], w["k"][0, :, h // G], w["v"][0, :, h // G],
                       [keys[keys <= r] for r in rows], 1.0 / np.sqrt(128))
    return time.perf_counter() - t0, float(len(ents) * 4 * 128 ** 3)


def _unit_gated(hi):
    import oracle
    from synth.workloads import thresholds_from_tile_max

    w = _W[4]
    h, i = hi
    # threshold of this row from the oracle's own tile maxima (the workload's recipe; untimed)
    t = oracle.tile_max_row(w["q"], w["k"], 0, h, i, 128, 128)
    T = thresholds_from_tile_max(t, i)
    t0 = time.perf_counter()
    _, _, keep, _ = oracle.gated_rows(w["q"], w["k"], w["v"], T, 0, h, i, np.arange(i * 128, (i + 1) * 128))
    dt = time.perf_counter() - t0
    return dt, float((i + 1 + int(keep.sum())) * 2 * 128 ** 3)


def _unit_vs(bhm):
    import oracle

    w = _W[5]
    b, h, m = bhm
    L = int(w["seqlens"][b])
    t0 = time.perf_counter()
    wins, cols = oracle.vs_convert_item(L, L, w["vertical"][b, h], w["slash"][b, h], m, 64, 64)
    rows = np.arange(m * 64, min(L, m * 64 + 64))
    oracle.vs_attention_rows(w["q"], w["k"], w["v"], b, h, rows, wins, cols, w["cu_seqlens"], w["cu_seqlens"], 64)
    dt = time.perf_counter() - t0
    return dt, float(4 * 64 * 128 * (64 * len(wins) + len(cols)))


def _unit_selected(bhr):
    import oracle

    w = _W[6]
    b, h, r0 = bhr
    L = int(w["seqlens"][b])
    rows = np.arange(r0, min(L, r0 + 16))
    hk = h // (w["Hq"] // w["Hkv"])
    sel = w["sel"][int(w["cu_seqlens"][b]) + rows, hk]
    t0 = time.perf_counter()
    oracle.selected_rows(w["q"], w["k"], w["v"], w["sel"], 64, w["cu_seqlens"], w["cu_seqlens"], b, h, rows)
    dt = time.perf_counter() - t0
    return dt, float((sel >= 0).sum() * 4 * 64 * 128)


def _unit_backward(hi):
    import oracle

    w = _W[7]
    h, i = hi
    G = w["Hq"] // w["Hkv"]
    ents = np.sort(w["index"][0, h, i, :w["count"][0, h, i]])     # the diagonal block last
    keys = np.concatenate([np.arange(j * 128, (j + 1) * 128) for j in ents])
    rows = slice(i * 128, (i + 1) * 128)
    q = w["q"][:, rows, h:h + 1]
    k = w["k"][:, keys, h // G:h // G + 1]
    v = w["v"][:, keys, h // G:h // G + 1]
    do = w["do"][:, rows, h:h + 1]
    t0 = time.perf_counter()
    oracle.block_sparse_bwd(q, k, v, do, causal=True)
    return time.perf_counter() - t0, float(len(ents) * 5 * 2 * 128 ** 3)


def _units(cfg, w):
    g = np.random.default_rng(cfg)
    if cfg == 1:
        return _unit_tiny, [None] * 100000
    if cfg == 2:
        u = [(b, h) for b in range(w["B"]) for h in range(w["Hkv"])]
        return _unit_decode, [u[j] for j in g.permutation(len(u))]
    if cfg in (3, 4, 7):
        nqb = w["Sq"] // 128
        u = [(int(h), int(i)) for h, i in zip(g.integers(0, w["Hq"], 8192), g.integers(0, nqb, 8192))]
        return {3: _unit_block, 4: _unit_gated, 7: _unit_backward}[cfg], u
    if cfg == 5:
        u = []
        for _ in range(8192):
            b = int(g.integers(0, 2))
            u.append((b, int(g.integers(0, w["H"])), int(g.integers(0, int(w["seqlens"][b]) // 64))))
        return _unit_vs, u
    u = []
    for _ in range(8192):
        b = int(g.integers(0, 2))
        u.append((b, int(g.integers(0, w["Hq"])), int(g.integers(0, int(w["seqlens"][b]) // 16)) * 16))
    return _unit_selected, u


CPU_UNIT = {1: ("ms/call", "calls of the whole workload (set A, set B, combine)"),
            2: ("GB/s", "(batch, kv head) groups: both passes and the combine"),
            3: ("TFLOP/s", "(head, 128-row query block) rows over their listed blocks"),
            4: ("TFLOP/s", "(head, 128-row query block) gated rows: tile maxima, keep rule, attention over kept tiles"
                           " (each row's threshold is picked from the oracle's tile maxima outside the timing)"),
            5: ("TFLOP/s", "(sequence, head, 64-row query block) items: conversion and attention"),
            6: ("TFLOP/s", "16-token runs of one (sequence, head)"),
            7: ("TFLOP/s", "(head, 128-row query block) rows: dQ and the block's dK/dV contributions")}


def cpu_baseline(cfg, w, budget, cores):
    """Float64 oracle rate on a random sample of the workload's independent units, run in a
    pool of `cores` forked workers (one BLAS thread each) until `budget` seconds of wall time
    have passed.  Each unit is timed in its worker; the rate is the work done over the summed
    unit seconds, times the worker count (the whole host's throughput)."""
    import multiprocessing as mp

    fn, units = _units(cfg, w)
    _W.clear()
    _W[cfg] = w
    ctx = mp.get_context("fork")
    secs, work, done = 0.0, 0.0, 0
    t0 = time.perf_counter()
    with ctx.Pool(cores, initializer=_worker_init) as pool:
        for dt, wk in pool.imap_unordered(fn, units):
            secs += dt
            work += wk
            done += 1
            if time.perf_counter() - t0 > budget:
                break
        pool.terminate()
    wall = time.perf_counter() - t0
    _W.clear()
    unit, what = CPU_UNIT[cfg]
    if cfg == 1:
        value = round(secs / done * 1e3, 4)  # per call, each call on one core
    else:
        rate = work / secs * cores
        value = round(rate / (1e9 if unit == "GB/s" else 1e12), 6)
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{'all ' if done == len(units) else ''}{done} {'' if done == len(units) else 'random '}{what} "
                      f"of the same workload, float64 NumPy, {cores} worker processes with "
                      f"one BLAS thread each, {wall:.1f} s wall ({secs:.1f} core-seconds inside the oracle)"}


# ---------------------------------------------------------------------------
# GPU timing helpers
# ---------------------------------------------------------------------------

class Timer:
    """HIP events around named launches on torch's current stream (where the library enqueues)."""

    def __init__(self, torch):
        self.torch = torch
        self.spans = {}

    def span(self, name):
        torch = self.torch
        timer = self

        class _S:
            def __enter__(self):
                self.a = torch.cuda.Event(enable_timing=True)
                self.b = torch.cuda.Event(enable_timing=True)
                self.a.record()

            def __exit__(self, *exc):
                self.b.record()
                timer.spans.setdefault(name, []).append((self.a, self.b))
        return _S()

    def mean_ms(self, name):
        return float(np.mean([a.elapsed_time(b) for a, b in self.spans[name]]))

    def reset(self):
        self.spans = {}


SETTLE_S = 0.2


MIN_TIMED_S = 0.25


def run_steps(torch, step, timer, steps, warmup, min_seconds=0.0):
    """`warmup` untimed steps, then `steps` timed ones (wall clock, synchronized on both sides);
    with min_seconds > 0, at least as many more as fill that long (the count is fixed from the
    settle phase's pace before timing starts).  Before the warm-up the step runs untimed for at least
    SETTLE_S seconds, so that the GPU clock has ramped up from idle (the first tens of
    milliseconds of a heavy kernel run slower); the clock then still wanders by up to 30% for
    tens of milliseconds at a time, which the longer timed window averages out.
    Returns (ms per step, steps timed)."""
    t0 = time.perf_counter()
    settled = 0
    while time.perf_counter() - t0 < SETTLE_S:
        step(timer)
        torch.cuda.synchronize()
        settled += 1
    per = (time.perf_counter() - t0) / settled if settled else None
    for _ in range(warmup):
        step(timer)
    torch.cuda.synchronize()
    n = steps
    if min_seconds > 0 and per is not None:  # without a settle phase there is no pace: K steps
        n = max(steps, min(int(np.ceil(min_seconds / per)), 100000))
    timer.reset()
    t0 = time.perf_counter()
    for _ in range(n):
        step(timer)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / n, n


# HBM bytes per decode launch on the speculative+sparse workload, from two rocprofv3
# --pmc passes (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) each scaled by what the same
# counter reads for a 1 GiB device copy (FETCH_SIZE reads half the bytes: x2.0; WRITE_SIZE
# x1.0).  Valid only for the sources the counters were taken on: the digest covers the
# kernel, its launch planning and the workload generator, and a mismatch reports null.
DECODE_TRAFFIC = {"bytes": 1_286_065_799, "fetch_kib": 624_062, "write_kib": 7_800,
                  "sha256": "e34f948b4bc55e6c18516cfec05dcc586d2dfa8c837e8b8a7b761df1210f0ced"}
TRAFFIC_SOURCES = ["long_context_attention_sparse_amd/csrc/" + f for f in
                   ("decode.cuh", "common.cuh", "args.cuh", "kernels_stream.hip", "decode_plan.h", "host_args.h")] + \
                  ["synth/workloads.py"]


def sources_digest():
    import hashlib

    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def capture(torch, fn):
    """Capture fn (library launches on torch's current stream) into a HIP graph; the
    outputs fn writes are preallocated, so replays reuse the same buffers."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def run_graph_steps(torch, g, steps, min_seconds=0.0, warmup=1):
    """`warmup` untimed replays of g, then wall-clock ms per replay, synchronized on both sides,
    over exactly `steps` replays;
    with min_seconds > 0, over at least as many more as fill that long.  The count is then fixed
    from the pace of SETTLE_S of untimed replays, each waited for, which also bring the clock up
    from idle.  A launch-bound step of tens of microseconds timed over a few replays reads up to
    twice its steady-state time.  Returns (ms per replay, replays timed)."""
    for _ in range(max(1, warmup)):
        g.replay()
    torch.cuda.synchronize()
    n = steps
    if min_seconds > 0:
        t0 = time.perf_counter()
        settled = 0
        while time.perf_counter() - t0 < SETTLE_S:
            g.replay()
            torch.cuda.synchronize()
            settled += 1
        per = (time.perf_counter() - t0) / settled
        n = max(steps, min(int(np.ceil(min_seconds / per)), 100000))
    steps = n
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps, steps


def kernel_mean_ms(torch, fn, per_graph=10, replays=5):
    """Mean device time of the launch fn makes: fn captured per_graph times back to back in
    one HIP graph, HIP events around each replay (so graph launch overhead is amortised and
    the figure compares with a profiler's per-dispatch duration)."""
    g = capture(torch, lambda: [fn() for _ in range(per_graph)])
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    ms = []
    for _ in range(replays):
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b) / per_graph)
    return float(np.mean(ms))


def rotating_mean_ms(torch, fns, reps=12):
    """Mean device time of one launch when its inputs are in no cache: the launches fns[i]
    read disjoint copies of the inputs and are enqueued back to back in turn (no host wait
    between them, one pair of HIP events around the whole run), so the bytes a launch reads
    were last touched len(fns) - 1 launches (gigabytes) earlier, the memory-side cache holds
    another copy, and nothing is written between the events but the launches' own outputs."""
    for f in fns:  # one untimed pass (first touch of each copy)
        f()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    n = reps - reps % len(fns)
    a.record()
    for i in range(n):
        fns[i % len(fns)]()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def free(torch):
    import gc

    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _roof(bound, achieved, kernel, avg_ms, **extra):
    peak = HBM_PEAK_GBS if bound == "hbm" else BF16_PEAK_TFLOPS
    d = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
         "frac": round(achieved / peak, 4), "traffic": None, "kernel": kernel, "avg_ms": round(avg_ms, 5)}
    d.update(extra)
    return d


# ---------------------------------------------------------------------------
# Workload 1: tiny sparse decode (latency)
# ---------------------------------------------------------------------------

def gpu_tiny(torch, bsa, w, args):
    from synth import to_torch_bf16

    dev = torch.device("cuda:0")
    q, k, v = (to_torch_bf16(w[n]).to(dev) for n in ("q", "k", "v"))
    B, H = w["B"], w["Hq"]
    pats = {}
    for name in ("set_a", "set_b"):
        lists = w[name]
        pats[name] = bsa.BlockPattern(torch.full((B, H, 1), lists.shape[-1], dtype=torch.int32, device=dev),
                                      torch.from_numpy(np.ascontiguousarray(lists[:, :, None, :])).to(dev), 128, 64)
    o_part = torch.empty((2, B, 1, H, w["D"]), dtype=torch.float32, device=dev)
    lse_part = torch.empty((2, B, H, 1), dtype=torch.float32, device=dev)
    out = torch.empty((B, 1, H, w["D"]), dtype=torch.bfloat16, device=dev)

    def step(timer):
        with timer.span("set A"):
            bsa.bsa_fwd(q, k, v, pats["set_a"], out=o_part[0], lse=lse_part[0])
        with timer.span("set B"):
            bsa.bsa_fwd(q, k, v, pats["set_b"], out=o_part[1], lse=lse_part[1])
        with timer.span("combine"):
            bsa.bsa_combine(o_part, lse_part, out=out)

    timer = Timer(torch)
    eager_ms, _ = run_steps(torch, step, timer, args.steps, args.warmup)
    spans = {n: round(timer.mean_ms(n) * 1e3, 2) for n in timer.spans}

    def set_a():
        bsa.bsa_fwd(q, k, v, pats["set_a"], out=o_part[0], lse=lse_part[0])

    def full_step():
        set_a()
        bsa.bsa_fwd(q, k, v, pats["set_b"], out=o_part[1], lse=lse_part[1])
        bsa.bsa_combine(o_part, lse_part, out=out)

    n_timed = args.steps
    if args.eager:
        ms, a_ms = eager_ms, timer.mean_ms("set A")
    else:
        # a step of tens of microseconds: timed over at least MIN_TIMED_S of replays
        ms, n_timed = run_graph_steps(torch, capture(torch, full_step), args.steps,
                                      MIN_TIMED_S if args.settle > 0 else 0.0, args.warmup)
        a_ms = kernel_mean_ms(torch, set_a)
    kv = B * H * 16 * 64 * w["D"] * 2 * 2
    a_bytes = B * H * 6 * 64 * w["D"] * 4
    return dict(workload="tiny sparse decode (sets A and B, combine)", value=round(ms, 4), unit="ms/call",
                higher_is_better=False, ms=ms,
                config={"B": B, "H": H, "D": w["D"], "Sk": w["Sk"], "block": 64, "kv_bytes": kv,
                        "timing": "eager" if args.eager else "hip graph replay", "timed_steps": n_timed,
                        "eager_ms_per_step": round(eager_ms, 4), "eager_launch_us": spans,
                        "algorithmic_units": "6 + 10 listed 64-key blocks per head (K and V: 16 KB each), 4 heads"},
                roofline=_roof("hbm", a_bytes / (a_ms * 1e-3) / 1e9, "void bsa::decode_kernel<64>(bsa::DecodeArgs) (set A)",
                               a_ms, note="latency-bound: a few tens of workgroups; HIP events over graph replays include the gap between dispatches, the kernel itself runs about 6 us in a trace"))


# ---------------------------------------------------------------------------
# Workload 2: speculative + sparse decode (headline)
# ---------------------------------------------------------------------------

def gpu_spec_decode(torch, bsa, w, args):
    from synth import to_torch_bf16

    dev = torch.device("cuda:0")
    q, k, v = (to_torch_bf16(w[n]).to(dev) for n in ("q", "k", "v"))
    B, Hq, Hkv, D, Sk, bs = w["B"], w["Hq"], w["Hkv"], w["D"], w["Sk"], w["block_size"]
    s0 = w["spec_start"]
    n_missed = w["missed"].shape[-1]
    count = torch.full((B, Hkv, 1), n_missed, dtype=torch.int32, device=dev)
    index = torch.from_numpy(np.ascontiguousarray(w["missed"][:, :, None, :])).to(dev)
    missed = bsa.BlockPattern(count, index, 128, bs)
    k_spec, v_spec = k[:, s0:], v[:, s0:]
    o_part, lse_part = bsa.bsa_speculative_partials(q, k_spec, v_spec, k, v, missed)
    out = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=dev)

    def step(timer):
        with timer.span("passes"):
            bsa.bsa_speculative_partials(q, k_spec, v_spec, k, v, missed, o_part=o_part, lse_part=lse_part)
        with timer.span("combine"):
            bsa.bsa_combine(o_part, lse_part, out=out, lse=lse)

    timer = Timer(torch)
    eager_ms, _ = run_steps(torch, step, timer, args.steps, args.warmup)
    spans = {n: round(timer.mean_ms(n) * 1e3, 2) for n in timer.spans}
    _log("decode eager per-launch us (host launch gaps included):", spans)

    def passes():
        bsa.bsa_speculative_partials(q, k_spec, v_spec, k, v, missed, o_part=o_part, lse_part=lse_part)

    def full_step():
        passes()
        bsa.bsa_combine(o_part, lse_part, out=out, lse=lse)

    if args.eager:
        ms, pass_ms = eager_ms, timer.mean_ms("passes")
    else:
        # a decode step replays as one HIP graph (launch overhead off the critical path)
        ms, _ = run_graph_steps(torch, capture(torch, full_step), args.steps, warmup=args.warmup)
        pass_ms = kernel_mean_ms(torch, passes)
    groups = B * Hkv
    blk_bytes = bs * D * 2 * 2
    kv_bytes = groups * (n_missed + (Sk - s0) // bs) * blk_bytes
    io_bytes = q.numel() * 2 + out.numel() * 2 + lse.numel() * 4 + index.numel() * 4 + count.numel() * 4
    step_bytes = kv_bytes + io_bytes
    pass_bytes = kv_bytes + q.numel() * 2 + index.numel() * 4 + count.numel() * 4
    achieved = pass_bytes / (pass_ms * 1e-3) / 1e9

    # cold caches: a second copy of K/V, launches alternating between the copies, so every
    # launch reads bytes last touched 1.3 GB of reads earlier (the memory-side cache holds 256 MB)
    k2, v2 = k.clone(), v.clone()
    o_part2, lse_part2 = torch.empty_like(o_part), torch.empty_like(lse_part)
    cold = [passes, lambda: bsa.bsa_speculative_partials(q, k2[:, s0:], v2[:, s0:], k2, v2, missed, o_part=o_part2,
                                                         lse_part=lse_part2)]
    cold_ms = rotating_mean_ms(torch, cold)
    # a plain device copy moving the same number of bytes (half read, half written), timed
    # the same way over two rotating source/destination pairs
    n_el = pass_bytes // 4
    bufs = [(torch.ones(n_el, dtype=torch.bfloat16, device=dev), torch.empty(n_el, dtype=torch.bfloat16, device=dev))
            for _ in range(2)]
    copy_ms = rotating_mean_ms(torch, [lambda p=p: p[1].copy_(p[0]) for p in bufs])
    del k2, v2, o_part2, lse_part2, bufs

    value = step_bytes / (ms * 1e-3) / 1e9
    return dict(workload="speculative+sparse decode", value=round(value, 2), unit="GB/s", ms=ms,
                config={"B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "Sk": Sk, "block": bs, "spec_tokens": Sk - s0,
                        "missed_blocks_per_group": n_missed, "partials": int(o_part.shape[0]),
                        "algorithmic_bytes_per_step": step_bytes,
                        "algorithmic_units": "152 listed 64-key blocks per (batch, kv head) x 256 groups, 32 KB of K "
                                             "and V each, plus Q, O, LSE and the lists",
                        "timing": "eager" if args.eager else "hip graph replay", "eager_ms_per_step": round(eager_ms, 4),
                        "eager_launch_us": spans},
                roofline=_roof("hbm", achieved, "void bsa::decode_kernel<128>(bsa::DecodeArgs) (both passes, one launch)",
                               pass_ms,
                               traffic=DECODE_TRAFFIC["bytes"] if DECODE_TRAFFIC["sha256"] == sources_digest() else None,
                               algorithmic_bytes=pass_bytes,
                               caches_cold={"avg_ms": round(cold_ms, 5),
                                            "achieved": round(pass_bytes / (cold_ms * 1e-3) / 1e9, 1),
                                            "frac": round(pass_bytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                            "method": "two copies of K/V, launches alternating between them, "
                                                      "enqueued back to back",
                                            "device_copy_same_bytes_ms": round(copy_ms, 5),
                                            "device_copy_achieved": round(pass_bytes / (copy_ms * 1e-3) / 1e9, 1)}))


# ---------------------------------------------------------------------------
# Workload 3: block-sparse causal prefill
# ---------------------------------------------------------------------------

def gpu_block_prefill(torch, bsa, w, args):
    from synth import to_torch_bf16

    dev = torch.device("cuda:0")
    q, k, v = (to_torch_bf16(w[n]).to(dev) for n in ("q", "k", "v"))
    pat = bsa.BlockPattern(torch.from_numpy(w["count"]).to(dev), torch.from_numpy(w["index"]).to(dev), 128, 128)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, w["Hq"], w["Sq"]), dtype=torch.float32, device=dev)

    def step(timer):
        with timer.span("prefill"):
            bsa.bsa_fwd(q, k, v, pat, causal=True, out=out, lse=lse)

    timer = Timer(torch)
    ms, n_timed = run_steps(torch, step, timer, args.steps, args.warmup, MIN_TIMED_S)
    tiles = int(w["count"].sum())
    flops = tiles * 4 * 128 ** 3
    kms = timer.mean_ms("prefill")
    return dict(workload="block-sparse causal prefill", value=round(flops / (ms * 1e-3) / 1e12, 2), unit="TFLOP/s",
                ms=ms,
                config={"timed_steps": n_timed, "B": 1, "Hq": 32, "Hkv": 8, "S": w["Sq"], "D": 128, "tile": 128,
                        "visited_tiles": tiles,
                        "flops": flops,
                        "algorithmic_units": f"{tiles} visited 128x128 tiles x 4*128^3 flop (QK and PV)"},
                roofline=_roof("mfma", flops / (kms * 1e-3) / 1e12, "void bsa::prefill_tile_kernel<1, 4>(bsa::PrefillArgs)",
                               kms))


# ---------------------------------------------------------------------------
# Workload 4: gated prefill
# ---------------------------------------------------------------------------

def gpu_gated(torch, bsa, w, args):
    from synth import to_torch_bf16
    from synth.workloads import thresholds_from_tile_max

    dev = torch.device("cuda:0")
    q, k, v = (to_torch_bf16(w[n]).to(dev) for n in ("q", "k", "v"))
    Hq, S = w["Hq"], w["Sq"]
    nqb = S // 128
    # Threshold calibration (the one-time step the gating method describes): exact tile maxima
    # of this input from the kernel with every tile kept, then per query block the gap
    # midpoint nearest half of the off-diagonal tiles.  Not used by any parity check.
    T_all = torch.full((1, Hq, nqb), float("-inf"), dtype=torch.float32, device=dev)
    _, _, _, tmax = bsa.bsa_fwd_gated(q, k, v, T_all, return_mask=False, return_tile_max=True)
    tm = tmax.cpu().numpy()
    T = np.array([[[thresholds_from_tile_max(tm[0, h, i], i) for i in range(nqb)] for h in range(Hq)]], np.float32)
    Td = torch.from_numpy(T).to(dev)
    del tmax
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    keep = [None]

    def step(timer):
        with timer.span("gated"):
            o, l, kmask, _ = bsa.bsa_fwd_gated(q, k, v, Td, out=out)
        keep[0] = kmask

    def step_dense(timer):
        with timer.span("ungated"):
            bsa.bsa_fwd_gated(q, k, v, T_all, out=out, return_mask=False)

    timer = Timer(torch)
    ms, n_timed = run_steps(torch, step, timer, args.steps, args.warmup, MIN_TIMED_S)
    kms = timer.mean_ms("gated")
    km = keep[0].cpu().numpy()
    lower = np.tril(np.ones((nqb, nqb), bool))
    kept = int(km[..., lower].sum())
    causal_tiles = Hq * int(lower.sum())
    flops = causal_tiles * 2 * 128 ** 3 + kept * 2 * 128 ** 3
    def step_count(timer):
        with timer.span("count"):
            bsa.bsa_fwd_gated(q, k, v, Td, out=out, return_mask=False, skipped="count")

    timer2 = Timer(torch)
    run_steps(torch, step_dense, timer2, max(3, args.steps // 4), 2, MIN_TIMED_S)
    ungated_ms = timer2.mean_ms("ungated")
    timer5 = Timer(torch)
    run_steps(torch, step_count, timer5, max(3, args.steps // 4), 2, MIN_TIMED_S)
    count_ms = timer5.mean_ms("count")
    off = lower & ~np.eye(nqb, dtype=bool)
    skip = 1.0 - float(km[..., off].mean())

    # threshold calibration on this input (k = 128 of 512 key blocks), then the gate at it
    k_cal = 128
    cal = {}

    def step_cal(timer):
        with timer.span("calibrate"):
            cal["T"], _ = bsa.bsfa_calibrate(q, k, k_cal)

    def step_cal_gate(timer):
        with timer.span("gated at calibrated T"):
            _, _, cal["keep"], _ = bsa.bsa_fwd_gated(q, k, v, cal["T"], out=out)

    timer3, timer4 = Timer(torch), Timer(torch)
    run_steps(torch, step_cal, timer3, 3, 1)
    run_steps(torch, step_cal_gate, timer4, 3, 1)
    cal_ms, cal_gate_ms = timer3.mean_ms("calibrate"), timer4.mean_ms("gated at calibrated T")
    ckeep = cal["keep"].cpu().numpy()
    realised = float(ckeep[..., lower].sum()) / (Hq * int(lower.sum()))
    target = float(np.sum(np.minimum(k_cal, np.arange(nqb)) + 1)) / int(lower.sum())
    cal_flops = causal_tiles * 2 * 128 ** 3  # the tile maxima: S on every causal tile
    calibration = {"k": k_cal, "ms": round(cal_ms, 4), "tflops": round(cal_flops / (cal_ms * 1e-3) / 1e12, 2),
                   "target_density": round(target, 4), "realised_density": round(realised, 4),
                   "gated_ms_at_calibrated_T": round(cal_gate_ms, 4)}
    return dict(workload="BSFA gated causal prefill", value=round(flops / (ms * 1e-3) / 1e12, 2), unit="TFLOP/s", ms=ms,
                config={"timed_steps": n_timed, "B": 1, "Hq": Hq, "Hkv": 8, "S": S, "D": 128, "tile": 128,
                        "skip_fraction_offdiag": round(skip, 4), "flops": flops,
                        "algorithmic_units": f"QK on {causal_tiles} causal 128x128 tiles and PV on {kept} kept tiles, "
                                             "2*128^3 flop each",
                        "gated_ms": round(kms, 4), "ungated_ms": round(ungated_ms, 4),
                        "gated_speedup": round(ungated_ms / kms, 3),
                        "skipped_counted_ms": round(count_ms, 4),
                        "skipped_counted_note": "the other reading of a skipped tile: its scores stay in the "
                                                "softmax maximum and normaliser (the timed line drops them)",
                        "calibration": calibration},
                roofline=_roof("mfma", flops / (kms * 1e-3) / 1e12, "void bsa::gated_kernel<false, false>(bsa::GatedArgs)", kms))


# ---------------------------------------------------------------------------
# Workload 5: vertical-slash conversion + varlen prefill
# ---------------------------------------------------------------------------

def gpu_vs(torch, bsa, w, args):
    from synth import to_torch_bf16

    dev = torch.device("cuda:0")
    q, k, v = (to_torch_bf16(w[n]).to(dev) for n in ("q", "k", "v"))
    sl = torch.from_numpy(w["seqlens"]).to(dev)
    vert = torch.from_numpy(w["vertical"]).to(dev)
    slash = torch.from_numpy(w["slash"]).to(dev)
    cu = torch.from_numpy(w["cu_seqlens"]).to(dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w["H"], q.shape[0]), dtype=torch.float32, device=dev)
    res = {}

    def step(timer):
        with timer.span("convert"):
            bc, bo, cc, ci = bsa.vs_convert_indexes(sl, sl, vert, slash, w["context_size"], 64, 64)
        with timer.span("attention"):
            bsa.bsa_fwd(q, k, v, bsa.VSPattern(bc, bo, cc, ci, 64, 64), causal=True, out=out, lse=lse,
                        cu_seqlens_q=cu, cu_seqlens_k=cu, max_seqlen_q=w["max_seqlen"], max_seqlen_k=w["max_seqlen"])
        res["m"] = (bc, cc)

    timer = Timer(torch)
    ms, n_timed = run_steps(torch, step, timer, args.steps, args.warmup, MIN_TIMED_S)
    bc, cc = (x.cpu().numpy().astype(np.int64) for x in res["m"])
    flops = int((4 * 64 * 128 * (64 * bc + cc)).sum())
    ams = timer.mean_ms("attention")
    cms = timer.mean_ms("convert")
    conv_bytes = int(4 * (bc.sum() + cc.sum() + bc.size + cc.size))
    return dict(workload="vertical-slash conversion + varlen causal prefill",
                value=round(flops / (ms * 1e-3) / 1e12, 2), unit="TFLOP/s", ms=ms,
                config={"timed_steps": n_timed, "seqlens": [65536, 32768], "H": 32, "D": 128, "block": 64,
                        "nnz_v": 1000, "nnz_s": 2000,
                        "flops": flops, "attention_ms": round(ams, 4), "convert_ms": round(cms, 4),
                        "convert_output_bytes": conv_bytes,
                        "convert_gbs": round(conv_bytes / (cms * 1e-3) / 1e9, 1),
                        "algorithmic_units": "per (sequence, head, 64-row query block): 4*64*128*(64*block_count + "
                                             "column_count) flop over its windows and columns"},
                roofline=_roof("mfma", flops / (ams * 1e-3) / 1e12, "void bsa::vs_pair_kernel<8>(bsa::PrefillArgs)",
                               ams))


# ---------------------------------------------------------------------------
# Selected attention (top-k key blocks per query token), the FSA module's example shape
# ---------------------------------------------------------------------------

def gpu_selected(torch, bsa, w, args):
    from synth import to_torch_bf16

    dev = torch.device("cuda:0")
    q, k, v = (to_torch_bf16(w[n]).to(dev) for n in ("q", "k", "v"))
    sel = torch.from_numpy(w["sel"]).to(dev)
    cu = torch.from_numpy(w["cu_seqlens"]).to(dev)
    Hq, Hkv, topk, T = w["Hq"], w["Hkv"], w["topk"], q.shape[0]
    G = Hq // Hkv
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty(bsa.bsa_selected_workspace_size(q, k, topk, cu_seqlens_q=cu, cu_seqlens_k=cu,
                                                     max_seqlen_q=w["max_seqlen"], max_seqlen_k=w["max_seqlen"]),
                     dtype=torch.uint8, device=dev)

    def call():
        bsa.bsa_fwd_selected(q, k, v, sel, out=out, lse=lse, workspace=ws, cu_seqlens_q=cu, cu_seqlens_k=cu,
                             max_seqlen_q=w["max_seqlen"], max_seqlen_k=w["max_seqlen"])

    def step(timer):
        with timer.span("selected"):
            call()

    timer = Timer(torch)
    ms, n_timed = run_steps(torch, step, timer, args.steps, args.warmup, MIN_TIMED_S)
    call_ms = kernel_mean_ms(torch, call)
    # work the call must do: every selection here is valid (the generator draws causal blocks)
    s_np = w["sel"]
    pairs = int((s_np >= 0).sum())
    empty = int(s_np.size - pairs)
    flops = pairs * G * 4 * 64 * 128
    lists = np.zeros(0, np.int64)
    nkb = -(-w["max_seqlen"] // 64)
    for b in range(len(w["seqlens"])):
        a0, a1 = int(w["cu_seqlens"][b]), int(w["cu_seqlens"][b + 1])
        for hk in range(Hkv):
            blk = s_np[a0:a1, hk][s_np[a0:a1, hk] >= 0]
            lists = np.concatenate([lists, np.bincount(blk, minlength=nkb)])
    tpc = 128 // G
    chunks = int(((lists + tpc - 1) // tpc).sum())
    row = 128 * 4 + 4                                         # a float32 partial (o, lse)
    alg_bytes = (pairs * (G * 256 + G * row + 2 * 4)          # gathered Q rows, partials, sel + list entry
                 + empty * (G * row + 4)                      # neutral partials of unused slots
                 + chunks * 64 * 256 * 2                      # one K and V tile per chunk
                 + T * Hq * (topk * row + 128 * 2 + 4))       # combine: read partials, write O (bf16), LSE
    gbs = alg_bytes / (call_ms * 1e-3) / 1e9
    return dict(workload="selected attention, top-k key blocks per query token (key-block-outer)",
                value=round(flops / (ms * 1e-3) / 1e12, 2), unit="TFLOP/s", ms=ms,
                config={"timed_steps": n_timed, "seqlens": [int(x) for x in w["seqlens"]], "Hq": Hq, "Hkv": Hkv,
                        "D": 128, "block": 64,
                        "topk": topk, "valid_pairs": pairs, "chunks": chunks, "flops": flops,
                        "algorithmic_bytes": alg_bytes,
                        "algorithmic_units": "gathered Q rows, one K/V tile per chunk of 128/G tokens, float32 "
                                             "partials written and read, bf16 O"},
                roofline=_roof("hbm", gbs, "bsa_fwd_selected (index inversion, selected_kernel, combine_kernel)",
                               call_ms))


# ---------------------------------------------------------------------------
# Backward of the block-sparse prefill workload
# ---------------------------------------------------------------------------

def gpu_backward(torch, bsa, w, args):
    from synth import to_torch_bf16

    dev = torch.device("cuda:0")
    q, k, v = (to_torch_bf16(w[n]).to(dev) for n in ("q", "k", "v"))
    do = to_torch_bf16(w["do"]).to(dev)
    pat = bsa.BlockPattern(torch.from_numpy(w["count"]).to(dev), torch.from_numpy(w["index"]).to(dev), 128, 128)
    out, lse = bsa.bsa_fwd(q, k, v, pat, causal=True, out_dtype=torch.bfloat16)
    ws = torch.empty(bsa.bsa_bwd_workspace_size(q, k, pat, causal=True), dtype=torch.uint8, device=dev)

    def step(timer):
        with timer.span("backward"):
            bsa.bsa_bwd(q, k, v, out, lse, do, pat, causal=True, workspace=ws)

    timer = Timer(torch)
    ms, n_timed = run_steps(torch, step, timer, args.steps, args.warmup, MIN_TIMED_S)
    bms = timer.mean_ms("backward")
    tiles = int(w["count"].sum())
    flops = tiles * 5 * 2 * 128 ** 3   # S (rebuilt), dP, dV, dQ, dK: five tile products
    return dict(workload="block-sparse causal prefill backward (dQ, dK, dV)",
                value=round(flops / (ms * 1e-3) / 1e12, 2), unit="TFLOP/s", ms=ms,
                config={"timed_steps": n_timed, "B": 1, "Hq": 32, "Hkv": 8, "S": 32768, "D": 128, "tile": 128,
                        "visited_tiles": tiles,
                        "flops": flops,
                        "algorithmic_units": "5 products of 2*128^3 per visited tile (S, dP, dV, dQ, dK); the dQ pass "
                                             "rebuilds S and dP a second time: 7 executed"},
                roofline=_roof("mfma", flops / (bms * 1e-3) / 1e12,
                               "bsa_bwd (bwd_dkdv_kernel + bwd_dq_kernel<4> + list inversion)", bms))


GPU = {1: gpu_tiny, 2: gpu_spec_decode, 3: gpu_block_prefill, 4: gpu_gated, 5: gpu_vs, 6: gpu_selected,
       7: gpu_backward}


def main():
    args = _args()
    global SETTLE_S
    SETTLE_S = args.settle
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the kernels are single-GPU and "
              "the multi-GPU sharding is a design note, not part of this build.", file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_attention_sparse_amd as bsa

    if args.copy_calibration:
        if not torch.cuda.is_available():
            sys.exit("bench.py needs a GPU")
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 4}), flush=True)
        return
    configs = [args.config] if args.config else list(ALL_CONFIGS)
    done = load_results(args.results) if args.resume else {}
    if done:
        _log(f"reusing stored results of workloads {sorted(set(done) & set(configs))} from {args.results}")

    # ---- phase 1: inputs and the oracle's CPU baseline (the GPU is not touched yet) ----
    work = {}
    cpu = {}
    cores = cpu_cores()
    for c in configs:
        if c in done:
            continue
        w = work[3] if c == 7 and 3 in work else None
        if w is not None:
            from synth import normal_bf16

            w = dict(w)
            w["do"] = normal_bf16(1007, "do", w["q"].shape)
        work[c] = w if w is not None else generate(c)
        if not args.no_cpu_baseline:
            t0 = time.perf_counter()
            cpu[c] = cpu_baseline(c, work[c], args.cpu_seconds, cores)
            _log(f"workload {c}: oracle sample {cpu[c]['value']} {cpu[c]['unit']} ({time.perf_counter() - t0:.1f} s)")

    # ---- phase 2: the GPU ----
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bsa.load()
    res = {}
    markers = _Markers(torch) if args.markers else None
    for c in configs:
        if c in done:
            res[c] = done[c]
            continue
        _log(f"workload {c}: timing on the GPU")
        if markers:
            markers.push(f"workload {c}")
        res[c] = GPU[c](torch, bsa, work[c], args)
        if markers:
            markers.pop()
        res[c]["cpu_baseline"] = cpu.get(c)
        free(torch)
        _log(f"workload {c}: {res[c]['value']} {res[c]['unit']}, {res[c]['ms']:.4f} ms per call")
        if args.results:
            append_result(args.results, c, res[c])

    head = HEADLINE if HEADLINE in res else configs[0]
    r = res[head]
    cfg = {"workload": r["workload"], **r["config"]}
    if len(configs) > 1:
        cfg["headline"] = f"workload {head} ({r['workload']})"
        cfg["per_config"] = {
            str(c): {"workload": res[c]["workload"], "ms_per_call": round(res[c]["ms"], 4), "value": res[c]["value"],
                     "unit": res[c]["unit"], "higher_is_better": res[c].get("higher_is_better", True),
                     "kernel": res[c]["roofline"]["kernel"], "config": res[c]["config"],
                     "roofline": res[c]["roofline"], "cpu_baseline": res[c]["cpu_baseline"]}
            for c in configs}
    line = {"metric": METRIC, "value": r["value"], "unit": r["unit"], "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(r["ms"], 4),
            "higher_is_better": r.get("higher_is_better", True), "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic", "config": cfg, "roofline": r["roofline"],
            "cpu_baseline": r["cpu_baseline"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
