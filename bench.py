#!/usr/bin/env python3
"""Throughput of tree-causal paged attention on one MI355X.

One *step* is the whole hot path of one decode step over one batch of
synthetic inputs: the plan (parent array -> ancestor bitmask, depth, position
ids), the paged prefix, the masked tree and the split-K merge, run as one
``tree_attn_plan_fwd`` call, which builds the plan inside the attention
kernel.  Inputs are resident in HBM before timing starts.  Steps are replayed
from HIP graphs holding one step per input replica (a replica cycle; a step
count short of a cycle replays a graph of the remaining steps, captured
beforehand), and successive steps rotate over enough replicas that the
working set does not stay in the 256 MB Infinity Cache.  Before any timing,
at least 1.5 s of untimed steps bring the clocks up (and keep the GPU
visibly busy to an outside utilisation sampler), whatever ``--warmup`` says; then ``--warmup`` untimed steps, then exactly ``--steps`` steps timed
with HIP events on the replay stream.  ``value`` is tree tokens per second of
that GPU time.  The headline workload then runs on, back to back, for
``--sustain-seconds`` of GPU time (default 8), reported as ``sustained``: the
rate over that run and its slowest half-second block.

Beside it: ``fwd_only`` (tree_attn_fwd alone, mask words from an earlier
plan), ``plan_only`` (tree_attn_plan alone), ``two_call`` (plan, then
forward), and the attention kernel's own mean launch time, from which
``roofline`` is computed.

Default workload: ``chain16`` (budget 16: 1 request, prefix 2048, a 16-node
chain, 32/8 heads, head_dim 128, bf16), the HBM-bound case.  The same run
also measures ``moe`` (budget 256: 32 requests, prefix 4096, best-first trees
of 256 nodes, 32/4 heads; under ``budget256``), ``tree256`` (one request of
budget 256) and ``mixed`` (8 requests, prefixes 512..8192, budget 64), each
with its roofline and CPU oracle baseline.  One JSON line goes to stdout;
diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import tree_masked_attention_plan_amd as ta  # noqa: E402
from tree_masked_attention_plan_amd import workloads as W  # noqa: E402

METRIC = "tree-attn tree tokens/s + % bf16 MFMA peak (budget 256) / % HBM BW (budget 16)"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3
KERNEL_SRC = os.path.join(HERE, "tree_masked_attention_plan_amd", "csrc", "attn.hip")
PROFILES = os.path.join(HERE, "profiles")
ROTATE_BYTES = 600 << 20       # cycle at least this much input per pass over replicas
MAX_REPLICAS = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- accounting

def node_depths(w: W.Workload) -> np.ndarray:
    """Path length of every node (host-side statistic for work accounting)."""
    par = w.parent.numpy()
    off = w.tree_off.numpy()
    d = np.zeros(w.N, dtype=np.int64)
    for b in range(w.B):
        for i in range(off[b + 1] - off[b]):
            p = par[off[b] + i]
            d[off[b] + i] = 1 if p < 0 else d[off[b] + p] + 1
    return d


def work(w: W.Workload, nsplit: int) -> dict:
    """Algorithmic work of one step (plan and attention in one call), over
    visible (query, key) pairs.

    flops = 4 * D * Hq * (sum_b T_b * L_b + sum_i depth_i)   (QK^T and PV)
    bytes = valid prefix K/V + tree K/V + Q + O + LSE + the parent array read
            and the plan's outputs written (mask words that can hold a
            visible bit, ceil(T_b / 64) per node, depth, position id, status)
            + live block-table entries.  ``kernel_bytes`` is the part the
            attention kernel itself must move: everything but O and LSE when
            a separate merge writes them (split count > 1)."""
    e = torch.tensor([], dtype=w.dtype).element_size()
    T = w.tree_sizes
    L = w.prefix_len.numpy().astype(np.int64)
    sdepth = int(node_depths(w).sum())
    pairs = int((T * L).sum()) + sdepth
    flops = 4.0 * w.D * w.Hq * pairs
    N = w.N
    kv = int(L.sum()) * w.Hkv * w.D * 2 * e + N * w.Hkv * w.D * 2 * e
    q = N * w.Hq * w.D * e
    o = N * w.Hq * w.D * e + N * w.Hq * 4
    plan = N * 4 + int((T * ((T + 63) // 64)).sum()) * 8 + N * 8 + w.B * 4
    bt = int(((L + w.page_size - 1) // w.page_size).sum()) * 4
    total = kv + q + o + plan + bt
    kernel = total if nsplit == 1 else total - o
    return {"flops": flops, "bytes": float(total), "kernel_bytes": float(kernel),
            "pairs": pairs, "sum_depth": sdepth, "tree_tokens": N}


# ---------------------------------------------------------------- device side

class Replica:
    def __init__(self, w: W.Workload, dev):
        self.w = w.to(dev)
        n, b = w.N, w.B
        self.plan_out = ta.PlanResult(torch.empty((n, ta.MASK_WORDS), dtype=torch.int64, device=dev),
                                      torch.empty(n, dtype=torch.int32, device=dev),
                                      torch.empty(n, dtype=torch.int32, device=dev),
                                      torch.empty(b, dtype=torch.int32, device=dev))
        # the plan writes anc_mask before the forward reads it; run it once
        # here so that the forward can be prepared against the same buffers
        ta.plan(self.w.parent, self.w.tree_off, self.w.prefix_len, max_tree=w.max_tree,
                out=self.plan_out)
        self.call = ta.prepare_fwd(self.w.q, self.w.k_tree, self.w.v_tree, self.w.k_cache,
                                   self.w.v_cache, self.w.block_table, self.w.prefix_len,
                                   self.w.tree_off, self.plan_out.anc_mask, max_tree=w.max_tree,
                                   max_prefix=w.max_prefix)
        # the same step as one call: the plan built inside the attention
        # kernel, into the same plan, output and workspace buffers
        self.pcall = ta.prepare_plan_fwd(self.w.q, self.w.k_tree, self.w.v_tree, self.w.k_cache,
                                         self.w.v_cache, self.w.block_table, self.w.prefix_len,
                                         self.w.tree_off, self.w.parent, max_tree=w.max_tree,
                                         max_prefix=w.max_prefix, plan_out=self.plan_out,
                                         out=self.call.out, lse=self.call.lse,
                                         workspace=self.call.workspace)
        self.max_tree = w.max_tree
        # with fp32 the one call runs the plan kernel and the attention kernel
        self.fused = w.dtype == torch.bfloat16

    def step(self):
        """Plan + attention + merge: tree_attn_plan_fwd."""
        self.pcall.run()

    def step_two_call(self):
        """The same step as tree_attn_plan, then tree_attn_fwd."""
        ta.plan(self.w.parent, self.w.tree_off, self.w.prefix_len, max_tree=self.max_tree,
                out=self.plan_out)
        self.call.partial()
        self.call.merge()

    def partial(self):
        """The attention kernel of the step alone."""
        if self.fused:
            self.pcall.partial()
        else:
            self.call.partial()

    def fwd(self):
        self.call.partial()
        self.call.merge()

    def plan(self):
        """The plan alone (tree_attn_plan), reported separately."""
        ta.plan(self.w.parent, self.w.tree_off, self.w.prefix_len, max_tree=self.max_tree,
                out=self.plan_out)


def replica_bytes(w: W.Workload) -> int:
    t = 0
    for x in (w.q, w.k_tree, w.v_tree, w.k_cache, w.v_cache):
        t += x.numel() * x.element_size()
    return t


def capture(fn, n_rep):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_rep):
            fn()
    return g


class Runner:
    """Graphs over the replicas: ``chunk`` runs one step on every replica in
    turn (one replica cycle), ``partial_chunk`` only the attention kernel on
    every replica (for the per-launch kernel time).  A step count that is not
    a whole number of cycles replays a graph of the remaining steps, captured
    beforehand by :meth:`prepare`, so that no capture and no per-step host
    launch falls inside a timed region."""

    def __init__(self, reps, compare=True):
        self.reps = reps
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for r in reps:        # eager warm-up before capture
                r.step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.chunk = capture(lambda: [r.step() for r in reps], 1)
        self.rest = {}
        self.partial_chunk = capture(lambda: [r.partial() for r in reps], 1)
        # the comparison forms launch the same attention kernel symbol; a
        # profiling run can leave them out so that its trace holds the step's
        # launches only
        self.fwd_chunk = capture(lambda: [r.fwd() for r in reps], 1) if compare else None
        self.two_call_chunk = capture(lambda: [r.step_two_call() for r in reps], 1) if compare else None
        self.plan_chunk = capture(lambda: [r.plan() for r in reps], 1) if compare else None
        torch.cuda.synchronize()

    def prepare(self, *counts):
        """Capture the remainder graphs that ``run_steps`` needs for these
        step counts (steps on replicas 0 .. k % R - 1), and replay each new
        one once, untimed: a graph's first replay also uploads it."""
        R = len(self.reps)
        for k in counts:
            m = k % R
            if m and m not in self.rest:
                self.rest[m] = capture(lambda: [r.step() for r in self.reps[:m]], 1)
                self.rest[m].replay()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(1000)   # load the spin kernel of _busy_stream outside any timing
        torch.cuda.synchronize()

    def run_steps(self, k):
        R = len(self.reps)
        for _ in range(k // R):
            self.chunk.replay()
        if k % R:
            self.rest[k % R].replay()


def ramp_clocks(runner: Runner, seconds: float = 1.5) -> float:
    """Untimed GPU work before any timing (whatever --warmup says): whole
    replica cycles until at least ``seconds`` of GPU time have passed, so
    that the timed steps do not catch the clocks ramping up.  Returns the
    GPU seconds spent."""
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    spent = 0.0
    n = 1
    while spent < seconds:
        e0.record(stream)
        for _ in range(n):
            runner.chunk.replay()
        e1.record(stream)
        e1.synchronize()
        spent += e0.elapsed_time(e1) / 1e3
        n = min(n * 2, 64)
    return spent


def _busy_stream(runner: Runner):
    """Untimed GPU work that keeps the stream busy while the host enqueues
    the start event and the timed steps, so that the GPU does not sit idle
    between that event and the first timed step (an idle gap of tens of
    microseconds that a short timed region would otherwise count): a spin
    of about 100 us, or one replica cycle without it."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(200_000)
    else:
        runner.chunk.replay()


def time_steps(runner: Runner, steps: int, warmup: int) -> tuple:
    """``warmup`` untimed steps, then exactly ``steps`` steps bracketed by
    device synchronisations.  Returns (GPU seconds from HIP events recorded
    on the replay stream around the steps, host wall seconds; the wall time
    also holds the short untimed spin ahead of the start event)."""
    runner.prepare(steps, warmup)
    runner.run_steps(warmup)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    _busy_stream(runner)
    e0.record(stream)
    runner.run_steps(steps)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall


def sustain(runner: Runner, seconds: float, tree_tokens: int) -> dict:
    """Whole replica cycles back to back for about ``seconds`` of GPU time,
    after the timed steps: whether the step rate holds over a long run, with
    clocks and power at steady state.  Timed with HIP events on the replay
    stream around blocks of about half a second; reports the rate over all
    blocks and the slowest block's."""
    R = len(runner.reps)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    runner.chunk.replay()
    e1.record(stream)
    e1.synchronize()
    per_cycle = max(e0.elapsed_time(e1) / 1e3, 1e-6)
    n = max(1, int(0.5 / per_cycle))                            # cycles per block
    blocks = max(1, int(round(seconds / (n * per_cycle))))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    _busy_stream(runner)
    ev[0].record(stream)
    for i in range(blocks):
        for _ in range(n):
            runner.chunk.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    times = [ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(blocks)]
    steps = blocks * n * R
    total = sum(times)
    return {"seconds": total, "steps": steps, "blocks": blocks,
            "value": tree_tokens * steps / total, "ms_per_step": total / steps * 1e3,
            "slowest_block_value": tree_tokens * n * R / max(times)}


def time_partial_kernel(runner: Runner, min_launches: int = 200, graph=None) -> float:
    """Average duration (s) of one attention-kernel launch (or, with
    ``graph``, of one call of what it captured per replica): HIP events on
    the stream the graph's kernels run on, around back-to-back replays."""
    R = len(runner.reps)
    reps = max(1, math.ceil(min_launches / R))
    graph = runner.partial_chunk if graph is None else graph
    graph.replay()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / (reps * R)


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(w: W.Workload, target_s: float) -> dict:
    """The fp64 oracle on this host, on a bounded sample of the workload.

    Inputs are widened to fp64 once, outside the timed calls; the oracle runs
    with one thread per available core."""
    import oracle
    threads = oracle.default_threads()
    arrays = [x.double().numpy() for x in (w.q, w.k_tree, w.v_tree, w.k_cache, w.v_cache)]
    ints = [x.numpy() for x in (w.block_table, w.prefix_len, w.tree_off, w.parent)]

    def run(rows=None):
        return oracle.tree_attn(*arrays, *ints, scale=w.scale, rows=rows, threads=threads)

    rows_total = w.N * w.Hq
    # estimate the cost per row from a small slice, then size the sample
    probe = np.arange(0, rows_total, max(1, rows_total // 256), dtype=np.int64)[:256]
    t0 = time.perf_counter()
    run(probe)
    per_row = max((time.perf_counter() - t0) / len(probe), 1e-9)
    if per_row * rows_total <= target_s:
        reps = max(1, int(target_s / (per_row * rows_total)))
        t0 = time.perf_counter()
        for _ in range(reps):
            run()
        dt = time.perf_counter() - t0
        tokens = w.N * reps
        sample = f"the whole workload ({w.N} tree tokens, {rows_total} rows), {reps} runs"
    else:
        n_nodes = max(1, min(w.N, int(target_s / per_row) // w.Hq))
        nodes = np.sort(np.random.default_rng(0).choice(w.N, size=n_nodes, replace=False))
        rows = (nodes[:, None] * w.Hq + np.arange(w.Hq)[None, :]).reshape(-1)
        t0 = time.perf_counter()
        run(rows)
        dt = time.perf_counter() - t0
        tokens = n_nodes
        sample = (f"{n_nodes} of {w.N} tree tokens (all {w.Hq} heads each), seeded uniform "
                  f"sample, 1 run")
    return {"value": tokens / dt, "unit": "tree tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3)}


# ---------------------------------------------------------------- traffic

def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def traffic_for(workload: str):
    """HBM bytes per launch of the attention kernel from committed counter
    summaries, or None if absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"fwd_bf16_kernel_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha256_16") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- main

def roofline(kind: str, wk: dict, t_kern: float, name: str, kernel: str, peak_flops: float) -> dict:
    """Roofline entry of the step's attention kernel: algorithmic FLOPs
    (``mfma``) or bytes (``hbm``) of one launch over its mean launch time."""
    if kind == "mfma":
        ach = wk["flops"] / t_kern / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": peak_flops, "unit": "TFLOP/s",
                "frac": ach / peak_flops, "traffic": traffic_for(name), "kernel": kernel,
                "kernel_us": t_kern * 1e6, "flops_per_launch": wk["flops"]}
    ach = wk["kernel_bytes"] / t_kern / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBS, "traffic": traffic_for(name), "kernel": kernel,
            "kernel_us": t_kern * 1e6, "bytes_per_launch": wk["kernel_bytes"]}


# which roofline bounds each workload's attention kernel (mixed sits near the
# ridge point, so both fractions are reported for it)
BOUND = {"tiny": "hbm", "chain16": "hbm", "tree256": "mfma", "mixed": "mfma", "moe": "mfma"}


def measure(name: str, steps: int, warmup: int, dev, cpu: bool, cpu_seconds: float,
            compare: bool = True, sustain_s: float = 0.0) -> dict:
    """One workload: ``warmup`` untimed steps after a clock ramp, then
    exactly ``steps`` steps timed with HIP events on the replay stream.
    ``value`` = tree tokens per second of GPU time over those steps.  With
    ``sustain_s`` > 0 the steps then run on for about that many seconds
    (:func:`sustain`)."""
    w = W.make_config(name)
    per = replica_bytes(w)
    R = max(1, min(MAX_REPLICAS, math.ceil(ROTATE_BYTES / per)))
    log(f"[bench] {name}: B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} max_prefix={w.max_prefix} "
        f"replicas={R} ({per / 2**20:.1f} MiB each)")
    reps = [Replica(w, dev) for _ in range(R)]
    ta.check_status(reps[0].plan_out.status)
    runner = Runner(reps, compare)
    nsplit = reps[0].call.num_splits
    wk = work(w, nsplit)
    runner.prepare(steps, warmup)   # before the ramp: no first replay in a timed region
    ramp = ramp_clocks(runner)
    gpu_s, wall_s = time_steps(runner, steps, warmup)
    ms = gpu_s / steps * 1e3
    t_kern = time_partial_kernel(runner)
    t_fwd = time_partial_kernel(runner, graph=runner.fwd_chunk) if compare else float("nan")
    t_two = time_partial_kernel(runner, graph=runner.two_call_chunk) if compare else float("nan")
    t_plan = time_partial_kernel(runner, graph=runner.plan_chunk) if compare else float("nan")
    log(f"[bench] {name}: {ms * 1e3:.2f} us/step of GPU time ({wall_s / steps * 1e6:.2f} us wall; "
        f"one call, the plan inside the attention kernel; {ramp * 1e3:.0f} ms clock ramp), "
        f"attention kernel {t_kern * 1e6:.2f} us/launch; forward call alone {t_fwd * 1e6:.2f} us, "
        f"plan alone {t_plan * 1e6:.2f} us, plan then forward {t_two * 1e6:.2f} us, splits={nsplit}")
    res = {
        "workload": name,
        "value": wk["tree_tokens"] * steps / gpu_s,
        "ms_per_step": ms,
        "wall_ms_per_step": wall_s / steps * 1e3,
        "steps": steps,
        "warmup": warmup,
        "num_splits": nsplit,
        "tflops": wk["flops"] / (ms * 1e-3) / 1e12,
        "kernel_us": t_kern * 1e6,
        # tree_attn_fwd alone (mask words from an earlier plan; attention
        # kernel and split merge), replayed back to back: tree tokens per
        # second over the forward call's GPU time, the plan excluded
        "fwd_only": ({"value": wk["tree_tokens"] / t_fwd, "unit": "tree tokens/s", "us": t_fwd * 1e6}
                     if compare else None),
        # tree_attn_plan alone, and the step as two calls (plan, then forward)
        "plan_only": {"us": t_plan * 1e6} if compare else None,
        "two_call": ({"value": wk["tree_tokens"] / t_two, "unit": "tree tokens/s", "us": t_two * 1e6}
                     if compare else None),
        "work": wk,
        "config": {"workload": name, "B": w.B, "tree_tokens": w.N, "max_tree": w.max_tree,
                   "prefix_tokens": int(w.prefix_len.sum()), "max_prefix": w.max_prefix,
                   "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D, "page_size": w.page_size,
                   "num_splits": nsplit, "replicas": R},
    }
    is_bf16 = w.dtype == torch.bfloat16
    kernel = "fwd_bf16_kernel" if is_bf16 else "fwd_f32_kernel"
    peak = PEAK_BF16_TFLOPS if is_bf16 else PEAK_FP32_TFLOPS
    res["roofline"] = roofline(BOUND[name], wk, t_kern, name, kernel, peak)
    if name == "mixed":
        res["roofline_hbm"] = roofline("hbm", wk, t_kern, name, kernel, peak)
    if sustain_s > 0:
        res["sustained"] = sustain(runner, sustain_s, wk["tree_tokens"])
        log(f"[bench] {name}: sustained {res['sustained']['ms_per_step'] * 1e3:.2f} us/step over "
            f"{res['sustained']['seconds']:.1f} s of GPU time ({res['sustained']['steps']} steps)")
    del runner, reps
    torch.cuda.empty_cache()
    if cpu:
        res["cpu_baseline"] = cpu_baseline(w, cpu_seconds)
        log(f"[bench] {name}: oracle {res['cpu_baseline']['value']:.1f} tree tokens/s on "
            f"{res['cpu_baseline']['cores']} cores ({res['cpu_baseline']['sample']})")
    return res


def _counter_mean_kib(dirpath: str, counter: str, kernel_substr: str) -> tuple:
    """Mean per-dispatch value of a rocprofv3 counter (summed over its
    instances) for the dispatches whose kernel name contains kernel_substr."""
    import csv
    import glob
    files = glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {dirpath}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter or kernel_substr not in r["Kernel_Name"]:
                continue
            key = (f, r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} samples for '{kernel_substr}' under {dirpath}")
    vals = sorted(per.values())
    return sum(vals) / len(vals), len(vals)


def summarize_traffic(workload: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str,
                      copy_write_dir: str, copy_mib: int, out_path: str):
    """HBM bytes per attention-kernel launch from FETCH_SIZE / WRITE_SIZE
    passes, each scaled by what the same counter reads for a plain copy of
    known size (the copy of --calibrate-copy-mib)."""
    kern = "fwd_bf16_kernel"
    copy_k = "vectorized_elementwise_kernel"
    f_kib, nf = _counter_mean_kib(fetch_dir, "FETCH_SIZE", kern)
    w_kib, nw = _counter_mean_kib(write_dir, "WRITE_SIZE", kern)
    cf_kib, _ = _counter_mean_kib(copy_fetch_dir, "FETCH_SIZE", copy_k)
    cw_kib, _ = _counter_mean_kib(copy_write_dir, "WRITE_SIZE", copy_k)
    copy_bytes = copy_mib << 20
    f_fac = cf_kib * 1024 / copy_bytes
    w_fac = cw_kib * 1024 / copy_bytes
    fetch = f_kib * 1024 / f_fac
    write = w_kib * 1024 / w_fac
    w = W.make_config(workload)
    nsplit = ta.num_splits(w.B, w.Hq, w.Hkv, w.D, w.max_tree, w.max_prefix, w.dtype)
    alg = work(w, nsplit)["kernel_bytes"]
    res = {"workload": workload, "kernel": kern, "kernel_src_sha256_16": kernel_hash(),
           "fetch_kib_per_launch_raw": f_kib, "write_kib_per_launch_raw": w_kib,
           "launches_fetch": nf, "launches_write": nw,
           "copy_fetch_factor": f_fac, "copy_write_factor": w_fac,
           "hbm_read_bytes_per_launch": fetch, "hbm_write_bytes_per_launch": write,
           "hbm_bytes_per_launch": fetch + write, "algorithmic_bytes_per_launch": alg,
           "traffic_over_algorithmic": (fetch + write) / alg}
    with open(out_path, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    print(json.dumps(res))


def time_calls(fn, reps: int, per_graph: int = 20) -> float:
    """Mean seconds per call of ``fn``: ``per_graph`` calls captured in one
    HIP graph, replayed back to back and timed with HIP events on the replay
    stream (so neither the Python launch path nor the host's graph-launch
    cost of a microsecond-scale kernel is in the figure)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # eager warm-up before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = capture(fn, per_graph)
    g.replay()
    torch.cuda.synchronize()
    n = max(1, reps // per_graph)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(200_000)   # the stream busy while the timed replays are enqueued
    e0.record()
    for _ in range(n):
        g.replay()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / 1e3 / (n * per_graph)


def measure_adjacent(dev) -> dict:
    """The steps next to the attention path, at the budget-256 (moe) shape:
    best-first draft-tree construction (32 requests, depth 16, 8 candidates
    per depth, budget 256) and the commit of accepted paths into the paged
    cache (32 requests, 4 kv heads, head_dim 128)."""
    rng = np.random.default_rng(2024)
    z = torch.from_numpy(rng.normal(0.0, 2.0, size=(32, 16, 8)))
    logp = torch.log_softmax(z, dim=-1).float().to(dev)
    t_tree = time_calls(lambda: ta.build_tree(logp, 256), 40, per_graph=10)
    parent, _, _ = ta.build_tree(logp, 256)
    trees = [t.numpy() for t in parent.cpu()]
    w = W.make_workload("moe-commit", [4096] * 32, trees, 32, 4, 128, torch.bfloat16, 1004,
                        reserve_tokens=16).to(dev)
    res = ta.plan(w.parent, w.tree_off, w.prefix_len, max_tree=256)
    acc_np = W.random_accepted(trees, np.random.default_rng(7), p_none=0.0)
    acc = torch.from_numpy(acc_np).to(dev)
    t_commit = time_calls(lambda: ta.commit(res.anc_mask, res.depth, w.tree_off, w.prefix_len, acc,
                                            w.k_tree, w.v_tree, w.k_cache, w.v_cache, w.block_table,
                                            max_tree=256), 400)
    depth = res.depth.cpu().numpy()
    off = w.tree_off.cpu().numpy()
    rows = int(sum(depth[off[b] + acc_np[b]] for b in range(32)))
    moved = rows * 4 * 128 * 2 * 2 * 2      # K and V rows, read once and written once
    log(f"[bench] draft tree (32 x budget 256): {t_tree * 1e6:.2f} us; commit of {rows} path rows: "
        f"{t_commit * 1e6:.2f} us ({moved / t_commit / 1e9:.1f} GB/s)")
    return {"draft_tree": {"us": t_tree * 1e6, "requests": 32, "budget": 256, "max_depth": 16,
                           "candidates": 8},
            "commit": {"us": t_commit * 1e6, "requests": 32, "path_rows": rows, "bytes": moved,
                       "GB/s": moved / t_commit / 1e9}}


def tree_blocks_visited(anc_mask: np.ndarray, tree_off: np.ndarray, G: int, rows_per_wg: int) -> int:
    """(row group, 64-key tree block) pairs with a visible key: a group of
    rows_per_wg query rows covers rows_per_wg / G consecutive nodes, and a
    workgroup holding those rows copies and computes a tree block when any
    of its nodes sees a key in it."""
    words = anc_mask.view(np.uint64)
    total = 0
    per = max(1, rows_per_wg // G)
    for b in range(len(tree_off) - 1):
        lo, hi = int(tree_off[b]), int(tree_off[b + 1])
        for s in range(lo, hi, per):
            total += int(np.count_nonzero(np.bitwise_or.reduce(words[s:min(s + per, hi)], axis=0)))
    return total


def measure_dfs(dev) -> dict:
    """Depth-first relabelling at budget 256 (tree256 and moe shapes): the
    attention call on best-first labels against the same call on the
    relabelled tree (inputs gathered once, outside the timing), with the
    tree blocks each visits, and the cost of tree_attn_plan_dfs itself
    against tree_attn_plan.  Same inputs call after call (warm caches): a
    relative figure."""
    out = {}
    for name in ("tree256", "moe"):
        w_host = W.make_config(name)
        mt, mp = w_host.max_tree, w_host.max_prefix
        w = w_host.to(dev)
        res = ta.plan(w.parent, w.tree_off, w.prefix_len, max_tree=mt)
        r = ta.plan_dfs(w.parent, w.tree_off, w.prefix_len, max_tree=mt)
        ta.check_status(res.status)
        ta.check_status(r.plan.status)
        q, kt, vt = (ta.gather_rows(t, r.perm) for t in (w.q, w.k_tree, w.v_tree))
        call_a = ta.prepare_fwd(w.q, w.k_tree, w.v_tree, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                w.tree_off, res.anc_mask, max_tree=mt, max_prefix=mp)
        call_b = ta.prepare_fwd(q, kt, vt, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                w.tree_off, r.plan.anc_mask, max_tree=mt, max_prefix=mp)
        reps, per = (100, 20) if name == "tree256" else (48, 4)
        # the first pass brings the clocks up (the first call timed was
        # otherwise several per cent slow); the second pass is kept
        for _ in range(2):
            t_a = time_calls(call_a.run, reps, per_graph=per)
            t_b = time_calls(call_b.run, reps, per_graph=per)
        t_plan = time_calls(lambda: ta.plan(w.parent, w.tree_off, w.prefix_len, max_tree=mt,
                                            out=res), 200)
        t_dfs = time_calls(lambda: ta.plan_dfs(w.parent, w.tree_off, w.prefix_len, max_tree=mt), 200)
        torch.cuda.synchronize()
        off = w.tree_off.cpu().numpy()
        G = w.Hq // w.Hkv
        geo = ta.num_splits(w.B, w.Hq, w.Hkv, w.D, mt, mp)
        rows_wg = 128        # counted per 128 query rows (4 row tiles of 32)
        vis_a = tree_blocks_visited(res.anc_mask.cpu().numpy(), off, G, rows_wg)
        vis_b = tree_blocks_visited(r.plan.anc_mask.cpu().numpy(), off, G, rows_wg)
        log(f"[bench] {name} attention: best-first labels {t_a * 1e6:.2f} us ({vis_a} tree blocks), "
            f"depth-first {t_b * 1e6:.2f} us ({vis_b}); plan {t_plan * 1e6:.2f} us, "
            f"plan_dfs {t_dfs * 1e6:.2f} us (splits {geo})")
        out[name] = {"attn_us_best_first": t_a * 1e6, "attn_us_depth_first": t_b * 1e6,
                     "tree_blocks_best_first": vis_a, "tree_blocks_depth_first": vis_b,
                     "plan_us": t_plan * 1e6, "plan_dfs_us": t_dfs * 1e6}
        del w, w_host, q, kt, vt, call_a, call_b
        torch.cuda.empty_cache()
    return out


def calibrate_copy(mib: int, reps: int):
    """A plain device copy of known size, for scaling HBM byte counters."""
    dev = torch.device("cuda:0")
    n = (mib << 20) // 4
    a = torch.randn(n, device=dev)
    b = torch.empty_like(a)
    for _ in range(reps):
        torch.add(a, 0.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": reps}))


SUB_KEYS = ("value", "unit", "ms_per_step", "wall_ms_per_step", "steps", "warmup", "tflops",
            "num_splits", "config", "roofline", "roofline_hbm", "cpu_baseline", "fwd_only",
            "plan_only", "two_call")


def sub_line(res: dict) -> dict:
    out = {"workload": res["workload"], "unit": "tree tokens/s"}
    out.update({k: res[k] for k in SUB_KEYS if k in res})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="chain16", choices=[n for n in W.CONFIG_NAMES])
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other bf16 workloads (moe, tree256, mixed) and the adjacent steps")
    ap.add_argument("--no-adjacent", action="store_true",
                    help="skip the adjacent steps (tree construction, commit, depth-first relabelling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the two-call, plan-only and forward-only timings (profiling runs)")
    ap.add_argument("--sustain-seconds", type=float, default=8.0,
                    help="GPU seconds of back-to-back steps after the timed ones, reported as "
                         "'sustained' (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget of the headline workload (the others get half)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain copy kernel of this many MiB (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                    "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/fwd_bf16_kernel_<workload>_traffic.json from rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE passes of this workload and of the copy "
                         "(--calibrate-copy-mib gives the copy size, default 256); no GPU needed")
    args = ap.parse_args()

    if args.summarize_traffic:
        out = os.path.join(PROFILES, f"fwd_bf16_kernel_{args.workload}_traffic.json")
        summarize_traffic(args.workload, *args.summarize_traffic, args.calibrate_copy_mib or 256, out)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the attention shards by request or by kv head with no exchange between GPUs, so "
              f"N GPUs run N independent copies of this measurement)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib, 10)
        return
    ta.load_library()
    dev = torch.device("cuda:0")
    cpu = not args.no_cpu_baseline
    compare = not args.no_compare
    main_res = measure(args.workload, args.steps, args.warmup, dev, cpu, args.cpu_seconds, compare,
                       args.sustain_seconds)
    w_dtype = "f32" if args.workload == "tiny" else "bf16"
    line = {
        "metric": METRIC,
        "value": main_res["value"],
        "unit": "tree tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w_dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, shuffled page pool, synthetic trees)",
        "config": main_res["config"],
        "roofline": main_res["roofline"],
    }
    if "cpu_baseline" in main_res:
        line["cpu_baseline"] = main_res["cpu_baseline"]
    line["value_definition"] = ("tree tokens (N) per second of GPU time over the timed steps; a step is "
                                "one tree_attn_plan_fwd call (plan, paged prefix, masked tree and split "
                                "merge), timed with HIP events on the replay stream")
    for k in ("wall_ms_per_step", "tflops", "kernel_us", "fwd_only", "plan_only", "two_call"):
        line[k] = main_res[k]
    if "sustained" in main_res:
        line["sustained"] = main_res["sustained"]
    if not args.no_secondary:
        # steps per workload: about the same GPU time as the headline's at
        # the default --steps; at least 20
        plan_steps = {"moe": max(20, args.steps // 10), "tree256": args.steps,
                      "mixed": max(20, args.steps // 5)}
        for name, key in (("moe", "budget256"), ("tree256", "tree256"), ("mixed", "mixed")):
            if name == args.workload:
                continue
            sec = measure(name, plan_steps[name], args.warmup, dev, cpu, args.cpu_seconds / 2, compare)
            line[key] = sub_line(sec)
    if not args.no_secondary and not args.no_adjacent:
        line["adjacent"] = measure_adjacent(dev)
        line["adjacent"]["depth_first_relabel"] = measure_dfs(dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
