#!/usr/bin/env python3
"""Benchmark: one CP4 rank's share of a 16,384-token packed budget on one MI355X.

A step is one pass of the whole per-rank hot path on the share's inputs (already
resident in HBM): one cpattn_fwd_chunks call, i.e. its work plan written into the
caller's workspace (by the library's planner kernel when the metadata is small, as for
every workload here; else built on the host and copied) and ONE attention launch that
walks every KV chunk of the share with the online softmax carried across chunks (the
ring loop's merges done in registers).  `value`
is the share's algorithmic causal FLOPs (4 * D * Hq per visible query/key pair)
divided by the step time.  The two other schedules of the same share -- per-chunk
launches accumulating in the epilogue (cpattn_fwd_chunk_accum), and per-chunk
partials merged by cpattn_merge -- are timed the same way under "schedules".
Further seeds of the CP4 share (other packs of the same shapes) are timed like the
step under "seeds", with the aggregate over all of them.

The other workloads (the 128K-context CP=4 share, the 4,096-token pack without
chunking and the Dynamic-CP mixed pack) are timed the same way in the same run and
reported under "workloads": a step is one cpattn_fwd_chunks launch per group of
the workload (the mixed pack has one group per CP size), with step time,
TFLOP/s, fraction of the bf16 MFMA peak and processed tokens.

The CPU baseline (the fp64 oracle on a bounded row sample of the CP4 share, in a
process pool over (row block, kv head) tasks) runs first, before the GPU is
initialised, so the forked workers never inherit a GPU context.

Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload cp4_share] [--seed 0]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "causal attn TFLOP/s + MFMA util%, 16K-token THD pack at CP4-share, 1 GPU"
BF16_PEAK_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
ATTN_SOURCE = os.path.join(HERE, "context_ring_attention_amd", "csrc", "attn_fwd_bf16.hip")
# HBM bytes per streaming attention launch, from rocprofv3 FETCH_SIZE and WRITE_SIZE runs
# (scaled by a plain-copy calibration), keyed by workload and the sha256 of the kernel source
# they were taken on.  Any other pair reports traffic as null until it is profiled again.
PROFILED_TRAFFIC = {
    ("cp4_share", "c884679021d39153783aaa25e0a2ceb2fdf2de8e8b23c4291b1b4e3189946f05"): 222803125,
    ("ctx128k_share", "c884679021d39153783aaa25e0a2ceb2fdf2de8e8b23c4291b1b4e3189946f05"): 3931767285,
}
# A pool for the CPU baseline never exceeds one GPU's share of the host's cores.
MAX_CPU_WORKERS = 16


def visible_pairs(cu_q, cu_k, q_off, k_off) -> int:
    """Visible (query, key) pairs per head under the causal mask, closed form per sequence."""
    total = 0
    for i in range(len(cu_q) - 1):
        nq = int(cu_q[i + 1] - cu_q[i]); nk = int(cu_k[i + 1] - cu_k[i])
        d0 = int(q_off[i]) - int(k_off[i])
        for_rows = np.clip(d0 + 1 + np.arange(nq, dtype=np.int64), 0, nk)
        total += int(for_rows.sum())
    return total


def pack_words(lengths) -> str:
    """'one 131,072-token sequence' or 'a 16,384-token THD pack of 2 sequences'."""
    total = int(sum(lengths))
    if len(lengths) == 1:
        return f"one {total:,}-token sequence"
    return f"a {total:,}-token THD pack of {len(lengths)} sequences"


def describe(w) -> str:
    """Text of a workload: what it is, with its sizes."""
    if w.name == "dcp_mixed":
        cps = [len(g.chunks) for g in w.groups]
        return (f"dcp_mixed (seed {w.seed}): {pack_words(w.lengths)}, lognormal lengths, "
                f"{len(w.groups)} groups by CP size {cps}, each sample's KV in cp chunks, "
                f"{w.hq}/{w.hkv} heads, D={w.d}, causal")
    g = w.groups[0]
    nch = len(g.chunks)
    tq = int(g.cu_q[-1])
    if nch == 1:
        return (f"{w.name} (seed {w.seed}): {pack_words(w.lengths)}, no chunking, "
                f"{w.hq}/{w.hkv} heads, D={w.d}, causal")
    return (f"{w.name} (seed {w.seed}): last CP{nch} rank of {pack_words(w.lengths)}, local Q "
            f"{tq} tokens in {len(g.cu_q) - 1} sequences, {nch} KV chunks of "
            f"{int(g.chunks[0].cu_k[-1])} tokens, {w.hq}/{w.hkv} heads, D={w.d}, causal")


# ---------------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample, in a process pool.

_POOL_DATA = {}


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:   # pragma: no cover - threadpoolctl missing: BLAS keeps its default
        pass


def _pool_task(task):
    """One (row block, kv head) task: the oracle's attention for those rows and the query
    heads of that kv head (their GQA group), against every visible key of the share."""
    from oracle import attention_ref
    rows, kvh = task
    g = _POOL_DATA["group"]
    hq, hkv = _POOL_DATA["hq"], _POOL_DATA["hkv"]
    grp = hq // hkv
    heads = slice(kvh * grp, (kvh + 1) * grp)
    nseq = len(g.cu_q) - 1
    attention_ref(g.q[:, heads], g.k_full[:, kvh:kvh + 1], g.v_full[:, kvh:kvh + 1], g.cu_q,
                  g.cu_full, g.q_off, np.zeros(nseq, np.int64), causal=True, rows=rows)
    return len(rows)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_rows: int = 4096, block_rows: int = 256):
    """Time the fp64 oracle on a row sample of the share, over a fork-based process pool."""
    import multiprocessing as mp
    g = w.groups[0]
    workers = max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))
    rng = np.random.default_rng(1234)
    tq = int(g.cu_q[-1])
    rows = np.sort(rng.choice(tq, size=min(budget_rows, tq), replace=False))
    seq = np.searchsorted(g.cu_q, rows, side="right") - 1
    pairs = 0
    for r, i in zip(rows, seq):
        pos = int(g.q_off[i]) + int(r - g.cu_q[i])
        pairs += min(pos + 1, int(g.cu_full[i + 1] - g.cu_full[i]))
    tasks = [(rows[b:b + block_rows], kvh) for b in range(0, len(rows), block_rows)
             for kvh in range(w.hkv)]
    _POOL_DATA.update(group=g, hq=w.hq, hkv=w.hkv)
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_pool_init) as pool:
        done = sum(pool.map(_pool_task, tasks, chunksize=1))
    dt = time.perf_counter() - t0
    assert done == len(rows) * w.hkv
    flops = 4 * w.d * w.hq * pairs
    return {"value": float(f"{flops / dt / 1e12:.4g}"), "unit": "TFLOP/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{len(rows)} random query rows of the {w.name} share (seed {w.seed}) x all "
                      f"{w.hq} heads against all their visible keys: fp64 numpy, {len(tasks)} "
                      f"(row block, kv head) tasks on {workers} worker processes with one BLAS "
                      f"thread each, {dt:.1f} s, {flops / 1e9:.1f} GFLOP",
            "cpu_model": cpu_model()}


# ---------------------------------------------------------------------------------------------
# GPU timing helpers.

class LaunchChain:
    """Durations of the launches of the timed steps from ONE event recorded after each launch
    (and one at the start): a launch's duration is the time from the previous event to its own.
    Each event is a marker the GPU stops at; a pair of events around every launch would put two
    markers between consecutive launches, which idled the GPU ~10 us per step (kernel traces).
    Consecutive differences tile the timed region, so they sum to the measured step time."""

    def __init__(self, ev, n: int):
        self.pool = [ev() for _ in range(n)]
        self.marks = []

    def mark(self, label, stream):
        e = self.pool[len(self.marks)]
        e.record(stream)
        self.marks.append((label, e))

    def durations_ms(self, label):
        return [a.elapsed_time(b) for (_, a), (lb, b) in zip(self.marks, self.marks[1:]) if lb == label]


def timed_steps(step, steps: int, warmup: int, stream, ev):
    """Run `step` warmup times, then time exactly `steps` of them between two events on the
    stream (with the garbage collector frozen: a full collection mid-step idles the GPU)."""
    import torch
    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    gc.collect()
    gc.freeze()
    gc.disable()
    try:
        t_start, t_end = ev(), ev()
        t_start.record(stream)
        for i in range(steps):
            step(i)
        t_end.record(stream)
        torch.cuda.synchronize()
    finally:
        gc.enable()
        gc.unfreeze()
    return t_start.elapsed_time(t_end) / steps


class GpuGroup:
    """Device copies and host metadata of one group (a Q pack and its KV chunks)."""

    def __init__(self, w, g):
        import torch
        import context_ring_attention_amd as cra
        bf = torch.bfloat16
        self.q = torch.from_numpy(g.q).to("cuda", bf)
        self.ks = [torch.from_numpy(c.k).to("cuda", bf) for c in g.chunks]
        self.vs = [torch.from_numpy(c.v).to("cuda", bf) for c in g.chunks]
        self.cu_q = np.ascontiguousarray(g.cu_q, np.int32)
        self.q_off = np.ascontiguousarray(g.q_off, np.int32)
        self.cu_ks = [np.ascontiguousarray(c.cu_k, np.int32) for c in g.chunks]
        self.k_offs = [np.ascontiguousarray(c.k_off, np.int32) for c in g.chunks]
        self.nch = len(g.chunks)
        self.bufs = cra.ShareBuffers.allocate(self.q, w.hkv, self.cu_q, self.nch)
        self.pairs_chunk = [visible_pairs(self.cu_q, c.cu_k, self.q_off, c.k_off) for c in g.chunks]
        self.flops = sum(4 * w.d * w.hq * p for p in self.pairs_chunk)
        self.tq = int(self.cu_q[-1])
        self.tk = sum(int(c[-1]) for c in self.cu_ks)
        self.alg_bytes = (self.tq * w.hq * w.d * 2 + 2 * self.tk * w.hkv * w.d * 2
                          + self.tq * w.hq * w.d * 4 + self.tq * w.hq * 4)

    def fwd(self, stream):
        import context_ring_attention_amd as cra
        cra.cpattn_fwd_chunks(self.q, self.ks, self.vs, self.cu_q, self.cu_ks, self.q_off,
                              self.k_offs, True, out=self.bufs.o_acc, lse=self.bufs.lse_acc,
                              workspace=self.bufs.workspace, stream=stream)


def time_backward(w, gg, steps, warmup, stream, ev, seed):
    """The share's backward in one pass (cpattn_bwd_chunks) from its forward output."""
    import torch
    import context_ring_attention_amd as cra
    gg.fwd(stream)
    gen = torch.Generator(device="cuda").manual_seed(seed + 1)
    dout = torch.randn(gg.q.shape, device="cuda", generator=gen).to(torch.bfloat16)
    f32 = dict(dtype=torch.float32, device="cuda")
    dq = torch.zeros(gg.q.shape, **f32)
    dks = [torch.zeros(k.shape, **f32) for k in gg.ks]
    dvs = [torch.zeros(v.shape, **f32) for v in gg.vs]
    bws = torch.empty(max(cra.cpattn_bwd_workspace_size_chunks(len(gg.cu_q) - 1, gg.cu_q, gg.cu_ks,
                                                               w.hq, w.hkv, w.d), 256),
                      dtype=torch.uint8, device="cuda")

    def step(_):
        cra.cpattn_bwd_chunks(gg.q, gg.ks, gg.vs, gg.bufs.o_acc, gg.bufs.lse_acc, dout, gg.cu_q,
                              gg.cu_ks, gg.q_off, gg.k_offs, True, dq=dq, dks=dks, dvs=dvs,
                              workspace=bws, stream=stream)

    ms = timed_steps(step, steps, max(1, warmup), stream, ev)
    flops = 10 * w.d * w.hq * sum(gg.pairs_chunk)
    del dq, dks, dvs, bws, dout
    return {"ms_per_step": round(ms, 4), "tflops": round(flops / (ms / 1e3) / 1e12, 2),
            "frac": round(flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "flops_per_step": flops,
            "counted_as": "10 D Hq per visible pair (5 products of the forward's 2 D Hq)",
            "launches_per_step": "delta, then one gradient launch (dQ and dK/dV work-groups over all chunks)"}


def stored_traffic(workload: str):
    with open(ATTN_SOURCE, "rb") as f:
        return PROFILED_TRAFFIC.get((workload, hashlib.sha256(f.read()).hexdigest()))


def time_workload(name, seed, steps, warmup, stream, ev, backward: bool):
    """A step = one cpattn_fwd_chunks launch per group; returns the workload's report."""
    import workloads as wl
    w = wl.make(name, seed)
    gs = [GpuGroup(w, g) for g in w.groups]
    chain = LaunchChain(ev, 1 + steps * len(gs))

    def step(i):
        if i is not False and i == 0:
            chain.mark("start", stream)
        for j, gg in enumerate(gs):
            gg.fwd(stream)
            if i is not False:
                chain.mark(j, stream)

    ms = timed_steps(step, steps, warmup, stream, ev)
    flops = sum(gg.flops for gg in gs)
    launch_ms = [sum(chain.durations_ms(j)) / steps for j in range(len(gs))]
    kern_ms = sum(launch_ms)
    tq = sum(gg.tq for gg in gs)
    tk = sum(gg.tk for gg in gs)
    rep = {"config": describe(w),
           "ms_per_step": round(ms, 4),
           "tflops": round(flops / (ms / 1e3) / 1e12, 2),
           "frac": round(flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "attn_launches_per_step": len(gs),
           "attn_avg_launch_us": [round(x * 1e3, 2) for x in launch_ms],
           "roofline": {"bound": "mfma", "achieved": round(flops / (kern_ms / 1e3) / 1e12, 2),
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(flops / (kern_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                        "traffic": stored_traffic(name) if len(gs) == 1 else None,
                        "algorithmic_bytes_per_step": sum(gg.alg_bytes for gg in gs)},
           "flops_per_step": flops,
           "tokens_per_step": {"query": tq, "key": tk},
           "query_tokens_per_s": round(tq / (ms / 1e3), 1)}
    if backward and len(gs) == 1:
        rep["backward"] = time_backward(w, gs[0], steps, warmup, stream, ev, seed)
    del gs
    return rep


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cp4_share")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedules", default="merge,accum,stream",
                    help="comma-separated schedules to time besides the step itself (stream is "
                         "always timed, last)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward of the shares (reported under 'backward')")
    ap.add_argument("--sweep-seeds", default=None,
                    help="comma-separated further seeds of the workload whose step is timed the same "
                         "way (reported under 'seeds'; default 1,2,3,4 for cp4_share, none otherwise)")
    ap.add_argument("--other-workloads", default="ctx128k_share,pack,dcp_mixed",
                    help="comma-separated workloads timed after the main one, reported under "
                         "'workloads' (empty for none)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run one plain elementwise copy of MIB MiB "
                         "(reference point for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}): this build has no "
              "multi-GPU path; each rank's share is what one GPU computes.", file=sys.stderr)
        return 2

    import workloads as wl
    w = wl.make(args.workload, args.seed)
    if len(w.groups) != 1 or w.dtype != "bf16":
        print("the main workload must be a single-group bf16 share (the others go under "
              "--other-workloads)", file=sys.stderr)
        return 2
    g = w.groups[0]

    # The CPU baseline first: its fork-based pool must start before anything touches the GPU.
    cb = None
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w)

    import torch
    import context_ring_attention_amd as cra

    cra.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    gg = GpuGroup(w, g)
    q, ks, vs, bufs = gg.q, gg.ks, gg.vs, gg.bufs
    cu_q, q_off, cu_ks, k_offs, nch = gg.cu_q, gg.q_off, gg.cu_ks, gg.k_offs, gg.nch
    flops_step = gg.flops
    tq = gg.tq
    merge_bytes = 3 * (tq * w.hq * w.d * 4 + tq * w.hq * 4)
    n_merge = nch - 1

    chains = {m: LaunchChain(ev, 1 + args.steps * (nch + n_merge)) for m in cra.MODES}

    def share_step(mode, i):
        """One step of `mode`; i is the timed step's index, or False during warm-up."""
        ch = chains[mode] if i is not False else None
        if ch and i == 0:
            ch.mark("start", stream)
        if mode == "stream":
            gg.fwd(stream)
            if ch:
                ch.mark("attn", stream)
            return
        for c in range(nch):
            first = c == 0
            out, lse = ((bufs.o_acc, bufs.lse_acc) if first or mode == "accum"
                        else (bufs.o_part, bufs.lse_part))
            fn = cra.cpattn_fwd_chunk if first or mode == "merge" else cra.cpattn_fwd_chunk_accum
            fn(q, ks[c], vs[c], cu_q, cu_ks[c], q_off, k_offs[c], True, out=out, lse=lse,
               workspace=bufs.workspace, stream=stream)
            if ch:
                ch.mark("attn", stream)
            if mode == "merge" and not first:
                cra.cpattn_merge(bufs.o_acc, bufs.lse_acc, bufs.o_part, bufs.lse_part, stream=stream)
                if ch:
                    ch.mark("merge", stream)

    wanted = [m for m in args.schedules.split(",") if m]
    if any(m not in cra.MODES for m in wanted):
        print(f"--schedules takes names from {cra.MODES}", file=sys.stderr)
        return 2
    order = [m for m in ("merge", "accum") if m in wanted] + ["stream"]
    schedules = {}
    for mode in order:   # the step's own schedule last, on a warm GPU
        ms = timed_steps(lambda i, m=mode: share_step(m, i), args.steps, args.warmup, stream, ev)
        launches = 1 if mode == "stream" else nch
        a_d = chains[mode].durations_ms("attn")
        a_ms = sum(a_d) / len(a_d)
        schedules[mode] = {"ms_per_step": round(ms, 4),
                           "tflops": round(flops_step / (ms / 1e3) / 1e12, 2),
                           "attn_launches_per_step": launches,
                           "attn_avg_launch_us": round(a_ms * 1e3, 2)}
    ms_step = schedules["stream"]["ms_per_step"]
    value = flops_step / (ms_step / 1e3) / 1e12
    attn_avg_ms = schedules["stream"]["attn_avg_launch_us"] / 1e3
    attn_tflops = flops_step / (attn_avg_ms / 1e3) / 1e12

    timed_merge = "merge" in schedules and n_merge > 0
    m_d = chains["merge"].durations_ms("merge") if timed_merge else []
    merge_avg_ms = sum(m_d) / max(1, len(m_d))
    merge_gbs = merge_bytes / (merge_avg_ms / 1e3) / 1e9 if timed_merge else None
    # Reference for the merge's HBM roof: torch's elementwise add over buffers of O's size (two
    # reads and one write, the merge's traffic without the LSE rows), timed the same way.
    add_gbs = None
    if timed_merge:
        xa, xb = bufs.o_acc, bufs.o_part
        xc = torch.empty_like(xa)
        add_ms = timed_steps(lambda i: torch.add(xa, xb, out=xc), 20, 3, stream, ev)
        add_gbs = 3 * xa.numel() * 4 / (add_ms / 1e3) / 1e9
        del xc

    backward = None if args.no_backward else time_backward(w, gg, args.steps, args.warmup, stream,
                                                           ev, args.seed)

    # Other packs of the same workload (further seeds: same shapes, other sequence lengths), the
    # step timed the same way, and the aggregate over all of them (total FLOPs / total time).
    sweep = args.sweep_seeds if args.sweep_seeds is not None else (
        "1,2,3,4" if args.workload == "cp4_share" else "")
    seeds = None
    sweep_list = [int(x) for x in sweep.split(",") if x.strip() and int(x) != w.seed]
    if sweep_list:
        per_seed = [{"seed": w.seed, "pieces": [int(x) for x in np.diff(cu_q)],
                     "ms_per_step": round(ms_step, 4), "tflops": round(value, 2)}]
        tot_flops, tot_ms = flops_step, ms_step
        for sd in sweep_list:
            w2 = wl.make(args.workload, sd)
            g2 = GpuGroup(w2, w2.groups[0])
            ms2 = timed_steps(lambda i: g2.fwd(stream), args.steps, args.warmup, stream, ev)
            per_seed.append({"seed": sd, "pieces": [int(x) for x in np.diff(g2.cu_q)],
                             "ms_per_step": round(ms2, 4),
                             "tflops": round(g2.flops / (ms2 / 1e3) / 1e12, 2)})
            tot_flops += g2.flops
            tot_ms += ms2
            del g2
        seeds = {"per_seed": per_seed,
                 "aggregate_tflops": round(tot_flops / (tot_ms / 1e3) / 1e12, 2),
                 "aggregate_frac": round(tot_flops / (tot_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    others = {}
    for name in [x for x in args.other_workloads.split(",") if x.strip()]:
        others[name] = time_workload(name, args.seed, args.steps, args.warmup, stream, ev,
                                     backward=not args.no_backward and name == "ctx128k_share")
        torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(w),
                   "global_batch": int(sum(w.lengths)), "seq_len": int(max(w.lengths)),
                   "parallelism": f"cp{nch}-share"},
        "mfma_util": round(value / BF16_PEAK_TFLOPS, 4),
        "tokens_per_step": {"query": tq, "key": gg.tk},
        "query_tokens_per_s": round(tq / (ms_step / 1e3), 1),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic(args.workload),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE x1)",
                     "algorithmic_bytes_per_launch": gg.alg_bytes,
                     "kernel": "attn_fwd_bf16_kernel<128,false> over all chunks (event-timed per "
                               "cpattn_fwd_chunks call, its plan kernel included)",
                     "avg_launch_us": round(attn_avg_ms * 1e3, 2),
                     "flops_per_launch": flops_step},
        "schedules": schedules,
        "seeds": seeds,
        "backward": backward,
        "workloads": others,
        "merge": {"schedule": "merge", "avg_launch_us": round(merge_avg_ms * 1e3, 2) if timed_merge else None,
                  "bytes_per_launch": merge_bytes, "achieved_GBs": round(merge_gbs, 1) if merge_gbs else None,
                  "hbm_frac": round(merge_gbs / HBM_PEAK_GBS, 4) if merge_gbs else None,
                  "torch_add_same_bytes_GBs": round(add_gbs, 1) if add_gbs else None},
        "flops_per_step": flops_step,
        "cpu_baseline": cb,
    }
    if args.copy_calibration:
        # A plain elementwise copy of known size whose source is not cache-resident:
        # fill the source, stream 2 GiB through the caches, then copy.
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        evict = torch.empty(2 << 28, dtype=torch.float32, device="cuda")
        evict.fill_(2.0)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del evict
        result["copy_calibration_bytes"] = {"read": n * 4, "written": n * 4}
    # The Dynamic-CP host scheduler on the Dynamic-CP mini-batch (65,536 tokens, lognormal
    # lengths) for DP x CP = 8 ranks under the CP4 per-rank limit of 4,096 tokens.
    dcp_lens = wl.lengths_for("dcp_mixed", args.seed)
    reps = 200
    t0 = time.perf_counter()
    for _ in range(reps):
        sched = cra.cpattn_dcp_schedule(dcp_lens, 8, 4096)
    dcp_us = (time.perf_counter() - t0) / reps * 1e6
    result["dcp_schedule"] = {"samples": len(dcp_lens), "tokens": int(sum(dcp_lens)), "world": 8,
                              "max_seqlen_per_rank": 4096, "micro_batches": sched["n_micro_batches"],
                              "host_us_per_call": round(dcp_us, 1)}
    if not args.no_cpu_baseline:
        from oracle.dcp import dcp_schedule_ref
        t0 = time.perf_counter()
        for _ in range(20):
            dcp_schedule_ref(dcp_lens, 8, 4096)
        result["dcp_schedule"]["oracle_host_us_per_call"] = round((time.perf_counter() - t0) / 20 * 1e6, 1)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
