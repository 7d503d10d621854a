#!/usr/bin/env python3
"""Benchmark: one CP4 rank's share of a 16,384-token packed budget on one MI355X.

A step is one pass of the whole per-rank hot path on the share's inputs (already
resident in HBM): host planning (into pinned memory the kernel reads) and ONE cpattn_fwd_chunks launch that
walks every KV chunk of the share with the online softmax carried across chunks
(the ring loop's merges done in registers).  `value` is the share's algorithmic
causal FLOPs (4 * D * Hq per visible query/key pair) divided by the step time.
The two other schedules of the same share -- per-chunk launches accumulating in
the epilogue (cpattn_fwd_chunk_accum), and per-chunk partials merged by
cpattn_merge -- are timed the same way and reported under "schedules".  Further seeds of the
CP4 share (other packs of the same shapes) are timed like the step and reported under "seeds",
with the aggregate over all of them (total FLOPs / total time).
Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload cp4_share] [--seed 0]
"""
from __future__ import annotations

import argparse
import gc
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
    ("cp4_share", "d10ef45935ad77971220ad11ea0fddab51b8812736092d9dafd710da2197323a"): 223394549,
    ("ctx128k_share", "d10ef45935ad77971220ad11ea0fddab51b8812736092d9dafd710da2197323a"): 2939329515,
}


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


def cpu_baseline(w, g, budget_rows: int = 4096):
    """Time the fp64 oracle on (a bounded row sample of) the same share, on the host CPU."""
    from oracle import share_ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:   # pragma: no cover - threadpoolctl missing
        threads = 1
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(int(g.cu_q[-1]), size=min(budget_rows, int(g.cu_q[-1])), replace=False))
    seq = np.searchsorted(g.cu_q, rows, side="right") - 1
    pairs = 0
    for r, i in zip(rows, seq):
        pos = int(g.q_off[i]) + int(r - g.cu_q[i])
        pairs += min(pos + 1, int(g.cu_full[i + 1] - g.cu_full[i]))
    t0 = time.perf_counter()
    share_ref(g, rows=rows)
    dt = time.perf_counter() - t0
    flops = 4 * w.d * w.hq * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(rows)} random query rows of the share x all {w.hq} heads against all "
                      f"their visible keys (fp64 numpy, {dt:.1f} s, {flops / 1e9:.1f} GFLOP)",
            "seconds": dt}


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
                    help="skip timing the backward of the share (reported under 'backward')")
    ap.add_argument("--sweep-seeds", default=None,
                    help="comma-separated further seeds of the workload whose step is timed the same "
                         "way (reported under 'seeds'; default 1,2,3,4 for cp4_share, none otherwise)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run one plain elementwise copy of MIB MiB "
                         "(reference point for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}): this build has no "
              "multi-GPU path; each rank's share is what one GPU computes.", file=sys.stderr)
        return 2

    import torch
    import workloads as wl
    import context_ring_attention_amd as cra

    cra.load()
    torch.cuda.set_device(0)
    w = wl.make(args.workload, args.seed)
    if len(w.groups) != 1 or w.dtype != "bf16":
        print("bench.py times single-group bf16 share workloads", file=sys.stderr)
        return 2
    g = w.groups[0]
    bf = torch.bfloat16
    q = torch.from_numpy(g.q).to("cuda", bf)
    ks = [torch.from_numpy(c.k).to("cuda", bf) for c in g.chunks]
    vs = [torch.from_numpy(c.v).to("cuda", bf) for c in g.chunks]
    cu_q = np.ascontiguousarray(g.cu_q, np.int32)
    q_off = np.ascontiguousarray(g.q_off, np.int32)
    cu_ks = [np.ascontiguousarray(c.cu_k, np.int32) for c in g.chunks]
    k_offs = [np.ascontiguousarray(c.k_off, np.int32) for c in g.chunks]
    nch = len(g.chunks)
    bufs = cra.ShareBuffers.allocate(q, w.hkv, cu_q, nch)
    stream = torch.cuda.current_stream()

    pairs_chunk = [visible_pairs(cu_q, c.cu_k, q_off, c.k_off) for c in g.chunks]
    flops_chunk = [4 * w.d * w.hq * p for p in pairs_chunk]
    flops_step = sum(flops_chunk)
    tq = int(cu_q[-1])
    merge_bytes = 3 * (tq * w.hq * w.d * 4 + tq * w.hq * 4)
    n_merge = nch - 1

    ev = lambda: torch.cuda.Event(enable_timing=True)
    attn_ev = {m: [[(ev(), ev()) for _ in g.chunks] for _ in range(args.steps)] for m in cra.MODES}
    merge_ev = [[(ev(), ev()) for _ in range(n_merge)] for _ in range(args.steps)]

    spare_attn = [(ev(), ev()) for _ in g.chunks]        # recorded during warm-up, unread
    spare_merge = [(ev(), ev()) for _ in range(n_merge)]

    def step(mode, a_ev, m_ev):
        if mode == "stream":
            a_ev[0][0].record(stream)
            cra.cpattn_fwd_chunks(q, ks, vs, cu_q, cu_ks, q_off, k_offs, True, out=bufs.o_acc,
                                  lse=bufs.lse_acc, workspace=bufs.workspace, stream=stream)
            a_ev[0][1].record(stream)
            return
        for c in range(nch):
            first = c == 0
            out, lse = ((bufs.o_acc, bufs.lse_acc) if first or mode == "accum"
                        else (bufs.o_part, bufs.lse_part))
            fn = cra.cpattn_fwd_chunk if first or mode == "merge" else cra.cpattn_fwd_chunk_accum
            a_ev[c][0].record(stream)
            fn(q, ks[c], vs[c], cu_q, cu_ks[c], q_off, k_offs[c], True, out=out, lse=lse,
               workspace=bufs.workspace, stream=stream)
            a_ev[c][1].record(stream)
            if mode == "merge" and not first:
                m_ev[c - 1][0].record(stream)
                cra.cpattn_merge(bufs.o_acc, bufs.lse_acc, bufs.o_part, bufs.lse_part, stream=stream)
                m_ev[c - 1][1].record(stream)

    def timed(mode):
        for _ in range(args.warmup):
            step(mode, spare_attn, spare_merge)
        torch.cuda.synchronize()
        # A full collection of the interpreter's heap takes tens of ms and would leave the GPU
        # idle mid-step: collect now, freeze what exists, and keep the collector off while timing.
        gc.collect()
        gc.freeze()
        gc.disable()
        try:
            t_start, t_end = ev(), ev()
            t_start.record(stream)
            for i in range(args.steps):
                step(mode, attn_ev[mode][i], merge_ev[i])
            t_end.record(stream)
            torch.cuda.synchronize()
        finally:
            gc.enable()
            gc.unfreeze()
        return t_start.elapsed_time(t_end) / args.steps

    wanted = [m for m in args.schedules.split(",") if m]
    if any(m not in cra.MODES for m in wanted):
        print(f"--schedules takes names from {cra.MODES}", file=sys.stderr)
        return 2
    order = [m for m in ("merge", "accum") if m in wanted] + ["stream"]
    schedules = {}
    for mode in order:   # the step's own schedule last, on a warm GPU
        ms = timed(mode)
        launches = 1 if mode == "stream" else nch
        a_ms = sum(row[c][0].elapsed_time(row[c][1]) for row in attn_ev[mode]
                   for c in range(launches)) / (args.steps * launches)
        schedules[mode] = {"ms_per_step": round(ms, 4),
                           "tflops": round(flops_step / (ms / 1e3) / 1e12, 2),
                           "attn_launches_per_step": launches,
                           "attn_avg_launch_us": round(a_ms * 1e3, 2)}
    ms_step = schedules["stream"]["ms_per_step"]
    value = flops_step / (ms_step / 1e3) / 1e12

    attn_avg_ms = schedules["stream"]["attn_avg_launch_us"] / 1e3
    attn_flops_per_launch = flops_step
    attn_tflops = attn_flops_per_launch / (attn_avg_ms / 1e3) / 1e12
    timed_merge = "merge" in schedules and n_merge > 0
    merge_ms = sum(a.elapsed_time(b) for row in merge_ev for a, b in row) if timed_merge else 0.0
    merge_avg_ms = merge_ms / max(1, args.steps * n_merge)
    merge_gbs = merge_bytes / (merge_avg_ms / 1e3) / 1e9 if timed_merge else None
    # Reference for the merge's HBM roof: torch's elementwise add over buffers of O's size (two
    # reads and one write, the merge's traffic without the LSE rows), timed the same way.
    add_gbs = None
    if timed_merge:
        xa, xb = bufs.o_acc, bufs.o_part
        xc = torch.empty_like(xa)
        for _ in range(3):
            torch.add(xa, xb, out=xc)
        torch.cuda.synchronize()
        a0, a1 = ev(), ev()
        a0.record(stream)
        for _ in range(20):
            torch.add(xa, xb, out=xc)
        a1.record(stream)
        torch.cuda.synchronize()
        add_gbs = 3 * xa.numel() * 4 / (a0.elapsed_time(a1) / 20 / 1e3) / 1e9
        del xc

    backward = None
    if not args.no_backward:
        # Backward of the share in one pass (cpattn_bwd_chunks: dq and every chunk's dk, dv) from
        # the share's forward (o, lse) and a synthetic gradient.
        o_f, lse_f = bufs.o_acc, bufs.lse_acc
        cra.cpattn_fwd_chunks(q, ks, vs, cu_q, cu_ks, q_off, k_offs, True, out=o_f, lse=lse_f,
                              workspace=bufs.workspace, stream=stream)
        gen = torch.Generator(device="cuda").manual_seed(args.seed + 1)
        dout = torch.randn(q.shape, device="cuda", generator=gen).to(bf)
        f32 = dict(dtype=torch.float32, device="cuda")
        dq = torch.zeros(q.shape, **f32)
        dks = [torch.zeros(k.shape, **f32) for k in ks]
        dvs = [torch.zeros(v.shape, **f32) for v in vs]
        bws = torch.empty(max(cra.cpattn_bwd_workspace_size_chunks(len(cu_q) - 1, cu_q, cu_ks,
                                                                   w.hq, w.hkv, w.d), 256),
                          dtype=torch.uint8, device="cuda")

        def bwd_step():
            cra.cpattn_bwd_chunks(q, ks, vs, o_f, lse_f, dout, cu_q, cu_ks, q_off, k_offs, True,
                                  dq=dq, dks=dks, dvs=dvs, workspace=bws, stream=stream)

        for _ in range(max(1, args.warmup)):
            bwd_step()
        torch.cuda.synchronize()
        gc.collect()
        gc.freeze()
        gc.disable()
        try:
            b0, b1 = ev(), ev()
            b0.record(stream)
            for _ in range(args.steps):
                bwd_step()
            b1.record(stream)
            torch.cuda.synchronize()
        finally:
            gc.enable()
            gc.unfreeze()
        bwd_ms = b0.elapsed_time(b1) / args.steps
        bwd_flops = 10 * w.d * w.hq * sum(pairs_chunk)
        backward = {"ms_per_step": round(bwd_ms, 4),
                    "tflops": round(bwd_flops / (bwd_ms / 1e3) / 1e12, 2),
                    "frac": round(bwd_flops / (bwd_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                    "flops_per_step": bwd_flops,
                    "counted_as": "10 D Hq per visible pair (5 products of the forward's 2 D Hq)",
                    "launches_per_step": "delta, dQ over all chunks, dK/dV over all chunks"}

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
            g2 = w2.groups[0]
            q2 = torch.from_numpy(g2.q).to("cuda", bf)
            ks2 = [torch.from_numpy(c.k).to("cuda", bf) for c in g2.chunks]
            vs2 = [torch.from_numpy(c.v).to("cuda", bf) for c in g2.chunks]
            cu_q2 = np.ascontiguousarray(g2.cu_q, np.int32)
            q_off2 = np.ascontiguousarray(g2.q_off, np.int32)
            cu_ks2 = [np.ascontiguousarray(c.cu_k, np.int32) for c in g2.chunks]
            k_offs2 = [np.ascontiguousarray(c.k_off, np.int32) for c in g2.chunks]
            bufs2 = cra.ShareBuffers.allocate(q2, w2.hkv, cu_q2, len(g2.chunks))
            flops2 = sum(4 * w2.d * w2.hq * visible_pairs(cu_q2, c.cu_k, q_off2, c.k_off)
                         for c in g2.chunks)

            def step2():
                cra.cpattn_fwd_chunks(q2, ks2, vs2, cu_q2, cu_ks2, q_off2, k_offs2, True,
                                      out=bufs2.o_acc, lse=bufs2.lse_acc, workspace=bufs2.workspace,
                                      stream=stream)

            for _ in range(args.warmup):
                step2()
            torch.cuda.synchronize()
            gc.collect()
            gc.freeze()
            gc.disable()
            try:
                s0, s1 = ev(), ev()
                s0.record(stream)
                for _ in range(args.steps):
                    step2()
                s1.record(stream)
                torch.cuda.synchronize()
            finally:
                gc.enable()
                gc.unfreeze()
            ms2 = s0.elapsed_time(s1) / args.steps
            per_seed.append({"seed": sd, "pieces": [int(x) for x in np.diff(cu_q2)],
                             "ms_per_step": round(ms2, 4),
                             "tflops": round(flops2 / (ms2 / 1e3) / 1e12, 2)})
            tot_flops += flops2
            tot_ms += ms2
            del q2, ks2, vs2, bufs2
        seeds = {"per_seed": per_seed,
                 "aggregate_tflops": round(tot_flops / (tot_ms / 1e3) / 1e12, 2),
                 "aggregate_frac": round(tot_flops / (tot_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    import hashlib
    with open(ATTN_SOURCE, "rb") as f:
        traffic = PROFILED_TRAFFIC.get((args.workload, hashlib.sha256(f.read()).hexdigest()))
    tk_all = sum(int(c[-1]) for c in cu_ks)
    attn_bytes = tq * w.hq * w.d * 2 + 2 * tk_all * w.hkv * w.d * 2 + tq * w.hq * w.d * 4 + tq * w.hq * 4
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
        "config": {"workload": f"{w.name} (seed {w.seed}): last CP{nch} rank of "
                               f"{pack_words(w.lengths)}, local Q {tq} tokens in "
                               f"{len(cu_q) - 1} sequences, {nch} KV chunks of "
                               f"{int(cu_ks[0][-1])} tokens, {w.hq}/{w.hkv} heads, D={w.d}, causal",
                   "global_batch": int(sum(w.lengths)), "seq_len": int(max(w.lengths)),
                   "parallelism": f"cp{nch}-share"},
        "mfma_util": round(value / BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE x1)",
                     "algorithmic_bytes_per_launch": attn_bytes,
                     "kernel": "attn_fwd_bf16_kernel<128,false> over all chunks (event-timed per "
                               "cpattn_fwd_chunks call)",
                     "avg_launch_us": round(attn_avg_ms * 1e3, 2),
                     "flops_per_launch": attn_flops_per_launch},
        "schedules": schedules,
        "seeds": seeds,
        "backward": backward,
        "merge": {"schedule": "merge", "avg_launch_us": round(merge_avg_ms * 1e3, 2) if timed_merge else None,
                  "bytes_per_launch": merge_bytes, "achieved_GBs": round(merge_gbs, 1) if merge_gbs else None,
                  "hbm_frac": round(merge_gbs / HBM_PEAK_GBS, 4) if merge_gbs else None,
                  "torch_add_same_bytes_GBs": round(add_gbs, 1) if add_gbs else None},
        "flops_per_step": flops_step,
        "cpu_baseline": None,
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
        cb = cpu_baseline(w, g)
        cb["value"] = float(f"{cb['value']:.4g}")
        cb.pop("seconds", None)
        result["cpu_baseline"] = cb
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
