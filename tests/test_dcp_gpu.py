"""Dynamic CP end to end on one GPU: the library's schedule places the samples of a mini-batch,
and every rank of a CP group runs its share through the attention path.

For each CP group the scheduler forms (samples in slot order), rank r of a group of g holds
piece r of every sample (ceil(L / g) tokens, the last piece the remainder) and sees the KV
pieces 0 .. g-1 at their global positions; the ranks' outputs, put back in token order, must
be attention over the whole samples (the oracle, on sampled rows).  Ring exchange is not run:
all pieces of a group are resident on the one GPU.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import attention_ref
from parity_util import check, dev, host, sample_rows

pytestmark = pytest.mark.gpu

WORLD, LIMIT = 8, 4096


def pieces(L, g):
    p = -(-L // g)
    return [(min(r * p, L), min((r + 1) * p, L)) for r in range(g)]


@pytest.mark.parametrize("seed", [0, 1])
def test_dcp_schedule_feeds_the_attention_path(gpu_lib, seed):
    import torch
    lens = [int(x) for x in wl.lengths_for("dcp_mixed", seed)]
    sched = gpu_lib.cpattn_dcp_schedule(lens, WORLD, LIMIT)
    # every CP group of micro-batch 0 with at least two ranks, plus one single-rank group
    groups = {}
    for i, L in enumerate(lens):
        if sched["micro_batch"][i] == 0:
            key = (int(sched["group_rank"][i]), int(sched["cp_size"][i]))
            groups.setdefault(key, []).append((int(sched["slot"][i]), i))
    chosen = [k for k in sorted(groups) if k[1] >= 2] + [k for k in sorted(groups) if k[1] == 1][:1]
    assert any(k[1] >= 2 for k in chosen), "micro-batch 0 has a multi-rank group"
    rng = np.random.default_rng(100 + seed)
    hq, hkv, d = 32, 8, 128
    for first, g in chosen:
        ids = [i for _, i in sorted(groups[(first, g)])]
        glens = [lens[i] for i in ids]
        cu = wl.cu_from_lengths(glens)
        T = int(cu[-1])
        q = wl.round_to_bf16(rng.standard_normal((T, hq, d), dtype=np.float32))
        k = wl.round_to_bf16(rng.standard_normal((T, hkv, d), dtype=np.float32))
        v = wl.round_to_bf16(rng.standard_normal((T, hkv, d), dtype=np.float32))
        # KV pieces of the group: piece c of every sample, at its global position
        ks, vs, cus, offs = [], [], [], []
        for c in range(g):
            rows = np.concatenate([np.arange(cu[j] + pieces(L, g)[c][0], cu[j] + pieces(L, g)[c][1])
                                   for j, L in enumerate(glens)]).astype(np.int64)
            ks.append(dev(k[rows], "bfloat16"))
            vs.append(dev(v[rows], "bfloat16"))
            cus.append(wl.cu_from_lengths([b - a for a, b in (pieces(L, g)[c] for L in glens)]))
            offs.append(np.array([pieces(L, g)[c][0] for L in glens], np.int32))
        o_full = np.zeros((T, hq, d))
        lse_full = np.full((hq, T), -np.inf)
        for r in range(g):                       # rank first + r of the group
            rows = np.concatenate([np.arange(cu[j] + pieces(L, g)[r][0], cu[j] + pieces(L, g)[r][1])
                                   for j, L in enumerate(glens)]).astype(np.int64)
            cu_q = wl.cu_from_lengths([b - a for a, b in (pieces(L, g)[r] for L in glens)])
            q_off = np.array([pieces(L, g)[r][0] for L in glens], np.int32)
            if rows.size == 0:
                continue
            o_r, l_r = gpu_lib.cpattn_fwd_chunks(dev(q[rows], "bfloat16"), ks, vs, cu_q, cus, q_off, offs)
            torch.cuda.synchronize()
            o_full[rows] = host(o_r)
            lse_full[:, rows] = host(l_r)
        sample = sample_rows(cu, 256, extra=96, seed=seed)
        ref = attention_ref(q, k, v, cu, cu, None, None, True, rows=sample)
        check(o_full[sample], lse_full[:, sample], *ref, "bf16",
              f"group at rank {first}, cp {g}, {len(ids)} samples, {T} tokens")
