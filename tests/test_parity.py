"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Workloads are the five seeded configurations of the generator: the tiny fp32
sequence (all rows), the 4,096-token pack (all rows), and at full size the
CP4 share of a 16,384-token budget, the 128K-context CP=4 share and the
dynamic-CP mixed pack (sampled rows, always including every sequence's first
and last rows and tile boundaries).  Each chunk's partial is checked against
the oracle's attention over that chunk, and the share -- in each of its three
schedules: one launch over all chunks, per-chunk launches accumulating in the
epilogue, per-chunk partials merged by the merge kernel -- against the oracle's
unsplit attention over all of the sequence's keys.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import attention_ref, merge_ref, share_ref
from parity_util import check, dev, dtype_name, host, sample_rows

pytestmark = pytest.mark.gpu


def _run_group(cra, w, g, rows=None, mode="stream"):
    import torch
    dt = dtype_name(w.dtype)
    q = dev(g.q, dt)
    ks = [dev(c.k, dt) for c in g.chunks]
    vs = [dev(c.v, dt) for c in g.chunks]
    o, lse = cra.cpattn_share(q, ks, vs, g.cu_q, [c.cu_k for c in g.chunks], g.q_off,
                              [c.k_off for c in g.chunks], causal=w.causal, mode=mode)
    torch.cuda.synchronize()
    o_h, l_h = host(o), host(lse)
    if rows is not None:
        o_h, l_h = o_h[rows], l_h[:, rows]
    return q, ks, vs, o_h, l_h


def _all_modes(cra, w, g, ref, rows=None, what=""):
    """Every schedule of the share (one launch over all chunks, epilogue accumulation,
    explicit partials + merge) against the same oracle result."""
    out = None
    for mode in cra.MODES:
        out = _run_group(cra, w, g, rows, mode)
        check(out[3], out[4], *ref, w.dtype if w.dtype == "bf16" else "fp32", f"{what} [{mode}]")
    return out


def test_tiny_fp32_share_and_chunks(gpu_lib):
    w = wl.make("tiny", 0)
    g = w.groups[0]
    q, ks, vs, o, lse = _all_modes(gpu_lib, w, g, share_ref(g), what="tiny share")
    for c, ch in enumerate(g.chunks):
        oc, lc = gpu_lib.cpattn_fwd_chunk(q, ks[c], vs[c], g.cu_q, ch.cu_k, g.q_off, ch.k_off)
        check(host(oc), host(lc), *attention_ref(g.q, ch.k, ch.v, g.cu_q, ch.cu_k, g.q_off, ch.k_off),
              "fp32", f"tiny chunk {c}")


@pytest.mark.parametrize("seed", [0, 1])
def test_pack_bf16_all_rows(gpu_lib, seed):
    w = wl.make("pack", seed)
    g = w.groups[0]
    _all_modes(gpu_lib, w, g, share_ref(g), what=f"pack seed {seed}")


def test_cp4_share_full_size(gpu_lib):
    """The benchmarked workload, in the benchmark's launch configuration."""
    w = wl.make("cp4_share", 0)
    g = w.groups[0]
    rows = sample_rows(g.cu_q, 32, extra=256)
    q, ks, vs, o, lse = _all_modes(gpu_lib, w, g, share_ref(g, rows=rows), rows, "cp4 share")
    for c, ch in enumerate(g.chunks):
        oc, lc = gpu_lib.cpattn_fwd_chunk(q, ks[c], vs[c], g.cu_q, ch.cu_k, g.q_off, ch.k_off)
        ref = attention_ref(g.q, ch.k, ch.v, g.cu_q, ch.cu_k, g.q_off, ch.k_off, rows=rows)
        check(host(oc)[rows], host(lc)[:, rows], *ref, "bf16", f"cp4 chunk {c}")


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_cp4_share_other_packs(gpu_lib, seed):
    """The other packs the benchmark times (same shapes, other sequence lengths), through the
    benchmarked call: one launch over all chunks."""
    w = wl.make("cp4_share", seed)
    g = w.groups[0]
    rows = sample_rows(g.cu_q, 32, extra=128, seed=seed)
    _, _, _, o, lse = _run_group(gpu_lib, w, g, rows, "stream")
    check(o, lse, *share_ref(g, rows=rows), "bf16", f"cp4 share seed {seed}")


def test_ctx128k_share_full_size(gpu_lib):
    """The 128K share on a sample of over 4,096 rows x all 8 heads: the first and last row of
    every 32-token tile (1,024 tiles), every row of the first 128 (the rows that see the
    fewest keys of the diagonal chunk), and 2,304 random draws (4,242 distinct rows)."""
    w = wl.make("ctx128k_share", 0)
    g = w.groups[0]
    rows = np.union1d(sample_rows(g.cu_q, 32, extra=2304, seed=11), np.arange(128))
    assert len(rows) >= 4096
    _all_modes(gpu_lib, w, g, share_ref(g, rows=rows), rows, "128k share")


def test_dcp_mixed_full_size(gpu_lib):
    w = wl.make("dcp_mixed", 0)
    for gi, g in enumerate(w.groups):
        rows = sample_rows(g.cu_q, 512, extra=64, seed=gi)
        _all_modes(gpu_lib, w, g, share_ref(g, rows=rows), rows, f"dcp group cp={len(g.chunks)}")


def test_merge_matches_oracle_and_is_exact_for_empty_sides(gpu_lib):
    import torch
    rng = np.random.default_rng(5)
    t, h, d = 1000, 8, 128
    oa = rng.standard_normal((t, h, d)).astype(np.float32)
    ob = rng.standard_normal((t, h, d)).astype(np.float32)
    la = (rng.standard_normal((h, t)) * 4).astype(np.float32)
    lb = (rng.standard_normal((h, t)) * 4).astype(np.float32)
    la[:, ::7] = -np.inf; oa[::7] = 0          # a empty on some rows
    lb[:, ::5] = -np.inf; ob[::5] = 0          # b empty on some rows (both empty on rows % 35)
    lb[:, 3] = la[:, 3] + 80.0                 # one side dominates
    A, LA, B, LB = (torch.from_numpy(x).cuda() for x in (oa, la, ob, lb))
    gpu_lib.cpattn_merge(A, LA, B, LB)
    torch.cuda.synchronize()
    o_ref, l_ref = merge_ref(oa, la, ob, lb)
    check(host(A), host(LA), o_ref, l_ref, "fp32", "merge")
    a_empty = np.isneginf(la)
    b_empty = np.isneginf(lb)
    got_o, got_l = A.cpu().numpy(), LA.cpu().numpy()
    # an empty side leaves the other exactly unchanged (bitwise)
    for hh in range(h):
        only_a = ~a_empty[hh] & b_empty[hh]
        only_b = a_empty[hh] & ~b_empty[hh]
        assert np.array_equal(got_o[only_a, hh], oa[only_a, hh])
        assert np.array_equal(got_l[hh, only_a], la[hh, only_a])
        assert np.array_equal(got_o[only_b, hh], ob[only_b, hh])
        assert np.array_equal(got_l[hh, only_b], lb[hh, only_b])


def test_merge_bandwidth_shape_d64(gpu_lib):
    import torch
    rng = np.random.default_rng(6)
    t, h, d = 333, 3, 64
    oa, ob = (rng.standard_normal((t, h, d)).astype(np.float32) for _ in range(2))
    la, lb = ((rng.standard_normal((h, t)) * 3).astype(np.float32) for _ in range(2))
    A, LA, B, LB = (torch.from_numpy(x).cuda() for x in (oa, la, ob, lb))
    gpu_lib.cpattn_merge(A, LA, B, LB)
    check(host(A), host(LA), *merge_ref(oa, la, ob, lb), "fp32", "merge d64")
