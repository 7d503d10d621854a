"""Dynamic CP scheduler: the library against the plain-Python reference, and the reference
pinned by closed forms, invariants and the workload generator's per-sample CP rule.

Constraints from the verl page "Dynamic Context Parallelism" (per-rank limit
max_seqlen_per_dp_cp_rank, power-of-two CP subgroups plus the full DP x CP group,
even world of at least two); the assignment rule is the reading documented in
oracle/dcp.py.  Host only: no GPU.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import context_ring_attention_amd as cra
import workloads as wl
from oracle.dcp import dcp_schedule_ref

pytestmark = pytest.mark.filterwarnings("ignore")


def check_schedule(lengths, world, limit, res):
    """Validity of a schedule, checked from its definition (independent of both implementations)."""
    n = len(lengths)
    nmb = res["n_micro_batches"]
    allowed = sorted({2 ** k for k in range(world.bit_length()) if 2 ** k <= world} | {world})
    groups = {}                      # (mb, first) -> size
    load = np.zeros((nmb, world), dtype=np.int64)
    slots = {}
    for i in range(n):
        L, g, b, f, s = (int(lengths[i]), int(res["cp_size"][i]), int(res["micro_batch"][i]),
                         int(res["group_rank"][i]), int(res["slot"][i]))
        assert g in allowed
        assert -(-L // g) <= limit, "pieces must fit the limit"
        smaller = [a for a in allowed if a < g]
        assert all(-(-L // a) > limit for a in smaller), "cp size must be the smallest that fits"
        assert 0 <= b < nmb and 0 <= f and f + g <= world
        assert (f % g == 0) if g & (g - 1) == 0 else f == 0, "groups are aligned"
        assert groups.setdefault((b, f), g) == g
        p = -(-L // g)
        piece = [max(0, min(p, L - r * p)) for r in range(g)]
        assert sum(piece) == L
        load[b, f:f + g] += piece
        slots.setdefault((b, f), []).append(s)
    assert (load <= limit).all(), "no rank exceeds the per-rank limit"
    for b in range(nmb):   # groups of one micro-batch do not overlap
        owned = np.zeros(world, dtype=np.int32)
        for (bb, f), g in groups.items():
            if bb == b:
                owned[f:f + g] += 1
        assert owned.max() <= 1
        assert any(bb == b for bb, _ in groups), "no empty micro-batch"
    for v in slots.values():
        assert sorted(v) == list(range(len(v)))
    total = sum(int(x) for x in lengths)
    assert nmb >= math.ceil(total / (world * limit)) if total else nmb >= (1 if n else 0)


def same(a, b):
    assert a["n_micro_batches"] == b["n_micro_batches"]
    for k in ("cp_size", "micro_batch", "group_rank", "slot"):
        assert list(map(int, a[k])) == list(map(int, b[k])), k


# ---------------------------------------------------------------------------------------------
# the reference, pinned
# ---------------------------------------------------------------------------------------------
def test_ref_cp_rule_is_the_workload_rule():
    """CP size = the per-sample rule the Dynamic-CP workload uses (smallest of 1, 2, 4, 8 with
    ceil(L / cp) <= 4096), written independently in workloads.py."""
    rng = np.random.default_rng(0)
    lens = list(wl.lengths_for("dcp_mixed", 0)) + list(rng.integers(0, 32769, 500)) + [0, 1, 4096,
                                                                                       4097, 8192, 8193,
                                                                                       16384, 16385,
                                                                                       32768]
    res = dcp_schedule_ref(lens, 8, 4096)
    assert res["cp_size"] == [wl.dcp_chunk_count(int(x), 4096) for x in lens]
    check_schedule(lens, 8, 4096, res)


@pytest.mark.parametrize("world", [2, 4, 8, 16])
def test_ref_closed_forms(world):
    M = 4096
    for n in (1, world - 1, world, 3 * world + 1):
        r = dcp_schedule_ref([M] * n, world, M)          # one full rank per sample
        assert r["cp_size"] == [1] * n and r["n_micro_batches"] == math.ceil(n / world)
        assert r["slot"] == [0] * n
        r = dcp_schedule_ref([M // 2] * n, world, M)     # two samples per rank
        assert r["n_micro_batches"] == math.ceil(n / (2 * world))
        r = dcp_schedule_ref([2 * M] * n, world, M)      # two ranks per sample
        assert r["cp_size"] == [2] * n and r["n_micro_batches"] == math.ceil(n / (world // 2))
        r = dcp_schedule_ref([world * M] * n, world, M)  # the whole world per sample
        assert r["cp_size"] == [world] * n and r["n_micro_batches"] == n
        assert r["group_rank"] == [0] * n


def test_ref_full_group_for_non_power_of_two_world():
    """world 6: a sample needing more than 4 ranks takes the full 6-rank group (the page's
    'full DPxCP group when needed'); shorter ones take aligned power-of-two groups."""
    M = 1000
    r = dcp_schedule_ref([5 * M, 3 * M, M, M], 6, M)
    assert r["cp_size"] == [6, 4, 1, 1]
    assert r["micro_batch"][0] == 0 and r["group_rank"][0] == 0
    # the 4-rank group cannot share micro-batch 0 (every rank is in the full group)
    assert r["micro_batch"][1] == 1 and r["group_rank"][1] == 0
    # the single-rank samples fill ranks 4 and 5 next to it
    assert sorted(r["group_rank"][2:]) == [4, 5] and r["micro_batch"][2:] == [1, 1]
    check_schedule([5 * M, 3 * M, M, M], 6, M, r)


def test_ref_first_fit_order():
    """Placement follows decreasing (cp, length) with first fit: a short sample joins the first
    group of its size that still has room."""
    r = dcp_schedule_ref([3000, 1000, 1200, 3500], 2, 4096)
    # order: 3500, 3000, 1200, 1000 (all cp 1); ranks: 3500 -> r0, 3000 -> r1, 1200 -> no room on
    # r0 (4700) but r1? 4200 > 4096 -> new micro-batch; 1000 -> r0 (4500)? no; r1 (4000) yes
    assert r["micro_batch"] == [0, 0, 1, 0]
    assert r["group_rank"] == [1, 1, 0, 0]
    assert r["slot"] == [0, 1, 0, 0]


@settings(max_examples=150, deadline=None)
@given(st.lists(st.integers(0, 40000), max_size=40), st.sampled_from([2, 4, 6, 8, 10, 16]),
       st.sampled_from([1024, 4096, 5000]))
def test_ref_invariants(lengths, world, limit):
    lengths = [x for x in lengths if -(-x // world) <= limit]
    check_schedule(lengths, world, limit, dcp_schedule_ref(lengths, world, limit))


# ---------------------------------------------------------------------------------------------
# the library against the reference
# ---------------------------------------------------------------------------------------------
@settings(max_examples=150, deadline=None)
@given(st.lists(st.integers(0, 40000), max_size=60), st.sampled_from([2, 4, 6, 8, 10, 16]),
       st.sampled_from([1024, 4096, 5000]))
def test_library_matches_reference(lengths, world, limit):
    lengths = [x for x in lengths if -(-x // world) <= limit]
    same(cra.cpattn_dcp_schedule(lengths, world, limit), dcp_schedule_ref(lengths, world, limit))


@pytest.mark.parametrize("seed", range(5))
def test_library_on_dynamic_cp_minibatches(seed):
    """The Dynamic-CP mix (65,536 tokens, lognormal lengths) on DPxCP = 8 with the CP4 limit,
    and a mini-batch 16x larger."""
    lens = wl.lengths_for("dcp_mixed", seed)
    for world in (8, 16):
        res = cra.cpattn_dcp_schedule(lens, world, 4096)
        same(res, dcp_schedule_ref(lens, world, 4096))
        check_schedule(lens, world, 4096, res)
    big = np.concatenate([wl.lengths_for("dcp_mixed", seed * 16 + k) for k in range(16)])
    same(cra.cpattn_dcp_schedule(big, 8, 4096), dcp_schedule_ref(big, 8, 4096))


def test_library_edges_and_errors():
    r = cra.cpattn_dcp_schedule([], 8, 4096)
    assert r["n_micro_batches"] == 0 and len(r["cp_size"]) == 0
    r = cra.cpattn_dcp_schedule([0, 0], 2, 1)
    assert r["n_micro_batches"] == 1 and list(r["cp_size"]) == [1, 1]
    for lengths, world, limit in [([10], 3, 100), ([10], 0, 100), ([10], -2, 100), ([10], 2, 0),
                                  ([-1], 2, 100), ([201], 2, 100)]:
        with pytest.raises(cra.CpattnError) as e:
            cra.cpattn_dcp_schedule(lengths, world, limit)
        assert e.value.status == cra._binding.ERR_INVALID_ARG


# ---------------------------------------------------------------------------------------------
# hand-derived placements (worked through the reading step by step; see each comment)
# ---------------------------------------------------------------------------------------------
def _lib_schedule(lengths, world, limit):
    r = cra.cpattn_dcp_schedule(lengths, world, limit)
    return {k: (list(map(int, v)) if k != "n_micro_batches" else v) for k, v in r.items()}


def test_world6_mixes_two_rank_and_one_rank_groups_in_one_micro_batch():
    """world 6, limit 1000, lengths [1900, 1500, 800, 600, 300]:
    cp sizes: 1900 and 1500 need 2 ranks (950 and 750 per rank), the rest fit one rank.
    Order 1900, 1500, 800, 600, 300.  1900 opens micro-batch 0 with the pair at rank 0
    (950 + 950).  1500 does not fit that pair (950 + 750 > 1000), so it opens the pair at
    rank 2 (750 + 750).  800 finds no one-rank group, and ranks 0-3 are taken, so it opens
    rank 4.  600 does not fit rank 4 (1400) and opens rank 5.  300 does not fit rank 4
    (1100) but fits rank 5 (900), as its second sample.  One micro-batch in all."""
    want = {"cp_size": [2, 2, 1, 1, 1], "micro_batch": [0, 0, 0, 0, 0],
            "group_rank": [0, 2, 4, 5, 5], "slot": [0, 0, 0, 0, 1], "n_micro_batches": 1}
    lengths = [1900, 1500, 800, 600, 300]
    ref = dcp_schedule_ref(lengths, 6, 1000)
    assert ref == want
    check_schedule(lengths, 6, 1000, ref)
    assert _lib_schedule(lengths, 6, 1000) == want


def test_a_third_micro_batch_is_opened_when_both_are_full():
    """world 2, limit 1000, lengths [2000, 1500, 900, 800] (5,200 tokens: at least
    ceil(5200 / 2000) = 3 micro-batches).  2000 takes the full pair of micro-batch 0
    (1000 + 1000).  1500 (750 + 750) fits no pair there and the world has one pair, so it
    opens micro-batch 1.  900 needs one rank, and every rank of micro-batches 0 and 1 is in
    a pair, so it opens micro-batch 2 at rank 0.  800 does not fit rank 0 there (1700) and
    opens rank 1 of micro-batch 2."""
    want = {"cp_size": [2, 2, 1, 1], "micro_batch": [0, 1, 2, 2], "group_rank": [0, 0, 0, 1],
            "slot": [0, 0, 0, 0], "n_micro_batches": 3}
    lengths = [2000, 1500, 900, 800]
    ref = dcp_schedule_ref(lengths, 2, 1000)
    assert ref == want
    check_schedule(lengths, 2, 1000, ref)
    assert _lib_schedule(lengths, 2, 1000) == want
