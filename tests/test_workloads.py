"""The seeded generator: determinism, budgets from the pages, length rules."""
import json
import os

import numpy as np
import pytest

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _fig(name):
    with open(GOLDEN) as f:
        return json.load(f)[name]["value"]


def test_lengths_are_deterministic_and_fill_budgets():
    for seed in range(5):
        assert wl.lengths_for("pack", seed) == wl.lengths_for("pack", seed)
        pack = wl.lengths_for("pack", seed)
        assert sum(pack) == 4096 and all(1 <= x <= 1024 for x in pack)
        assert all(64 <= x for x in pack[:-1])
        dcp = wl.lengths_for("dcp_mixed", seed)
        assert sum(dcp) == 65536 and all(1 <= x <= 32768 for x in dcp)
        assert all(32 <= x for x in dcp[:-1])


def test_cp4_share_matches_the_pages_budget():
    fig = _fig("dcp_static_budget")
    for seed in range(5):
        pieces = wl.lengths_for("cp4_share", seed)
        assert sum(pieces) == fig["per_rank_limit"]
        assert sum(fig["context_parallel_size"] * p for p in pieces) == fig["packed_budget_tokens"]
        assert all(512 <= p <= 4096 for p in pieces[:-1])


def test_ctx128k_share_matches_the_pages_split():
    fig = _fig("ctx128k_cp4")
    assert wl.lengths_for("ctx128k_share") == [fig["tokens_per_gpu"]]
    assert fig["tokens_per_gpu"] * fig["context_parallel_size"] == fig["context_tokens"]


def test_dcp_chunk_rule():
    sizes = _fig("dcp_power_of_two_groups")["cp_sizes"]
    for L in [1, 32, 4096, 4097, 8192, 8193, 16384, 16385, 32768]:
        cp = wl.dcp_chunk_count(L)
        assert cp in sizes
        assert -(-L // cp) <= 4096
        smaller = [c for c in sizes if c < cp]
        assert all(-(-L // c) > 4096 for c in smaller)


def test_round_to_bf16_is_round_to_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.00390625, 0.0, -0.0, 3.0e38], np.float32)])
    got = wl.round_to_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_small_workloads_layout():
    w = wl.make("tiny", 0)
    g = w.groups[0]
    assert g.q.shape == (256, 2, 64) and g.q.dtype == np.float32
    assert [c.k.shape[0] for c in g.chunks] == [128, 128]
    assert [int(c.k_off[0]) for c in g.chunks] == [0, 128]
    np.testing.assert_array_equal(np.concatenate([c.k for c in g.chunks]), g.k_full)
    w = wl.make("pack", 3)
    g = w.groups[0]
    assert g.q.shape == (4096, 32, 128) and len(g.chunks) == 1
    assert np.array_equal(g.chunks[0].cu_k, g.cu_q)
    assert np.array_equal(wl.round_to_bf16(g.q), g.q)
    a = wl.make("pack", 3)
    assert np.array_equal(a.groups[0].q, g.q) and np.array_equal(a.groups[0].chunks[0].v, g.chunks[0].v)


def test_cp4_share_chunks_are_pieces_of_the_global_sequences():
    w = wl.make("cp4_share", 1)
    g = w.groups[0]
    pieces = wl.lengths_for("cp4_share", 1)
    assert np.array_equal(np.diff(g.cu_q), pieces)
    assert np.array_equal(g.q_off, [3 * p for p in pieces])
    for c, ch in enumerate(g.chunks):
        assert np.array_equal(ch.cu_k, g.cu_q)
        assert np.array_equal(ch.k_off, [c * p for p in pieces])
        for i, p in enumerate(pieces):
            glob = g.k_full[g.cu_full[i] + c * p: g.cu_full[i] + (c + 1) * p]
            np.testing.assert_array_equal(ch.k[ch.cu_k[i]:ch.cu_k[i + 1]], glob)
