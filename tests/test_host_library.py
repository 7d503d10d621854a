"""Host side of libcpattn, on the CPU: exported symbols, the planner, error paths.

No compute call reaches a GPU here: the planner is host code, and every
invalid-argument path returns before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads as wl
from oracle import visible_pairs_ref

cra = pytest.importorskip("context_ring_attention_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return cra.load()


def test_library_exports_every_declared_symbol(lib):
    with open(os.path.join(ROOT, "include", "cpattn.h")) as f:
        text = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(cpattn_\w+)\s*\(", text, re.M))
    assert declared == set(cra.EXPORTED), declared ^ set(cra.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    # ...and that they are real dynamic symbols of the shared object
    out = os.popen(f"nm -D --defined-only {cra.LIB_PATH}").read()
    for name in declared:
        assert re.search(rf"\bT {name}$", out, re.M), name


def test_status_strings(lib):
    for s in range(5):
        assert lib.cpattn_status_string(s)
    assert b"unknown" in lib.cpattn_status_string(99)


def _rows_of(entries):
    return [(int(e["row0"]), int(e["nrows"])) for e in entries]


@pytest.mark.parametrize("dtype,hq,hkv", [(cra.BF16, 32, 8), (cra.BF16, 8, 1), (cra.BF16, 4, 4),
                                          (cra.BF16, 6, 3), (cra.BF16, 4, 2), (cra.FP32, 2, 2)])
def test_plan_covers_every_query_once_and_every_visible_key(dtype, hq, hkv):
    rng = np.random.default_rng(hq * 7 + hkv)
    for trial in range(25):
        causal = trial % 5 != 0
        nseq = int(rng.integers(0, 6))
        q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, nseq, 300, 1, 1, 1, dtype="fp32")
        entries, info = cra.cpattn_plan_build(cu_q, cu_k, qo, ko, hq=hq, hkv=hkv, d=128,
                                              dtype=dtype, causal=causal)
        tt, bn = info["tokens_per_tile"], info["block_n"]
        assert hq % info["heads_per_tile"] == 0 and (hq // hkv) % info["heads_per_tile"] == 0
        assert info["n_tiles"] == info["n_entries"] * hq // info["heads_per_tile"]
        assert info["visible_pairs"] == visible_pairs_ref(cu_q, cu_k, qo, ko, causal)
        # every query row appears in exactly one entry
        cover = np.zeros(int(cu_q[-1]), dtype=int)
        for e in entries:
            assert 1 <= e["nrows"] <= tt
            cover[e["row0"]:e["row0"] + e["nrows"]] += 1
            i = int(e["seq"])
            assert cu_q[i] <= e["row0"] and e["row0"] + e["nrows"] <= cu_q[i + 1]
            assert e["row0"] == cu_q[i] + e["tblock"] * tt
            assert e["k_start"] == cu_k[i] and e["k_len"] == cu_k[i + 1] - cu_k[i]
            # the blocks visited cover every visible key of every row, and no more blocks
            kpos = ko[i] + np.arange(e["k_len"])
            last_visible = -1
            for r in range(int(e["nrows"])):
                t = e["row0"] - cu_q[i] + r
                vis = (kpos <= qo[i] + t) if causal else np.ones_like(kpos, bool)
                # the kernel's rule: row r sees u <= delta + r
                rule = np.arange(e["k_len"]) <= e["delta"] + r
                assert np.array_equal(vis, rule)
                if vis.any():
                    last_visible = max(last_visible, int(np.nonzero(vis)[0].max()))
            assert e["cost"] == (last_visible + bn) // bn if last_visible >= 0 else e["cost"] == 0
        assert np.all(cover == 1)
        # longest first, ties in (sequence, block) order
        costs = entries["cost"]
        assert np.all(costs[:-1] >= costs[1:])
        for a, b in zip(entries[:-1], entries[1:]):
            if a["cost"] == b["cost"]:
                assert (a["seq"], a["tblock"]) < (b["seq"], b["tblock"])


def test_workspace_size_bounds_every_geometry():
    rng = np.random.default_rng(3)
    for _ in range(20):
        nseq = int(rng.integers(0, 8))
        cu = wl.cu_from_lengths(rng.integers(0, 500, size=nseq))
        for dtype, hq, hkv in [(cra.BF16, 32, 8), (cra.BF16, 8, 8), (cra.FP32, 4, 2)]:
            _, info = cra.cpattn_plan_build(cu, cu, None, None, hq=hq, hkv=hkv, d=64, dtype=dtype)
            assert cra.cpattn_workspace_size(nseq, cu, hq, hkv, 64) >= info["plan_bytes"]


def test_share_workload_plans():
    """The 4,096-token CP4 share: diagonal chunk tiles cost 1..n blocks, the others n."""
    pieces = wl.lengths_for("cp4_share", 0)
    cu = wl.cu_from_lengths(pieces)
    for c in range(4):
        entries, info = cra.cpattn_plan_build(cu, cu, [3 * p for p in pieces], [c * p for p in pieces],
                                              hq=32, hkv=8, d=128)
        assert info["visible_pairs"] == visible_pairs_ref(cu, cu, [3 * p for p in pieces],
                                                          [c * p for p in pieces])
        if c < 3:
            assert all(e["cost"] == -(-e["k_len"] // 64) for e in entries)
        else:
            assert entries["cost"].min() == 1


# ----------------------------------------------------------------------------
# error paths (all return a status, never abort, and touch no GPU)
# ----------------------------------------------------------------------------
BAD_PLANS = [
    (dict(cu_q=[0, 5, 3], cu_k=[0, 5, 6]), cra._binding.ERR_INVALID_ARG),          # decreasing
    (dict(cu_q=[1, 5], cu_k=[0, 5]), cra._binding.ERR_INVALID_ARG),                # does not start at 0
    (dict(cu_q=[0, 5], cu_k=[0, 5], qo=[-1]), cra._binding.ERR_INVALID_ARG),       # negative offset
    (dict(cu_q=[0, 5], cu_k=[0, 5], ko=[2**31 - 3]), cra._binding.ERR_INVALID_ARG),  # overflow
    (dict(hq=6, hkv=4), cra._binding.ERR_INVALID_ARG),                            # hq % hkv
    (dict(hq=0), cra._binding.ERR_INVALID_ARG),
    (dict(d=96), cra._binding.ERR_UNSUPPORTED),
    (dict(d=256), cra._binding.ERR_UNSUPPORTED),
    (dict(dtype=7), cra._binding.ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,status", BAD_PLANS)
def test_invalid_plan_arguments(kw, status):
    args = dict(cu_q=[0, 5], cu_k=[0, 5], qo=None, ko=None, hq=4, hkv=2, d=64, dtype=cra.BF16)
    args.update(kw)
    with pytest.raises(cra.CpattnError) as ei:
        cra.cpattn_plan_build(args["cu_q"], args["cu_k"], args["qo"], args["ko"], hq=args["hq"],
                              hkv=args["hkv"], d=args["d"], dtype=args["dtype"])
    assert ei.value.status == status


def _i32(a):
    arr = np.ascontiguousarray(a, dtype=np.int32)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def test_fwd_chunk_rejects_bad_arguments_without_a_gpu(lib):
    cu, pcu = _i32([0, 64])
    fake = ctypes.c_void_p(4096)          # never dereferenced: validation fails first
    mis = ctypes.c_void_p(4096 + 8)       # not 16-byte aligned
    ws = ctypes.c_void_p(1 << 20)
    call = lambda **kw: lib.cpattn_fwd_chunk(
        kw.get("q", fake), kw.get("k", fake), kw.get("v", fake), kw.get("cuq", pcu),
        kw.get("cuk", pcu), None, None, kw.get("nseq", 1), kw.get("hq", 4), kw.get("hkv", 2),
        kw.get("d", 64), kw.get("dtype", 0), 1, kw.get("o", ctypes.c_void_p(1 << 30)),
        kw.get("lse", ctypes.c_void_p(1 << 31)), kw.get("ws", ws), kw.get("wsb", 1 << 20), None)
    assert call(q=ctypes.c_void_p(0)) == cra._binding.ERR_INVALID_ARG
    assert call(q=mis) == cra._binding.ERR_INVALID_ARG
    assert call(d=80) == cra._binding.ERR_UNSUPPORTED
    assert call(hq=3) == cra._binding.ERR_INVALID_ARG
    assert call(dtype=5) == cra._binding.ERR_INVALID_ARG
    assert call(nseq=-1) == cra._binding.ERR_INVALID_ARG
    assert call(ws=ctypes.c_void_p(0)) == cra._binding.ERR_WORKSPACE
    assert call(wsb=8) == cra._binding.ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p((1 << 20) + 16)) == cra._binding.ERR_WORKSPACE   # misaligned
    assert call(o=ctypes.c_void_p(4096)) == cra._binding.ERR_INVALID_ARG            # o aliases q
    bad, pbad = _i32([0, 70, 64])
    assert call(cuq=pbad, nseq=2) == cra._binding.ERR_INVALID_ARG
    assert b"non-decreasing" in lib.cpattn_last_error()
    empty, pempty = _i32([0])
    assert call(cuq=pempty, cuk=pempty, nseq=0) == cra._binding.OK                # nothing to do


def test_merge_rejects_bad_arguments_without_a_gpu(lib):
    a, b = ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 32)
    la, lb = ctypes.c_void_p(1 << 33), ctypes.c_void_p(1 << 34)
    assert lib.cpattn_merge(a, la, b, lb, 16, 2, 96, None) == cra._binding.ERR_INVALID_ARG
    assert lib.cpattn_merge(a, la, b, lb, -1, 2, 64, None) == cra._binding.ERR_INVALID_ARG
    assert lib.cpattn_merge(a, la, a, lb, 16, 2, 64, None) == cra._binding.ERR_INVALID_ARG   # alias
    assert lib.cpattn_merge(None, la, b, lb, 16, 2, 64, None) == cra._binding.ERR_INVALID_ARG
    assert lib.cpattn_merge(a, la, b, lb, 0, 2, 64, None) == cra._binding.OK              # empty


# ----------------------------------------------------------------------------
# plans over several KV chunks (cpattn_fwd_chunks)
# ----------------------------------------------------------------------------
def _random_split(rng, cu_k, ko, nchunks):
    """Cut every sequence's keys into nchunks contiguous pieces (empty pieces allowed)."""
    nseq = len(cu_k) - 1
    cus, offs = [], []
    cuts = [sorted(rng.integers(0, cu_k[i + 1] - cu_k[i] + 1, size=nchunks - 1).tolist())
            for i in range(nseq)]
    for c in range(nchunks):
        lens, off = [], []
        for i in range(nseq):
            b = [0] + cuts[i] + [int(cu_k[i + 1] - cu_k[i])]
            lens.append(b[c + 1] - b[c])
            off.append(int(ko[i]) + b[c])
        cus.append(wl.cu_from_lengths(lens))
        offs.append(np.array(off, np.int32))
    return cus, offs


FIELDS = ("row0", "nrows", "k_start", "k_len", "delta", "cost", "seq", "tblock")


@pytest.mark.parametrize("dtype,hq,hkv", [(cra.BF16, 32, 8), (cra.BF16, 8, 1), (cra.FP32, 4, 2)])
def test_multi_chunk_plan_is_the_per_chunk_plans_tile_major(dtype, hq, hkv):
    rng = np.random.default_rng(hq + 100 * hkv)
    for trial in range(20):
        causal = trial % 4 != 0
        nseq = int(rng.integers(0, 6))
        nch = int(rng.integers(1, 9))
        _, _, _, cu_q, cu_k, qo, ko = wl.random_pack(rng, nseq, 300, 1, 1, 1, dtype="fp32")
        cus, offs = _random_split(rng, cu_k, ko, nch)
        ent, info = cra.cpattn_plan_build_chunks(cu_q, cus, qo, offs, hq=hq, hkv=hkv, d=128,
                                                 dtype=dtype, causal=causal)
        assert info["n_chunks"] == nch and len(ent) == info["n_entries"]
        assert len(ent) % nch == 0
        n_t = len(ent) // nch
        assert info["n_tiles"] == n_t * hq // info["heads_per_tile"]
        assert info["visible_pairs"] == sum(visible_pairs_ref(cu_q, cus[c], qo, offs[c], causal)
                                            for c in range(nch))
        assert info["key_blocks"] == int(ent["cost"].sum())
        singles = []
        for c in range(nch):
            e1, _ = cra.cpattn_plan_build(cu_q, cus[c], qo, offs[c], hq=hq, hkv=hkv, d=128,
                                          dtype=dtype, causal=causal)
            singles.append({(int(e["seq"]), int(e["tblock"])): e for e in e1})
        tiles = ent.reshape(n_t, nch) if n_t else ent.reshape(0, nch)
        keys = []
        for t in range(n_t):
            key = (int(tiles[t, 0]["seq"]), int(tiles[t, 0]["tblock"]))
            keys.append(key)
            for c in range(nch):
                ref = singles[c][key]
                assert all(tiles[t, c][f] == ref[f] for f in FIELDS), (t, c)
        assert len(set(keys)) == n_t and set(keys) == set(singles[0]) if nch else True
        totals = tiles["cost"].sum(axis=1) if n_t else np.zeros(0)
        assert np.all(totals[:-1] >= totals[1:])
        for t in range(n_t - 1):
            if totals[t] == totals[t + 1]:
                assert keys[t] < keys[t + 1]


def test_one_chunk_plan_equals_plan_build():
    rng = np.random.default_rng(8)
    _, _, _, cu_q, cu_k, qo, ko = wl.random_pack(rng, 5, 400, 1, 1, 1, dtype="fp32")
    a, ia = cra.cpattn_plan_build(cu_q, cu_k, qo, ko, hq=32, hkv=8, d=128)
    b, ib = cra.cpattn_plan_build_chunks(cu_q, [cu_k], qo, [ko], hq=32, hkv=8, d=128)
    assert np.array_equal(a, b) and ia == ib


def test_workspace_size_chunks_bounds_every_plan():
    rng = np.random.default_rng(9)
    for _ in range(20):
        nseq = int(rng.integers(0, 8))
        cu = wl.cu_from_lengths(rng.integers(0, 500, size=nseq))
        nch = int(rng.integers(1, 17))
        for dtype, hq, hkv in [(cra.BF16, 32, 8), (cra.BF16, 8, 8), (cra.FP32, 4, 2)]:
            _, info = cra.cpattn_plan_build_chunks(cu, [cu] * nch, None, None, hq=hq, hkv=hkv,
                                                   d=64, dtype=dtype)
            assert cra.cpattn_workspace_size_chunks(nseq, cu, hq, hkv, 64, nch) >= info["plan_bytes"]
    cu = wl.cu_from_lengths([10, 20])
    assert cra.cpattn_workspace_size_chunks(2, cu, 4, 2, 64, 0) == 0
    assert cra.cpattn_workspace_size_chunks(2, cu, 4, 2, 64, cra.MAX_CHUNKS + 1) == 0
    assert cra.cpattn_workspace_size_chunks(2, cu, 4, 2, 64, 1) == cra.cpattn_workspace_size(2, cu, 4, 2, 64)


def test_plan_build_chunks_rejects_bad_chunk_counts(lib):
    cu, pcu = _i32([0, 5])
    info = cra._binding.PlanInfo()
    for nch in (0, -1, cra.MAX_CHUNKS + 1):
        st = lib.cpattn_plan_build_chunks(pcu, pcu, None, None, nch, 1, 4, 2, 64, 0, 1, None, 0,
                                          ctypes.byref(info))
        assert st == cra._binding.ERR_INVALID_ARG
    bad, pbad = _i32([0, 5, 0, -3])  # second chunk's prefix sums decrease
    st = lib.cpattn_plan_build_chunks(pcu, pbad, None, None, 2, 1, 4, 2, 64, 0, 1, None, 0,
                                      ctypes.byref(info))
    assert st == cra._binding.ERR_INVALID_ARG
    bad, pbad = _i32([0, 5, 1, 4])   # second chunk does not start at 0
    st = lib.cpattn_plan_build_chunks(pcu, pbad, None, None, 2, 1, 4, 2, 64, 0, 1, None, 0,
                                      ctypes.byref(info))
    assert st == cra._binding.ERR_INVALID_ARG and b"chunk 1" in lib.cpattn_last_error()


def test_fwd_chunks_rejects_bad_arguments_without_a_gpu(lib):
    cu, pcu = _i32([0, 64])
    cu2, pcu2 = _i32([0, 64, 0, 64])
    fake = ctypes.c_void_p(4096)
    ptrs = lambda *a: (ctypes.c_void_p * len(a))(*a)
    ks, vs = ptrs(1 << 24, 1 << 25), ptrs(1 << 26, 1 << 27)
    ws = ctypes.c_void_p(1 << 20)

    def call(**kw):
        return lib.cpattn_fwd_chunks(
            kw.get("q", fake), kw.get("ks", ks), kw.get("vs", vs), kw.get("nch", 2), pcu,
            kw.get("cuk", pcu2), None, None, 1, 4, 2, 64, kw.get("dtype", 0), 1, kw.get("acc", 0),
            kw.get("o", ctypes.c_void_p(1 << 30)), ctypes.c_void_p(1 << 31), ws, 1 << 20, None)

    assert call(nch=0) == cra._binding.ERR_INVALID_ARG
    assert call(nch=cra.MAX_CHUNKS + 1) == cra._binding.ERR_INVALID_ARG
    assert call(ks=None) == cra._binding.ERR_INVALID_ARG
    assert call(acc=2) == cra._binding.ERR_INVALID_ARG
    assert call(ks=ptrs(1 << 24, (1 << 25) + 8)) == cra._binding.ERR_INVALID_ARG     # misaligned k
    assert call(vs=ptrs(1 << 26, None)) == cra._binding.ERR_INVALID_ARG             # null v
    assert call(o=ctypes.c_void_p(1 << 25)) == cra._binding.ERR_INVALID_ARG         # o overlaps chunk 1's k
    assert b"overlap" in lib.cpattn_last_error()


def test_bwd_rejects_bad_arguments_without_a_gpu(lib):
    cu, pcu = _i32([0, 64])
    cu2, pcu2 = _i32([0, 64, 0, 64])
    fake = ctypes.c_void_p(4096)
    ptrs = lambda *a: (ctypes.c_void_p * len(a))(*a)
    ks, vs = ptrs(1 << 24, 1 << 25), ptrs(1 << 26, 1 << 27)
    dks, dvs = ptrs(1 << 34, 1 << 35), ptrs(1 << 36, 1 << 37)
    ws = ctypes.c_void_p(1 << 20)

    def call(**kw):
        return lib.cpattn_bwd_chunks(
            kw.get("q", fake), kw.get("ks", ks), kw.get("vs", vs), kw.get("nch", 2),
            ctypes.c_void_p(1 << 28), ctypes.c_void_p(1 << 29), ctypes.c_void_p(1 << 30), pcu,
            kw.get("cuk", pcu2), None, None, 1, 4, 2, 64, kw.get("dtype", 0), 1,
            kw.get("dq", ctypes.c_void_p(1 << 33)), kw.get("dks", dks), kw.get("dvs", dvs), ws,
            1 << 20, None)

    assert call(nch=0) == cra._binding.ERR_INVALID_ARG
    assert call(nch=cra.MAX_CHUNKS + 1) == cra._binding.ERR_INVALID_ARG
    assert call(dks=None) == cra._binding.ERR_INVALID_ARG
    assert call(dtype=1) == cra._binding.ERR_UNSUPPORTED                    # fp32: forward only
    assert call(q=ctypes.c_void_p(0)) == cra._binding.ERR_INVALID_ARG
    assert call(dq=ctypes.c_void_p(1 << 24)) == cra._binding.ERR_INVALID_ARG  # dq overlaps k of chunk 0
    assert call(dvs=ptrs(1 << 36, 1 << 34)) == cra._binding.ERR_INVALID_ARG  # dv aliases dk
    assert b"overlap" in lib.cpattn_last_error()
    assert cra.cpattn_bwd_workspace_size_chunks(1, [0, 64], [[0, 64]] * 2, 4, 2, 64) >= \
        cra.cpattn_bwd_workspace_size(1, [0, 64], [0, 64], 4, 2, 64)


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 1), (4, 4)])
def test_key_plan_covers_every_key_once_and_every_query_that_sees_it(hq, hkv):
    """The backward's key-stationary plan (cpattn_key_plan_build) on random packs split into
    random chunks: every key row of every chunk is in exactly one tile; a tile's rule
    (query t sees tile key r iff t >= delta + r) is the causal mask by global position;
    every query that sees a tile key lies in the visited range [max(delta, 0), q_len), whose
    length in query blocks is the cost; tiles are ordered longest first."""
    rng = np.random.default_rng(hq + 3 * hkv)
    for trial in range(20):
        causal = trial % 4 != 0
        nseq = int(rng.integers(0, 5))
        nch = int(rng.integers(1, 5))
        lq = rng.integers(0, 300, size=nseq)
        cu_q = wl.cu_from_lengths(lq)
        q_off = rng.integers(0, 600, size=nseq).astype(np.int32)
        cu_ks, k_offs = [], []
        for c in range(nch):
            cu_ks.append(wl.cu_from_lengths(rng.integers(0, 400, size=nseq)))
            k_offs.append(rng.integers(0, 900, size=nseq).astype(np.int32))
        tiles, info = cra.cpattn_key_plan_build(cu_q, cu_ks, q_off, k_offs, hq=hq, hkv=hkv, d=128,
                                                causal=causal)
        kt, qb = info["keys_per_tile"], info["query_block"]
        assert info["n_tiles"] == len(tiles)
        cover = [np.zeros(int(ck[-1]), dtype=int) for ck in cu_ks]
        for t in tiles:
            c = int(t["chunk"])
            ck = cu_ks[c]
            assert 1 <= t["nrows"] <= kt
            i = int(np.searchsorted(ck, t["row0"], side="right") - 1)
            assert ck[i] <= t["row0"] and t["row0"] + t["nrows"] <= ck[i + 1]
            assert (t["row0"] - ck[i]) % kt == 0
            assert t["q_start"] == cu_q[i] and t["q_len"] == lq[i]
            cover[c][t["row0"]:t["row0"] + t["nrows"]] += 1
            nq = int(lq[i])
            qpos = int(q_off[i]) + np.arange(nq)
            first = max(int(t["delta"]), 0)
            for r in range(int(t["nrows"])):
                kpos = int(k_offs[c][i]) + int(t["row0"] - ck[i]) + r
                vis = (qpos >= kpos) if causal else np.ones(nq, bool)
                rule = np.arange(nq) >= int(t["delta"]) + r
                assert np.array_equal(vis, rule)
                if vis.any():
                    assert int(np.nonzero(vis)[0].min()) >= first
            assert t["cost"] == max(0, -(-(nq - first) // qb))
        for c in range(nch):
            assert np.all(cover[c] == 1)
        costs = tiles["cost"]
        assert np.all(costs[:-1] >= costs[1:])
        for a, b in zip(tiles[:-1], tiles[1:]):
            if a["cost"] == b["cost"]:
                assert (a["chunk"], a["row0"]) < (b["chunk"], b["row0"])


def test_key_plan_rejects_bad_arguments(lib):
    cu = np.array([0, 10], np.int32)
    p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    # hq not a multiple of hkv, a bad head dim, a short plan buffer
    assert lib.cpattn_key_plan_build(p, p, None, None, 1, 1, 6, 4, 128, 1, None, 0, None) == 1
    assert lib.cpattn_key_plan_build(p, p, None, None, 1, 1, 4, 4, 96, 1, None, 0, None) == 2
    buf = ctypes.create_string_buffer(16)
    assert lib.cpattn_key_plan_build(p, p, None, None, 1, 1, 4, 4, 128, 1, buf, 16, None) == 3


def test_binding_refuses_host_tensors_before_any_launch():
    """Every tensor the kernels write through (outputs, gradients, the workspace) must be a
    CUDA tensor on q's device; the binding checks that before it touches the library, so a
    host pointer never reaches a kernel."""
    import torch
    from context_ring_attention_amd import _binding as b
    dev0 = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="CUDA"):
        b._on_device("out", torch.zeros(4), dev0)
    with pytest.raises(ValueError, match="CUDA"):
        b._workspace(torch.zeros(256, dtype=torch.uint8), 16, dev0)
    with pytest.raises(ValueError, match="CUDA"):
        b._on_device("dk", torch.zeros((3, 2, 64)), dev0)
