"""GPU edge cases and properties of cpattn_fwd_chunk / cpattn_share against the oracle.

Covers: empty and one-token sequences, zero-length key chunks, chunks wholly
after the queries (every row empty), causal diagonals inside a tile, ragged
tails, non-causal mode, both head dims, every GQA grouping the tile geometry
distinguishes, outputs poisoned before launch (unwritten rows are caught),
guard bands after the outputs, determinism, random KV splits merged on the
GPU against unsplit attention, and tensors whose offsets pass 2^32 bytes.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import attention_ref
from parity_util import check, dev, host

pytestmark = pytest.mark.gpu


def _fwd(cra, q, k, v, cu_q, cu_k, qo, ko, causal, dtype, guard=0):
    """Run one chunk with NaN-poisoned outputs and a guard band after each buffer."""
    import torch
    dt = "bfloat16" if dtype == "bf16" else "float32"
    tq, hq, d = q.shape
    Q, K, V = dev(q, dt), dev(k, dt), dev(v, dt)
    o_buf = torch.full((tq * hq * d + guard,), float("nan"), device="cuda")
    l_buf = torch.full((hq * tq + guard,), float("nan"), device="cuda")
    if guard:
        o_buf[tq * hq * d:] = 12345.0
        l_buf[hq * tq:] = 12345.0
    o = o_buf[:tq * hq * d].view(tq, hq, d)
    lse = l_buf[:hq * tq].view(hq, tq)
    cra.cpattn_fwd_chunk(Q, K, V, cu_q, cu_k, qo, ko, causal, out=o, lse=lse)
    torch.cuda.synchronize()
    if guard:
        assert torch.all(o_buf[tq * hq * d:] == 12345.0), "write past the end of O"
        assert torch.all(l_buf[hq * tq:] == 12345.0), "write past the end of LSE"
    return host(o), host(lse)


def _case(cra, q, k, v, cu_q, cu_k, qo, ko, causal=True, dtype="bf16", what=""):
    o, l = _fwd(cra, q, k, v, cu_q, cu_k, qo, ko, causal, dtype, guard=4096)
    check(o, l, *attention_ref(q, k, v, cu_q, cu_k, qo, ko, causal), dtype, what)
    return o, l


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_empty_and_tiny_sequences(gpu_lib, dtype, d):
    rng = np.random.default_rng(d)
    lq = [0, 1, 5, 0, 33, 1, 70]
    lk = [3, 1, 0, 0, 40, 7, 129]
    cu_q, cu_k = wl.cu_from_lengths(lq), wl.cu_from_lengths(lk)
    q = wl._normal(rng, (int(cu_q[-1]), 4, d), dtype)
    k = wl._normal(rng, (int(cu_k[-1]), 2, d), dtype)
    v = wl._normal(rng, (int(cu_k[-1]), 2, d), dtype)
    qo = np.array([0, 0, 9, 0, 7, 0, 58], np.int32)
    ko = np.array([0, 0, 0, 0, 0, 3, 0], np.int32)
    o, l = _case(gpu_lib, q, k, v, cu_q, cu_k, qo, ko, True, dtype, "tiny seqs")
    # sequence 1: its one query (row 0) at position 0 sees exactly its one key (key row 3)
    np.testing.assert_allclose(o[0], np.repeat(v[3], 2, axis=0), atol=1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_chunk_after_queries_is_all_empty(gpu_lib, dtype):
    rng = np.random.default_rng(1)
    q = wl._normal(rng, (100, 8, 128), dtype)
    k = wl._normal(rng, (50, 2, 128), dtype)
    v = wl._normal(rng, (50, 2, 128), dtype)
    o, l = _case(gpu_lib, q, k, v, [0, 100], [0, 50], [0], [100], True, dtype, "future chunk")
    assert np.all(np.isneginf(l)) and np.all(o == 0)


@pytest.mark.parametrize("delta", [-40, -31, -1, 0, 1, 17, 31, 32, 63, 64, 65, 200])
def test_diagonal_positions(gpu_lib, delta):
    """q_off - k_off = delta moves the causal diagonal across tile and block boundaries."""
    rng = np.random.default_rng(abs(delta) + 3)
    nq, nk = 150, 190
    q = wl._normal(rng, (nq, 8, 128), "bf16")
    k = wl._normal(rng, (nk, 2, 128), "bf16")
    v = wl._normal(rng, (nk, 2, 128), "bf16")
    ko = 300
    _case(gpu_lib, q, k, v, [0, nq], [0, nk], [ko + delta], [ko], True, "bf16", f"delta {delta}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (8, 2), (8, 1), (6, 2), (6, 3), (32, 8), (3, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_gqa_groupings(gpu_lib, hq, hkv, d):
    rng = np.random.default_rng(hq * 31 + hkv + d)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 4, 200, hq, hkv, d, dtype="bf16", min_len=1)
    _case(gpu_lib, q, k, v, cu_q, cu_k, qo, ko, True, "bf16", f"gqa {hq}/{hkv} d{d}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_non_causal(gpu_lib, dtype):
    rng = np.random.default_rng(11)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 5, 180, 4, 2, 128, dtype=dtype)
    _case(gpu_lib, q, k, v, cu_q, cu_k, qo, ko, False, dtype, "non-causal")


def test_random_packs(gpu_lib):
    rng = np.random.default_rng(12)
    for trial in range(12):
        hq, hkv = [(32, 8), (8, 1), (4, 4), (16, 2)][trial % 4]
        d = [64, 128][trial % 2]
        q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, int(rng.integers(1, 8)), 700, hq, hkv, d,
                                                     dtype="bf16")
        _case(gpu_lib, q, k, v, cu_q, cu_k, qo, ko, bool(trial % 3), "bf16", f"random {trial}")


def test_large_positions(gpu_lib):
    rng = np.random.default_rng(13)
    q = wl._normal(rng, (64, 4, 64), "bf16")
    k = wl._normal(rng, (96, 4, 64), "bf16")
    v = wl._normal(rng, (96, 4, 64), "bf16")
    big = 2**31 - 200
    _case(gpu_lib, q, k, v, [0, 64], [0, 96], [big - 64 + 10], [big - 96], True, "bf16", "large pos")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_random_splits_merged_on_gpu_equal_unsplit(gpu_lib, dtype):
    import torch
    rng = np.random.default_rng(21)
    for trial in range(6):
        q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 3, 300, 8, 2, 128, dtype=dtype, min_len=1)
        n_chunks = int(rng.integers(1, 6))
        parts_rows, parts_cu, parts_off = [], [], []
        cuts = [sorted(rng.integers(0, cu_k[i + 1] - cu_k[i] + 1, size=n_chunks - 1).tolist())
                for i in range(3)]
        for c in range(n_chunks):
            rows, lens, offs = [], [], []
            for i in range(3):
                n = int(cu_k[i + 1] - cu_k[i])
                b = [0] + cuts[i] + [n]
                rows.append(np.arange(cu_k[i] + b[c], cu_k[i] + b[c + 1]))
                lens.append(b[c + 1] - b[c])
                offs.append(int(ko[i]) + b[c])
            parts_rows.append(np.concatenate(rows).astype(np.int64))
            parts_cu.append(wl.cu_from_lengths(lens))
            parts_off.append(np.array(offs, np.int32))
        dt = "bfloat16" if dtype == "bf16" else "float32"
        Q = dev(q, dt)
        ref = attention_ref(q, k, v, cu_q, cu_k, qo, ko, True)
        for mode in gpu_lib.MODES:
            o, lse = gpu_lib.cpattn_share(Q, [dev(k[r], dt) for r in parts_rows],
                                          [dev(v[r], dt) for r in parts_rows], cu_q, parts_cu, qo,
                                          parts_off, causal=True, mode=mode)
            torch.cuda.synchronize()
            check(host(o), host(lse), *ref, dtype, f"split trial {trial} ({n_chunks} chunks, {mode})")


def test_deterministic(gpu_lib):
    rng = np.random.default_rng(14)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 4, 500, 32, 8, 128, dtype="bf16", min_len=1)
    a = _fwd(gpu_lib, q, k, v, cu_q, cu_k, qo, ko, True, "bf16")
    b = _fwd(gpu_lib, q, k, v, cu_q, cu_k, qo, ko, True, "bf16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_nothing_to_do(gpu_lib):
    import torch
    q = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    o, l = gpu_lib.cpattn_fwd_chunk(q, k, k, [0], [0])
    assert o.shape == (0, 4, 64) and l.shape == (4, 0)
    q = dev(np.ones((3, 4, 64), np.float32), "bfloat16")
    o, l = gpu_lib.cpattn_fwd_chunk(q, k, k, [0, 3], [0, 0])     # no keys at all
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


def test_host_buffers_are_refused_before_any_launch(gpu_lib):
    """A host tensor given as an output, a gradient or the workspace is refused by the
    binding (its pointer would be written by a kernel); nothing is launched."""
    import torch
    rng = np.random.default_rng(3)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 3, 40, 4, 2, 64)
    Q, K, V = dev(q, "bfloat16"), dev(k, "bfloat16"), dev(v, "bfloat16")
    tq, hq, d = q.shape
    host_o = torch.zeros((tq, hq, d), dtype=torch.float32)
    host_l = torch.zeros((hq, tq), dtype=torch.float32)
    host_ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="CUDA"):
        gpu_lib.cpattn_fwd_chunk(Q, K, V, cu_q, cu_k, qo, ko, out=host_o)
    with pytest.raises(ValueError, match="CUDA"):
        gpu_lib.cpattn_fwd_chunk(Q, K, V, cu_q, cu_k, qo, ko, lse=host_l)
    with pytest.raises(ValueError, match="CUDA"):
        gpu_lib.cpattn_fwd_chunks(Q, [K], [V], cu_q, [cu_k], qo, [ko], workspace=host_ws)
    o, lse = gpu_lib.cpattn_fwd_chunk(Q, K, V, cu_q, cu_k, qo, ko)
    do = dev(rng.standard_normal(q.shape).astype(np.float32), "bfloat16")
    with pytest.raises(ValueError, match="CUDA"):
        gpu_lib.cpattn_bwd_chunk(Q, K, V, o, lse, do, cu_q, cu_k, qo, ko,
                                 dk=torch.zeros(k.shape, dtype=torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        gpu_lib.cpattn_bwd_chunks(Q, [K], [V], o, lse, do, cu_q, [cu_k], qo, [ko],
                                  workspace=host_ws)
    torch.cuda.synchronize()


def test_stream_capture_is_refused_for_host_planned_calls(gpu_lib):
    """A call whose plan is built on the host and copied (metadata too large for the device
    planner: here 300 sequences) returns CPATTN_ERR_UNSUPPORTED on a stream that is being
    captured, before anything is enqueued (the copy would read a host buffer freed at return)."""
    import torch
    rng = np.random.default_rng(4)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 300, 6, 4, 2, 64, min_len=1)
    Q, K, V = dev(q, "bfloat16"), dev(k, "bfloat16"), dev(v, "bfloat16")
    tq, hq, d = q.shape
    o = torch.zeros((tq, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.zeros((hq, tq), dtype=torch.float32, device="cuda")
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    err = None
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        graph.capture_begin()
        try:
            gpu_lib.cpattn_fwd_chunk(Q, K, V, cu_q, cu_k, qo, ko, out=o, lse=lse, workspace=ws,
                                     stream=s)
        except gpu_lib.CpattnError as e:
            err = e
        finally:
            graph.capture_end()
    torch.cuda.synchronize()
    assert err is not None and err.status == 2 and "captur" in str(err)
    # the library is unaffected: an ordinary call still matches the oracle
    o2, l2 = gpu_lib.cpattn_fwd_chunk(Q, K, V, cu_q, cu_k, qo, ko)
    torch.cuda.synchronize()
    check(host(o2), host(l2), *attention_ref(q, k, v, cu_q, cu_k, qo, ko), "bf16", "after capture")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_many_sequences_host_planned(gpu_lib, dtype):
    """200 short sequences in 3 chunks: metadata too large for the device planner, so the plan
    is built on the host and copied; all rows against the oracle."""
    rng = np.random.default_rng(17)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 200, 12, 4, 2, 64, dtype=dtype, min_len=1)
    dt = "bfloat16" if dtype == "bf16" else "float32"
    Q, K, V = dev(q, dt), dev(k, dt), dev(v, dt)
    # three chunks: cut every sequence's keys at two points
    cuts = [sorted(rng.integers(0, cu_k[i + 1] - cu_k[i] + 1, size=2).tolist()) for i in range(200)]
    ks, vs, cus, offs = [], [], [], []
    for c in range(3):
        rows, lens, off = [], [], []
        for i in range(200):
            b = [0] + cuts[i] + [int(cu_k[i + 1] - cu_k[i])]
            rows.append(np.arange(cu_k[i] + b[c], cu_k[i] + b[c + 1]))
            lens.append(b[c + 1] - b[c])
            off.append(int(ko[i]) + b[c])
        r = np.concatenate(rows).astype(np.int64)
        ks.append(K[r].contiguous()); vs.append(V[r].contiguous())
        cus.append(wl.cu_from_lengths(lens)); offs.append(np.array(off, np.int32))
    o, lse = gpu_lib.cpattn_fwd_chunks(Q, ks, vs, cu_q, cus, qo, offs)
    import torch
    torch.cuda.synchronize()
    check(host(o), host(lse), *attention_ref(q, k, v, cu_q, cu_k, qo, ko), dtype,
          f"200 sequences, host-planned ({dtype})")


def test_offsets_beyond_32_bits(gpu_lib):
    """A 132 x 4,096-token pack at 32/8 heads, D = 128: O holds 2.2e9 elements (8.9 GB, byte
    offsets past 2^32) and the plan is built on the host (16,896 tiles).  Inputs are drawn on the
    device from a seeded generator; rows at the start and end of the last sequence (the highest
    offsets) are checked against the oracle, and the merge of the result with itself at that size
    against its closed form (the same O, LSE + ln 2)."""
    import math

    import torch
    nseq, ln, hq, hkv, d = 132, 4096, 32, 8, 128
    t = nseq * ln
    assert t * hq * d > 2**31
    gen = torch.Generator(device="cuda").manual_seed(2024)
    q = torch.randn((t, hq, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    k = torch.randn((t, hkv, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    v = torch.randn((t, hkv, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    cu = np.arange(0, t + 1, ln, dtype=np.int32)
    o, lse = gpu_lib.cpattn_fwd_chunk(q, k, v, cu, cu)
    torch.cuda.synchronize()
    s0 = t - ln   # first token of the last sequence
    ks, vs = host(k[s0:]), host(v[s0:])
    for lo in (0, ln - 64):   # the sequence's first and last 64 rows
        rows = slice(s0 + lo, s0 + lo + 64)
        o_ref, l_ref = attention_ref(host(q[rows]), ks, vs, [0, 64], [0, ln], [lo], [0], True)
        check(host(o[rows]), host(lse[:, rows]), o_ref, l_ref, "bf16", f"offsets > 2^32, rows {lo}..")
    del q, k, v
    o_keep, l_keep = o[s0:].clone(), lse[:, s0:].clone()
    gpu_lib.cpattn_merge(o, lse, o.clone(), lse.clone())
    torch.cuda.synchronize()
    assert torch.allclose(o[s0:], o_keep, rtol=1e-6, atol=1e-7), "merge with itself moved O"
    assert torch.allclose(lse[:, s0:], l_keep + math.log(2.0), rtol=0, atol=2e-6), "LSE + ln 2"
