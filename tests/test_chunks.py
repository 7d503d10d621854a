"""GPU tests of the multi-chunk and accumulating entry points.

cpattn_fwd_chunks (all chunks of a share in one launch, the online softmax
carried across chunks) and cpattn_fwd_chunk_accum (a chunk's partial folded into
a running result in the kernel epilogue) against the fp64 oracle, plus the
exactness properties the header promises: one chunk through cpattn_fwd_chunks is
cpattn_fwd_chunk bit for bit, accumulating into an empty result (LSE = -inf)
gives the plain partial bit for bit, and rows a chunk shows no key keep their
values bit for bit.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import attention_ref, share_ref
from parity_util import check, dev, host

pytestmark = pytest.mark.gpu


def _split(rng, k, v, cu_k, ko, nchunks, min_empty=False):
    """Cut every sequence's keys into nchunks contiguous pieces (some may be empty)."""
    nseq = len(cu_k) - 1
    cuts = [sorted(rng.integers(0, cu_k[i + 1] - cu_k[i] + 1, size=nchunks - 1).tolist())
            for i in range(nseq)]
    rows, cus, offs = [], [], []
    for c in range(nchunks):
        r, lens, off = [], [], []
        for i in range(nseq):
            b = [0] + cuts[i] + [int(cu_k[i + 1] - cu_k[i])]
            r.append(np.arange(cu_k[i] + b[c], cu_k[i] + b[c + 1]))
            lens.append(b[c + 1] - b[c])
            off.append(int(ko[i]) + b[c])
        rows.append(np.concatenate(r).astype(np.int64) if r else np.zeros(0, np.int64))
        cus.append(wl.cu_from_lengths(lens))
        offs.append(np.array(off, np.int32))
    return rows, cus, offs


def _tdt(dtype):
    return "bfloat16" if dtype == "bf16" else "float32"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("nchunks", [1, 2, 3, 8, 16])
def test_fwd_chunks_equals_unsplit_attention(gpu_lib, dtype, nchunks):
    import torch
    rng = np.random.default_rng(100 + nchunks)
    hq, hkv = (32, 8) if dtype == "bf16" else (4, 2)
    for trial in range(3):
        q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 4, 400, hq, hkv, 128, dtype=dtype,
                                                     min_len=1)
        rows, cus, offs = _split(rng, k, v, cu_k, ko, nchunks)
        dt = _tdt(dtype)
        Q = dev(q, dt)
        ks = [dev(k[r], dt) for r in rows]
        vs = [dev(v[r], dt) for r in rows]
        tq = int(cu_q[-1])
        o = torch.full((tq, hq, 128), float("nan"), device="cuda")
        lse = torch.full((hq, tq), float("nan"), device="cuda")
        gpu_lib.cpattn_fwd_chunks(Q, ks, vs, cu_q, cus, qo, offs, True, out=o, lse=lse)
        torch.cuda.synchronize()
        check(host(o), host(lse), *attention_ref(q, k, v, cu_q, cu_k, qo, ko, True), dtype,
              f"{nchunks} chunks, trial {trial}")


def test_one_chunk_stream_is_fwd_chunk_bitwise(gpu_lib):
    import torch
    rng = np.random.default_rng(7)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 5, 700, 32, 8, 128, dtype="bf16", min_len=1)
    Q, K, V = dev(q, "bfloat16"), dev(k, "bfloat16"), dev(v, "bfloat16")
    o1, l1 = gpu_lib.cpattn_fwd_chunk(Q, K, V, cu_q, cu_k, qo, ko)
    o2, l2 = gpu_lib.cpattn_fwd_chunks(Q, [K], [V], cu_q, [cu_k], qo, [ko])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_accumulate_exactness(gpu_lib, dtype):
    """Into an empty result: the plain partial, bitwise.  A chunk wholly after the
    queries (no visible key anywhere): the running result untouched, bitwise."""
    import torch
    rng = np.random.default_rng(11)
    hq, hkv = (8, 2)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 3, 300, hq, hkv, 64, dtype=dtype, min_len=1)
    dt = _tdt(dtype)
    Q, K, V = dev(q, dt), dev(k, dt), dev(v, dt)
    tq = int(cu_q[-1])
    o_ref, l_ref = gpu_lib.cpattn_fwd_chunk(Q, K, V, cu_q, cu_k, qo, ko)
    o = torch.zeros((tq, hq, 64), device="cuda")
    lse = torch.full((hq, tq), float("-inf"), device="cuda")
    gpu_lib.cpattn_fwd_chunk_accum(Q, K, V, cu_q, cu_k, qo, ko, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    # a chunk placed after every query: nothing visible, result unchanged
    o_before = torch.randn((tq, hq, 64), device="cuda")
    l_before = torch.randn((hq, tq), device="cuda")
    o, lse = o_before.clone(), l_before.clone()
    far = (np.asarray(qo) + 10_000).astype(np.int32)
    gpu_lib.cpattn_fwd_chunk_accum(Q, K, V, cu_q, cu_k, qo, far, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_before) and torch.equal(lse, l_before)
    # same through the multi-chunk entry point with accumulate=True
    gpu_lib.cpattn_fwd_chunks(Q, [K, K], [V, V], cu_q, [cu_k, cu_k], qo, [far, far + 1],
                              accumulate=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_before) and torch.equal(lse, l_before)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_accumulate_chain_and_streamed_halves(gpu_lib, dtype):
    """Per-chunk epilogue accumulation, and two multi-chunk launches where the second
    accumulates, both equal unsplit attention."""
    import torch
    rng = np.random.default_rng(12)
    hq, hkv = (16, 4) if dtype == "bf16" else (4, 4)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 4, 500, hq, hkv, 128, dtype=dtype, min_len=1)
    rows, cus, offs = _split(rng, k, v, cu_k, ko, 6)
    dt = _tdt(dtype)
    Q = dev(q, dt)
    ks = [dev(k[r], dt) for r in rows]
    vs = [dev(v[r], dt) for r in rows]
    ref = attention_ref(q, k, v, cu_q, cu_k, qo, ko, True)
    tq = int(cu_q[-1])
    o = torch.zeros((tq, hq, 128), device="cuda")
    lse = torch.full((hq, tq), float("-inf"), device="cuda")
    for c in range(6):
        gpu_lib.cpattn_fwd_chunk_accum(Q, ks[c], vs[c], cu_q, cus[c], qo, offs[c], out=o, lse=lse)
    torch.cuda.synchronize()
    check(host(o), host(lse), *ref, dtype, "accumulate chain")
    o2, l2 = gpu_lib.cpattn_fwd_chunks(Q, ks[:4], vs[:4], cu_q, cus[:4], qo, offs[:4])
    gpu_lib.cpattn_fwd_chunks(Q, ks[4:], vs[4:], cu_q, cus[4:], qo, offs[4:], accumulate=True,
                              out=o2, lse=l2)
    torch.cuda.synchronize()
    check(host(o2), host(l2), *ref, dtype, "streamed halves")


def test_chunk_order_does_not_matter(gpu_lib):
    """The chunks of a share in ring order and reversed give the same result to rounding."""
    import torch
    w = wl.make("pack", 0)
    g = w.groups[0]
    rng = np.random.default_rng(3)
    rows, cus, offs = _split(rng, g.k_full, g.v_full, g.cu_full, np.zeros(len(g.cu_full) - 1, np.int32), 4)
    Q = dev(g.q, "bfloat16")
    ks = [dev(g.k_full[r], "bfloat16") for r in rows]
    vs = [dev(g.v_full[r], "bfloat16") for r in rows]
    ref = attention_ref(g.q, g.k_full, g.v_full, g.cu_q, g.cu_full, g.q_off,
                        np.zeros(len(g.cu_full) - 1, np.int32), True)
    a = gpu_lib.cpattn_fwd_chunks(Q, ks, vs, g.cu_q, cus, g.q_off, offs)
    torch.cuda.synchronize()
    check(host(a[0]), host(a[1]), *ref, "bf16", "ring order")
    b = gpu_lib.cpattn_fwd_chunks(Q, ks[::-1], vs[::-1], g.cu_q, cus[::-1], g.q_off, offs[::-1])
    torch.cuda.synchronize()
    check(host(b[0]), host(b[1]), *ref, "bf16", "reversed order")


def test_guard_bands_and_poisoned_outputs_multi_chunk(gpu_lib):
    """Every row written (NaN poison gone), nothing written past the outputs."""
    import torch
    rng = np.random.default_rng(13)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 6, 333, 32, 8, 128, dtype="bf16", min_len=0)
    rows, cus, offs = _split(rng, k, v, cu_k, ko, 5)
    Q = dev(q, "bfloat16")
    ks = [dev(k[r], "bfloat16") for r in rows]
    vs = [dev(v[r], "bfloat16") for r in rows]
    tq, hq, d = q.shape
    guard = 4096
    o_buf = torch.full((tq * hq * d + guard,), float("nan"), device="cuda")
    l_buf = torch.full((hq * tq + guard,), float("nan"), device="cuda")
    o_buf[tq * hq * d:] = 12345.0
    l_buf[hq * tq:] = 12345.0
    o = o_buf[:tq * hq * d].view(tq, hq, d)
    lse = l_buf[:hq * tq].view(hq, tq)
    gpu_lib.cpattn_fwd_chunks(Q, ks, vs, cu_q, cus, qo, offs, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o_buf[tq * hq * d:] == 12345.0) and torch.all(l_buf[hq * tq:] == 12345.0)
    check(host(o), host(lse), *attention_ref(q, k, v, cu_q, cu_k, qo, ko, True), "bf16", "guarded")


def test_cp4_share_stream_full_size_every_row_of_one_head(gpu_lib):
    """The benchmarked call (all four chunks in one launch) on every query row of head 0
    and head 31, against the oracle."""
    import torch
    w = wl.make("cp4_share", 0)
    g = w.groups[0]
    Q = dev(g.q, "bfloat16")
    ks = [dev(c.k, "bfloat16") for c in g.chunks]
    vs = [dev(c.v, "bfloat16") for c in g.chunks]
    o, lse = gpu_lib.cpattn_fwd_chunks(Q, ks, vs, g.cu_q, [c.cu_k for c in g.chunks], g.q_off,
                                       [c.k_off for c in g.chunks])
    torch.cuda.synchronize()
    o_h, l_h = host(o), host(lse)
    for head in (0, 31):
        sub = wl.Group(q=g.q[:, head:head + 1], cu_q=g.cu_q, q_off=g.q_off, chunks=[],
                       k_full=g.k_full[:, head // 4:head // 4 + 1],
                       v_full=g.v_full[:, head // 4:head // 4 + 1], cu_full=g.cu_full)
        o_ref, l_ref = share_ref(sub)
        check(o_h[:, head:head + 1], l_h[head:head + 1], o_ref, l_ref, "bf16", f"cp4 head {head}")


def test_repeated_calls_are_exact(gpu_lib):
    """Two different packs called alternately, 150 times each, with the outputs reused: every
    result is bitwise the first one of its pack (each call plans into its own workspace on the
    stream; nothing carries over between calls)."""
    import torch
    rng = np.random.default_rng(31)
    packs = []
    for _ in range(2):
        q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 5, 1200, 32, 8, 128, dtype="bf16", min_len=400)
        rows, cus, offs = _split(rng, k, v, cu_k, ko, 16)
        Q = dev(q, "bfloat16")
        ks = [dev(k[r], "bfloat16") for r in rows]
        vs = [dev(v[r], "bfloat16") for r in rows]
        o, lse = gpu_lib.cpattn_fwd_chunks(Q, ks, vs, cu_q, cus, qo, offs)
        torch.cuda.synchronize()
        packs.append((Q, ks, vs, cu_q, cus, qo, offs, o.clone(), lse.clone()))
    outs = [(torch.empty_like(p[7]), torch.empty_like(p[8])) for p in packs]
    for it in range(150):
        for (Q, ks, vs, cu_q, cus, qo, offs, o_ref, l_ref), (o, lse) in zip(packs, outs):
            gpu_lib.cpattn_fwd_chunks(Q, ks, vs, cu_q, cus, qo, offs, out=o, lse=lse)
        if it % 10 == 9:
            torch.cuda.synchronize()
            for p, (o, lse) in zip(packs, outs):
                assert torch.equal(o, p[7]) and torch.equal(lse, p[8]), f"call pair {it}"


def test_too_many_chunks_is_rejected(gpu_lib):
    import torch
    q = dev(np.ones((4, 2, 64), np.float32), "bfloat16")
    k = dev(np.ones((4, 2, 64), np.float32), "bfloat16")
    n = gpu_lib.MAX_CHUNKS + 1
    with pytest.raises(gpu_lib.CpattnError) as ei:
        gpu_lib.cpattn_fwd_chunks(q, [k] * n, [k] * n, [0, 4], [[0, 4]] * n)
    assert ei.value.status == 1
    torch.cuda.synchronize()
