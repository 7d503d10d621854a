"""GPU parity of the backward (cpattn_bwd_chunks, cpattn_bwd_chunk) against the fp64
oracle's gradients.

The forward runs on the GPU (one launch over all chunks, giving the share's O and
LSE), then the backward: one pass over all chunks, or (per_chunk) once per chunk
with dq accumulating over the calls and each call yielding that chunk's dk and dv.  The oracle differentiates the unsplit attention of
the share; dq is compared whole, dk / dv chunk by chunk against the oracle's rows
of that chunk's keys.

Tolerance (bf16 inputs, fp32 accumulation; not stated by the benchmark spec, derived here):
P and dS are rounded to bf16 before their products (each at most 2^-8 = 3.9e-3
relative, about 2^-9 on average, errors of both signs, so the relative L2 error of a
sum of many such terms sits near 2^-9), and the forward's fp32 O enters
delta = rowsum(dO * O) with the forward's own error.  The bar is the forward's
relative L2 bound, 5e-3 per gradient, plus a max-abs error of 1e-2 of the gradient's
largest magnitude (measured on the GPU: rel-L2 1.4-1.7e-3, max-abs 1.5-3.1e-3).
"""
import numpy as np
import pytest

import workloads as wl
from oracle import attention_bwd_ref, share_bwd_ref
from parity_util import GRAD_RECORD, dev, host

pytestmark = pytest.mark.gpu

BWD_REL_L2, BWD_MAX_REL = 5e-3, 1e-2


def check_grad(got, ref, what):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), f"non-finite gradient {what}"
    nrm = float(np.linalg.norm(ref))
    err = float(np.linalg.norm(got - ref))
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    worst = float(np.abs(got - ref).max()) if ref.size else 0.0
    if nrm == 0.0:
        assert worst <= 1e-6, f"{what}: expected zero gradient, max {worst:.3e}"
        return 0.0
    print(f"{what}: rel-L2 {err / nrm:.2e}, max-abs / max {worst / scale:.2e}")
    GRAD_RECORD.append((what, err / nrm, worst / scale))
    assert err / nrm <= BWD_REL_L2, f"{what}: rel-L2 {err / nrm:.3e} > {BWD_REL_L2}"
    assert worst <= BWD_MAX_REL * scale, f"{what}: max-abs {worst:.3e} > {BWD_MAX_REL} x {scale:.3e}"
    return err / nrm


def _split(rng, cu_k, ko, nchunks):
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


def _run(cra, q, k, v, do, cu_q, cu_k, qo, ko, causal, nchunks, rng, per_chunk=False):
    """GPU forward over the chunks, then the backward; returns dq and full-length dk, dv."""
    import torch
    rows, cus, offs = _split(rng, cu_k, ko, nchunks)
    Q, DO = dev(q, "bfloat16"), dev(do, "bfloat16")
    ks = [dev(k[r], "bfloat16") for r in rows]
    vs = [dev(v[r], "bfloat16") for r in rows]
    o, lse = cra.cpattn_fwd_chunks(Q, ks, vs, cu_q, cus, qo, offs, causal)
    dq, dks, dvs = cra.cpattn_share_bwd(Q, ks, vs, o, lse, DO, cu_q, cus, qo, offs, causal,
                                        per_chunk=per_chunk)
    torch.cuda.synchronize()
    dk = np.zeros(k.shape); dv = np.zeros(v.shape)
    for c, r in enumerate(rows):
        dk[r] = host(dks[c]); dv[r] = host(dvs[c])
    return host(dq), dk, dv


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 1, 128), (8, 2, 64), (4, 4, 64), (6, 3, 128)])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_random_packs(gpu_lib, hq, hkv, d, causal):
    rng = np.random.default_rng(hq * 31 + hkv * 7 + d + causal)
    for trial in range(2):
        q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 3, 300, hq, hkv, d, dtype="bf16",
                                                     min_len=1, k_extra=96)
        do = wl.round_to_bf16(rng.standard_normal(q.shape, dtype=np.float32))
        nch = int(rng.integers(1, 5))
        dq, dk, dv = _run(gpu_lib, q, k, v, do, cu_q, cu_k, qo, ko, causal, nch, rng)
        rq, rk, rv = attention_bwd_ref(q, k, v, do, cu_q, cu_k, qo, ko, causal)
        what = f"{hq}/{hkv} d={d} causal={causal} trial {trial} ({nch} chunks)"
        check_grad(dq, rq, "dq " + what)
        check_grad(dk, rk, "dk " + what)
        check_grad(dv, rv, "dv " + what)


def test_backward_empty_rows_and_sequences(gpu_lib):
    """Empty sequences, queries before every key (LSE = -inf rows), a chunk after every query:
    those rows and keys get exactly zero gradient, the rest match the oracle."""
    import torch
    rng = np.random.default_rng(5)
    lens_q, lens_k = [0, 40, 70, 1, 33], [10, 0, 90, 5, 64]
    cu_q, cu_k = wl.cu_from_lengths(lens_q), wl.cu_from_lengths(lens_k)
    qo = np.array([0, 0, 10, 0, 0], np.int32)
    ko = np.array([0, 0, 30, 0, 40], np.int32)      # sequence 2: rows 0-19 see nothing
    q = wl.round_to_bf16(rng.standard_normal((int(cu_q[-1]), 8, 128), dtype=np.float32))
    k = wl.round_to_bf16(rng.standard_normal((int(cu_k[-1]), 2, 128), dtype=np.float32))
    v = wl.round_to_bf16(rng.standard_normal((int(cu_k[-1]), 2, 128), dtype=np.float32))
    do = wl.round_to_bf16(rng.standard_normal(q.shape, dtype=np.float32))
    dq, dk, dv = _run(gpu_lib, q, k, v, do, cu_q, cu_k, qo, ko, True, 2, rng)
    rq, rk, rv = attention_bwd_ref(q, k, v, do, cu_q, cu_k, qo, ko, True)
    check_grad(dq, rq, "dq"); check_grad(dk, rk, "dk"); check_grad(dv, rv, "dv")
    assert np.all(dq[cu_q[2]:cu_q[2] + 20] == 0.0)            # rows with no visible key
    assert np.all(dk[cu_k[4]:] == 0.0) and np.all(dv[cu_k[4]:] == 0.0)  # keys after every query
    torch.cuda.synchronize()


def test_backward_accumulates_and_is_deterministic(gpu_lib):
    import torch
    rng = np.random.default_rng(9)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 3, 200, 16, 4, 128, dtype="bf16", min_len=1)
    do = wl.round_to_bf16(rng.standard_normal(q.shape, dtype=np.float32))
    Q, K, V, DO = (dev(x, "bfloat16") for x in (q, k, v, do))
    o, lse = gpu_lib.cpattn_fwd_chunk(Q, K, V, cu_q, cu_k, qo, ko)
    a = gpu_lib.cpattn_bwd_chunk(Q, K, V, o, lse, DO, cu_q, cu_k, qo, ko)
    b = gpu_lib.cpattn_bwd_chunk(Q, K, V, o, lse, DO, cu_q, cu_k, qo, ko)
    twice = gpu_lib.cpattn_bwd_chunk(Q, K, V, o, lse, DO, cu_q, cu_k, qo, ko,
                                     dq=a[0].clone(), dk=a[1].clone(), dv=a[2].clone())
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, twice):
        assert torch.equal(x, y)                      # deterministic: no atomics
        assert torch.equal(z, x + y)                  # adds into the given buffers


@pytest.mark.parametrize("kvh", [0, 5])
def test_backward_cp4_share_full_size(gpu_lib, kvh):
    """The benchmarked share at full size (all heads on the GPU); the oracle differentiates
    one GQA group (query heads 4 kvh .. 4 kvh + 3 and kv head kvh), for the first group and
    one from the other half of the heads."""
    import torch
    w = wl.make("cp4_share", 0)
    g = w.groups[0]
    rng = np.random.default_rng(77)
    do = wl.round_to_bf16(rng.standard_normal(g.q.shape, dtype=np.float32))
    Q, DO = dev(g.q, "bfloat16"), dev(do, "bfloat16")
    ks = [dev(c.k, "bfloat16") for c in g.chunks]
    vs = [dev(c.v, "bfloat16") for c in g.chunks]
    cus = [c.cu_k for c in g.chunks]
    offs = [c.k_off for c in g.chunks]
    o, lse = gpu_lib.cpattn_fwd_chunks(Q, ks, vs, g.cu_q, cus, g.q_off, offs)
    hs = slice(4 * kvh, 4 * kvh + 4)
    sub = wl.Group(q=g.q[:, hs], cu_q=g.cu_q, q_off=g.q_off, chunks=[],
                   k_full=g.k_full[:, kvh:kvh + 1], v_full=g.v_full[:, kvh:kvh + 1], cu_full=g.cu_full)
    rq, rk, rv = share_bwd_ref(sub, do[:, hs])
    lengths = np.diff(g.cu_full)
    # one pass over all chunks, then the ring's order (one call per chunk, dq accumulating)
    for per_chunk in (False, True):
        dq, dks, dvs = gpu_lib.cpattn_share_bwd(Q, ks, vs, o, lse, DO, g.cu_q, cus, g.q_off, offs,
                                                per_chunk=per_chunk)
        torch.cuda.synchronize()
        how = f"kv head {kvh}, " + ("per chunk" if per_chunk else "one pass")
        check_grad(host(dq)[:, hs], rq, f"cp4 dq ({how})")
        # chunk c holds piece c of every sequence: map the oracle's full-sequence key rows
        for c, ch in enumerate(g.chunks):
            rows = np.concatenate([np.arange(g.cu_full[i] + int(ch.k_off[i]),
                                             g.cu_full[i] + int(ch.k_off[i]) + int(ch.cu_k[i + 1] - ch.cu_k[i]))
                                   for i in range(len(lengths))])
            check_grad(host(dks[c])[:, kvh:kvh + 1], rk[rows], f"cp4 dk chunk {c} ({how})")
            check_grad(host(dvs[c])[:, kvh:kvh + 1], rv[rows], f"cp4 dv chunk {c} ({how})")


def test_backward_ctx128k_share_full_size(gpu_lib):
    """The 128K share (one sequence, 32768 queries at offset 98304, 4 key chunks of 32768,
    8 query heads on one kv head) at full size, in the benchmark's launch configuration.

    The oracle cannot differentiate the whole share in seconds, so it checks what it can
    compute exactly, and identities of the gradient cover the rest:
      * the last 160 queries are the only ones that see the last 160 keys: the oracle's
        backward over those queries (each against all its keys) gives their dq and those
        keys' dk, dv exactly (one full key tile and part of the one before);
      * dq of a few more rows, each from the oracle's backward over that row alone;
      * each row's softmax sums to one, so the dv of all keys sums to the dO of all rows
        and query heads; the dS of a row sums to zero (delta is rowsum(P * dP)), so the dk
        of all keys sums to zero.
    Tolerance of the identities: rounding P and dS to bf16 leaves each row's sums off by
    about 2^-9 of a row's single terms, which over 2^18 (row, head) pairs adds up to about
    1e-5 of |sum dO| for dv and about 3e-3 of |dk| for dk; the bars are 1e-3 and 3e-2
    (leaving delta out of dS gives a dk sum larger than |dk|).
    """
    import torch
    w = wl.make("ctx128k_share", 0)
    g = w.groups[0]
    assert len(g.cu_q) == 2 and g.k_full.shape[1] == 1
    rng = np.random.default_rng(128)
    do = wl.round_to_bf16(rng.standard_normal(g.q.shape, dtype=np.float32))
    Q, DO = dev(g.q, "bfloat16"), dev(do, "bfloat16")
    ks = [dev(c.k, "bfloat16") for c in g.chunks]
    vs = [dev(c.v, "bfloat16") for c in g.chunks]
    cus = [c.cu_k for c in g.chunks]
    offs = [c.k_off for c in g.chunks]
    o, lse = gpu_lib.cpattn_fwd_chunks(Q, ks, vs, g.cu_q, cus, g.q_off, offs)
    dq, dks, dvs = gpu_lib.cpattn_share_bwd(Q, ks, vs, o, lse, DO, g.cu_q, cus, g.q_off, offs)
    torch.cuda.synchronize()
    dq = host(dq)
    dk = np.zeros(g.k_full.shape); dv = np.zeros(g.v_full.shape)
    for c, ch in enumerate(g.chunks):
        a = int(ch.k_off[0])
        dk[a:a + ch.k.shape[0]] = host(dks[c]); dv[a:a + ch.k.shape[0]] = host(dvs[c])
    tq, nk, q0 = g.q.shape[0], g.k_full.shape[0], int(g.q_off[0])
    assert q0 + tq == nk
    # the last m queries and the last m keys
    m = 160
    kk = np.array([0, nk], np.int64)
    rq, rk, rv = attention_bwd_ref(g.q[tq - m:], g.k_full, g.v_full, do[tq - m:], [0, m], kk,
                                   [q0 + tq - m], [0], True)
    check_grad(dq[tq - m:], rq, "128k dq, last rows")
    check_grad(dk[nk - m:], rk[nk - m:], "128k dk, last keys")
    check_grad(dv[nk - m:], rv[nk - m:], "128k dv, last keys")
    for t in [0, 1, 127, 128, 16383] + sorted(int(x) for x in rng.integers(0, tq - m, size=27)):
        rq1, _, _ = attention_bwd_ref(g.q[t:t + 1], g.k_full, g.v_full, do[t:t + 1], [0, 1], kk,
                                      [q0 + t], [0], True)
        check_grad(dq[t:t + 1], rq1, f"128k dq row {t}")
    # identities over all keys
    sum_do = do.astype(np.float64).sum(axis=(0, 1))
    sum_dv = dv.sum(axis=(0, 1))
    rel_v = float(np.linalg.norm(sum_dv - sum_do) / np.linalg.norm(sum_do))
    rel_k = float(np.linalg.norm(dk.sum(axis=(0, 1))) / np.linalg.norm(dk))
    print(f"128k identities: |sum dv - sum dO| / |sum dO| {rel_v:.2e}, |sum dk| / |dk| {rel_k:.2e}")
    assert rel_v <= 1e-3, f"dv does not sum to the rows' dO: {rel_v:.3e}"
    assert rel_k <= 3e-2, f"dk does not sum to zero: {rel_k:.3e}"


def test_backward_rejects_fp32(gpu_lib):
    import torch
    q = torch.zeros((4, 2, 64), device="cuda")
    lse = torch.zeros((2, 4), device="cuda")
    with pytest.raises(gpu_lib.CpattnError) as ei:
        gpu_lib.cpattn_bwd_chunk(q, q, q, q, lse, q, [0, 4], [0, 4])
    assert ei.value.status == 2


@pytest.mark.parametrize("per_chunk", [False, True])
@pytest.mark.parametrize("nchunks", [1, 3, 8, 16])
def test_backward_chunk_counts_both_schedules(gpu_lib, nchunks, per_chunk):
    rng = np.random.default_rng(300 + nchunks)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 4, 260, 16, 4, 128, dtype="bf16",
                                                 min_len=1, k_extra=64)
    do = wl.round_to_bf16(rng.standard_normal(q.shape, dtype=np.float32))
    dq, dk, dv = _run(gpu_lib, q, k, v, do, cu_q, cu_k, qo, ko, True, nchunks, rng, per_chunk)
    rq, rk, rv = attention_bwd_ref(q, k, v, do, cu_q, cu_k, qo, ko, True)
    what = f"{nchunks} chunks, per_chunk={per_chunk}"
    check_grad(dq, rq, "dq " + what)
    check_grad(dk, rk, "dk " + what)
    check_grad(dv, rv, "dv " + what)


def test_backward_too_many_chunks_is_rejected(gpu_lib):
    import torch
    q = dev(np.ones((4, 2, 64), np.float32), "bfloat16")
    o = torch.zeros((4, 2, 64), device="cuda")
    lse = torch.zeros((2, 4), device="cuda")
    n = gpu_lib.MAX_CHUNKS + 1
    with pytest.raises(gpu_lib.CpattnError) as ei:
        gpu_lib.cpattn_bwd_chunks(q, [q] * n, [q] * n, o, lse, q, [0, 4], [[0, 4]] * n)
    assert ei.value.status == 1


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 2, 64)])
def test_backward_key_tile_edges(gpu_lib, hq, hkv, d):
    """Key counts one below, at and one above the dK/dV kernel's 16-key tiles, its 48-key wave
    pairs and its 96-key work-group tiles, with the causal diagonal crossing those boundaries
    (queries offset so that a sequence's first query sees a few keys of a tile) and query counts
    around its 32-query blocks."""
    rng = np.random.default_rng(11 + d)
    lens_k = [15, 16, 17, 47, 48, 49, 95, 96, 97, 143, 193]
    lens_q = [31, 32, 33, 40, 64, 65, 96, 97, 100, 130, 161]
    qo = np.array([0, 3, 16, 20, 47, 1, 60, 0, 90, 15, 100], np.int32)
    ko = np.zeros(len(lens_k), np.int32)
    cu_q, cu_k = wl.cu_from_lengths(lens_q), wl.cu_from_lengths(lens_k)
    q = wl.round_to_bf16(rng.standard_normal((int(cu_q[-1]), hq, d), dtype=np.float32))
    k = wl.round_to_bf16(rng.standard_normal((int(cu_k[-1]), hkv, d), dtype=np.float32))
    v = wl.round_to_bf16(rng.standard_normal((int(cu_k[-1]), hkv, d), dtype=np.float32))
    do = wl.round_to_bf16(rng.standard_normal(q.shape, dtype=np.float32))
    for causal in (True, False):
        dq, dk, dv = _run(gpu_lib, q, k, v, do, cu_q, cu_k, qo, ko, causal, 1, rng)
        rq, rk, rv = attention_bwd_ref(q, k, v, do, cu_q, cu_k, qo, ko, causal)
        what = f"key-tile edges {hq}/{hkv} d={d} causal={causal}"
        check_grad(dq, rq, "dq " + what)
        check_grad(dk, rk, "dk " + what)
        check_grad(dv, rv, "dv " + what)


def test_backward_split_key_tiles_match_and_repeat_bitwise(gpu_lib):
    """Sequences long enough that the dK/dV launch splits its longest key tiles between two
    work-groups (half of each GQA group's query heads each, the second to finish adding the
    two partials): gradients match the oracle, and a second run gives the same bits whichever
    half finishes second.  The workspace is filled with NaN before each run, so a partial read
    before the other half's writes were visible would poison the result."""
    import torch
    rng = np.random.default_rng(21)
    lens = [3000, 700]          # with 16 query heads per kv head, the first ten key tiles of
    cu = wl.cu_from_lengths(lens)   # sequence 0 have >= 1,024 (query block, head) steps
    hq, hkv, d = 16, 1, 64
    q = wl.round_to_bf16(rng.standard_normal((int(cu[-1]), hq, d), dtype=np.float32))
    k = wl.round_to_bf16(rng.standard_normal((int(cu[-1]), hkv, d), dtype=np.float32))
    v = wl.round_to_bf16(rng.standard_normal((int(cu[-1]), hkv, d), dtype=np.float32))
    do = wl.round_to_bf16(rng.standard_normal(q.shape, dtype=np.float32))
    zeros = np.zeros(len(lens), np.int32)
    Q, K, V, DO = dev(q, "bfloat16"), dev(k, "bfloat16"), dev(v, "bfloat16"), dev(do, "bfloat16")
    o, lse = gpu_lib.cpattn_fwd_chunks(Q, [K], [V], cu, [cu], zeros, [zeros], True)
    nbytes = gpu_lib.cpattn_bwd_workspace_size_chunks(len(lens), cu, [cu], hq, hkv, d)
    runs = []
    for _ in range(2):
        ws = torch.full(((nbytes + 3) // 4,), float("nan"), dtype=torch.float32, device="cuda")
        dq, dks, dvs = gpu_lib.cpattn_bwd_chunks(Q, [K], [V], o, lse, DO, cu, [cu], zeros,
                                                 [zeros], True, workspace=ws)
        torch.cuda.synchronize()
        runs.append((host(dq), host(dks[0]), host(dvs[0])))
        del ws
    rq, rk, rv = attention_bwd_ref(q, k, v, do, cu, cu, zeros, zeros, True)
    check_grad(runs[0][0], rq, "dq split tiles")
    check_grad(runs[0][1], rk, "dk split tiles")
    check_grad(runs[0][2], rv, "dv split tiles")
    for a, b in zip(runs[0], runs[1]):
        assert np.array_equal(a, b)


def test_backward_offsets_beyond_32_bits(gpu_lib):
    """A 132 x 4,096-token pack at 32/8 heads, D = 128 (O, dQ: 2.2e9 elements, 8.9 GB each),
    inputs drawn on the device from a seeded generator.  The last 64 queries of the last sequence
    are the only ones that see its last 64 keys (causal), so the oracle on those 64 rows gives
    their dq exactly and the complete dk, dv of those keys: the highest offsets of every
    gradient."""
    import torch
    nseq, ln, hq, hkv, d = 132, 4096, 32, 8, 128
    t = nseq * ln
    assert t * hq * d > 2**31
    gen = torch.Generator(device="cuda").manual_seed(2025)
    q = torch.randn((t, hq, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    k = torch.randn((t, hkv, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    v = torch.randn((t, hkv, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    do = torch.randn((t, hq, d), generator=gen, device="cuda", dtype=torch.bfloat16)
    cu = np.arange(0, t + 1, ln, dtype=np.int32)
    o, lse = gpu_lib.cpattn_fwd_chunk(q, k, v, cu, cu)
    dq, dk, dv = gpu_lib.cpattn_bwd_chunk(q, k, v, o, lse, do, cu, cu)
    torch.cuda.synchronize()
    s0, lo = t - ln, ln - 64
    rows = slice(s0 + lo, t)
    dq_r, dk_r, dv_r = attention_bwd_ref(host(q[rows]), host(k[s0:]), host(v[s0:]), host(do[rows]),
                                         [0, 64], [0, ln], [lo], [0], True)
    check_grad(host(dq[rows]), dq_r, "dq, offsets > 2^32")
    check_grad(host(dk[rows]), dk_r[lo:], "dk, offsets > 2^32")
    check_grad(host(dv[rows]), dv_r[lo:], "dv, offsets > 2^32")
