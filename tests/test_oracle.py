"""Pins for the CPU fp64 oracle, against things other than the oracle itself.

Each test fixes the oracle to something the pages or the mathematics determine:
  * brute force: an independent scalar implementation on tiny packs;
  * closed forms: zero keys, constant values, one-hot values, single visible key,
    a dominating score, and a two-key score with a known softmax;
  * a library routine: torch's scaled_dot_product_attention (float64, CPU) with an
    explicit boolean mask, including its own GQA head grouping;
  * invariants from the ring-attention description in the "Megatron 6D
    parallelism guide" (section 6): merging any split of the keys gives the
    unsplit result, whatever the order of the chunks; an empty chunk changes
    nothing; sequences in one pack never see each other.
A plausible slip in the oracle (a dropped scale, the mask off by one or
reversed, a wrong GQA mapping, K and V swapped, a wrong merge weight) breaks at
least one of these.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import attention_ref, merge_ref, visible_pairs_ref, flops_ref, share_ref
import workloads as wl


# ----------------------------------------------------------------------------
# an independent scalar implementation (pure Python loops, math.fsum)
# ----------------------------------------------------------------------------
def brute_attention(q, k, v, cu_q, cu_k, q_off, k_off, causal):
    tq, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -math.inf)
    for i in range(len(cu_q) - 1):
        for t in range(int(cu_q[i]), int(cu_q[i + 1])):
            qpos = int(q_off[i]) + (t - int(cu_q[i]))
            for h in range(hq):
                g = h // group
                keys = []
                for u in range(int(cu_k[i]), int(cu_k[i + 1])):
                    kpos = int(k_off[i]) + (u - int(cu_k[i]))
                    if (not causal) or kpos <= qpos:
                        keys.append(u)
                if not keys:
                    continue
                sc = [math.fsum(float(q[t, h, j]) * float(k[u, g, j]) for j in range(d)) / math.sqrt(d)
                      for u in keys]
                top = max(sc)
                w = [math.exp(s - top) for s in sc]
                z = math.fsum(w)
                for j in range(d):
                    out[t, h, j] = math.fsum(wi * float(v[u, g, j]) for wi, u in zip(w, keys)) / z
                lse[h, t] = top + math.log(z)
    return out, lse


def _rand_pack(seed, nseq, max_len, hq, hkv, d, min_len=0):
    rng = np.random.default_rng(seed)
    return wl.random_pack(rng, nseq, max_len, hq, hkv, d, dtype="fp32", min_len=min_len)


def _close(a, b, tol):
    a = np.asarray(a); b = np.asarray(b)
    assert a.shape == b.shape
    fin = np.isfinite(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    if fin.any():
        assert np.max(np.abs(a[fin] - b[fin])) <= tol, np.max(np.abs(a[fin] - b[fin]))


@settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2**31 - 1), nseq=st.integers(0, 4), max_len=st.integers(0, 12),
       hkv=st.sampled_from([1, 2]), group=st.sampled_from([1, 2]), d=st.sampled_from([1, 4, 8]),
       causal=st.booleans())
def test_matches_brute_force(seed, nseq, max_len, hkv, group, d, causal):
    hq = hkv * group
    q, k, v, cu_q, cu_k, qo, ko = _rand_pack(seed, nseq, max_len, hq, hkv, d)
    o_ref, l_ref = attention_ref(q, k, v, cu_q, cu_k, qo, ko, causal)
    o_bf, l_bf = brute_attention(q, k, v, cu_q, cu_k, qo, ko, causal)
    _close(o_ref, o_bf, 1e-12)
    _close(l_ref, l_bf, 1e-12)


def test_tiny_workload_matches_brute_force_rows():
    """The tiny fp32 workload (one 256-token sequence, 2 heads, D=64) on sampled rows."""
    w = wl.make("tiny", 0)
    g = w.groups[0]
    rows = [0, 1, 63, 127, 128, 200, 255]
    o_ref, l_ref = share_ref(g, rows=rows)
    sub_q = g.q[rows]
    # brute force each sampled row as a 1-token sequence at its global position
    for j, r in enumerate(rows):
        o_b, l_b = brute_attention(sub_q[j:j + 1], g.k_full, g.v_full, [0, 1], [0, 256], [r], [0], True)
        _close(o_ref[j:j + 1], o_b, 1e-12)
        _close(l_ref[:, j:j + 1], l_b, 1e-12)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def test_zero_keys_average_visible_values():
    """K = 0: every visible score is 0, so O is the mean of the visible V and LSE = ln |U_t|."""
    rng = np.random.default_rng(1)
    nq, nk, d = 9, 13, 4
    q = rng.standard_normal((nq, 1, d)); k = np.zeros((nk, 1, d)); v = rng.standard_normal((nk, 1, d))
    q_off, k_off = 7, 3          # query t sees keys u with 3 + u <= 7 + t, i.e. u <= t + 4
    o, lse = attention_ref(q, k, v, [0, nq], [0, nk], [q_off], [k_off], True)
    for t in range(nq):
        n_vis = min(nk, t + 5)
        assert lse[0, t] == pytest.approx(math.log(n_vis), abs=1e-14)
        np.testing.assert_allclose(o[t, 0], v[:n_vis, 0].mean(axis=0), atol=1e-14)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(2)
    nq, nk, d = 6, 10, 8
    c = rng.standard_normal(d)
    q = rng.standard_normal((nq, 2, d)); k = rng.standard_normal((nk, 2, d))
    v = np.broadcast_to(c, (nk, 2, d)).copy()
    o, lse = attention_ref(q, k, v, [0, nq], [0, nk], [4], [0], True)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-13)


def test_one_hot_values_recover_the_softmax_row():
    """V = identity: O_t[u] is the probability of key u, which equals exp(s_u - LSE)."""
    rng = np.random.default_rng(3)
    nq, nk = 5, 8
    d = nk
    q = rng.standard_normal((nq, 1, d)); k = rng.standard_normal((nk, 1, d))
    v = np.eye(nk).reshape(nk, 1, d)
    o, lse = attention_ref(q, k, v, [0, nq], [0, nk], [2], [0], True)
    for t in range(nq):
        vis = np.arange(nk) <= t + 2
        s = (k[:, 0] @ q[t, 0]) / math.sqrt(d)
        np.testing.assert_allclose(o[t, 0].sum(), 1.0, atol=1e-14)
        np.testing.assert_allclose(o[t, 0][vis], np.exp(s[vis] - lse[0, t]), atol=1e-14)
        assert np.all(o[t, 0][~vis] == 0.0)


def test_single_visible_key():
    """A query that sees exactly one key returns that key's value; LSE is its score."""
    rng = np.random.default_rng(4)
    d = 16
    q = rng.standard_normal((1, 1, d)); k = rng.standard_normal((5, 1, d)); v = rng.standard_normal((5, 1, d))
    o, lse = attention_ref(q, k, v, [0, 1], [0, 5], [10], [10], True)
    np.testing.assert_allclose(o[0, 0], v[0, 0], atol=0)
    assert lse[0, 0] == pytest.approx(float(q[0, 0] @ k[0, 0]) / 4.0, abs=1e-14)


def test_two_keys_logistic_weight_pins_the_scale():
    """Scores a/sqrt(D) and 0 give weights sigmoid(a/sqrt(D)) and its complement."""
    d = 64
    a = 3.0
    q = np.zeros((1, 1, d)); q[0, 0, 0] = a
    k = np.zeros((2, 1, d)); k[0, 0, 0] = 1.0           # score a/8 ; key 1 scores 0
    v = np.zeros((2, 1, d)); v[0, 0, 1] = 1.0; v[1, 0, 2] = 1.0
    o, lse = attention_ref(q, k, v, [0, 1], [0, 2], [5], [0], True)
    w0 = 1.0 / (1.0 + math.exp(-a / 8.0))
    assert o[0, 0, 1] == pytest.approx(w0, abs=1e-15)
    assert o[0, 0, 2] == pytest.approx(1.0 - w0, abs=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(math.exp(a / 8.0) + 1.0), abs=1e-15)


def test_dominating_score_selects_its_value():
    d = 4
    q = np.array([[[10.0, 0, 0, 0]]])
    k = np.zeros((3, 1, d)); k[1, 0, 0] = 100.0          # score 500 against 0, 0
    v = np.arange(12, dtype=float).reshape(3, 1, d)
    o, _ = attention_ref(q, k, v, [0, 1], [0, 3], [2], [0], True)
    np.testing.assert_allclose(o[0, 0], v[1, 0], atol=1e-12)


def test_empty_rows_are_zero_and_minus_inf():
    """Queries before the chunk's first key, and empty sequences, give (0, -inf)."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 2, 8)); k = rng.standard_normal((3, 1, 8)); v = rng.standard_normal((3, 1, 8))
    cu_q = [0, 0, 4, 4]; cu_k = [0, 2, 2, 3]      # seq0: no queries; seq1: no keys; seq2: no queries
    o, lse = attention_ref(q, k, v, cu_q, cu_k, [0, 0, 0], [0, 0, 0], True)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    cu_k = [0, 0, 3, 3]
    o, lse = attention_ref(q, k, v, cu_q, cu_k, [0, 0, 0], [0, 2, 0], True)
    assert np.all(np.isneginf(lse[:, :2])) and np.all(o[:2] == 0)      # positions 0,1 < 2
    assert np.all(np.isfinite(lse[:, 2:]))


# ----------------------------------------------------------------------------
# torch's scaled_dot_product_attention as an independent library routine
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed,hq,hkv,d,causal", [(0, 4, 2, 16, True), (1, 8, 1, 32, True),
                                                   (2, 2, 2, 8, False), (3, 6, 3, 4, True)])
def test_matches_torch_sdpa(seed, hq, hkv, d, causal):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    q, k, v, cu_q, cu_k, qo, ko = _rand_pack(seed, 3, 40, hq, hkv, d, min_len=1)
    o_ref, _ = attention_ref(q, k, v, cu_q, cu_k, qo, ko, causal)
    for i in range(3):
        qs = torch.from_numpy(np.asarray(q[cu_q[i]:cu_q[i + 1]], np.float64)).permute(1, 0, 2)
        ks = torch.from_numpy(np.asarray(k[cu_k[i]:cu_k[i + 1]], np.float64)).permute(1, 0, 2)
        vs = torch.from_numpy(np.asarray(v[cu_k[i]:cu_k[i + 1]], np.float64)).permute(1, 0, 2)
        nq, nk = qs.shape[1], ks.shape[1]
        if causal:
            mask = (ko[i] + torch.arange(nk))[None, :] <= (qo[i] + torch.arange(nq))[:, None]
        else:
            mask = torch.ones(nq, nk, dtype=torch.bool)
        rows = mask.any(dim=1)
        if not rows.any():
            continue
        out = F.scaled_dot_product_attention(qs[:, rows], ks.contiguous(), vs.contiguous(),
                                             attn_mask=mask[rows], enable_gqa=True)
        np.testing.assert_allclose(o_ref[cu_q[i]:cu_q[i + 1]][rows.numpy()],
                                   out.permute(1, 0, 2).numpy(), atol=1e-12)


def test_lse_matches_torch_logsumexp():
    torch = pytest.importorskip("torch")
    q, k, v, cu_q, cu_k, qo, ko = _rand_pack(11, 2, 30, 4, 2, 16, min_len=1)
    _, lse = attention_ref(q, k, v, cu_q, cu_k, qo, ko, True)
    for i in range(2):
        for h in range(4):
            qs = torch.tensor(q[cu_q[i]:cu_q[i + 1], h], dtype=torch.float64)
            ks = torch.tensor(k[cu_k[i]:cu_k[i + 1], h // 2], dtype=torch.float64)
            s = qs @ ks.T / math.sqrt(16)
            mask = (ko[i] + torch.arange(ks.shape[0]))[None, :] <= (qo[i] + torch.arange(qs.shape[0]))[:, None]
            want = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=1).numpy()
            _close(lse[h, cu_q[i]:cu_q[i + 1]], want, 1e-12)


# ----------------------------------------------------------------------------
# invariants of the method
# ----------------------------------------------------------------------------
def _split_keys(k, v, cu_k, k_off, cuts):
    """Split every sequence's keys at relative positions cuts[i] (list of increasing ints)."""
    nseq = len(cu_k) - 1
    n_chunks = len(cuts[0]) + 1
    out = []
    for c in range(n_chunks):
        rows, lens, offs = [], [], []
        for i in range(nseq):
            n = int(cu_k[i + 1] - cu_k[i])
            b = [0] + list(cuts[i]) + [n]
            lo, hi = min(b[c], n), min(b[c + 1], n)
            rows.append(np.arange(cu_k[i] + lo, cu_k[i] + hi))
            lens.append(hi - lo)
            offs.append(int(k_off[i]) + lo)
        r = np.concatenate(rows).astype(np.int64)
        out.append((k[r], v[r], wl.cu_from_lengths(lens), np.array(offs)))
    return out


@settings(max_examples=30, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), n_chunks=st.integers(1, 5), causal=st.booleans(),
       order=st.permutations(range(5)))
def test_any_split_merged_in_any_order_equals_unsplit(seed, n_chunks, causal, order):
    rng = np.random.default_rng(seed)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 3, 24, 4, 2, 8, dtype="fp32")
    cuts = []
    for i in range(3):
        n = int(cu_k[i + 1] - cu_k[i])
        cuts.append(sorted(rng.integers(0, n + 1, size=n_chunks - 1).tolist()))   # empty chunks allowed
    parts = _split_keys(k, v, cu_k, ko, cuts)
    o_full, l_full = attention_ref(q, k, v, cu_q, cu_k, qo, ko, causal)
    idx = [c for c in order if c < n_chunks]

    def chunk_attention(c):
        kc, vc, cuc, offc = parts[c]
        return attention_ref(q, kc, vc, cu_q, cuc, qo, offc, causal)

    o_acc, l_acc = chunk_attention(idx[0])
    for c in idx[1:]:
        o_acc, l_acc = merge_ref(o_acc, l_acc, *chunk_attention(c))
    _close(o_acc, o_full, 1e-12)
    _close(l_acc, l_full, 1e-12)


def test_merge_identity_commutative_associative():
    rng = np.random.default_rng(7)
    t, h, d = 5, 3, 4
    def part():
        o = rng.standard_normal((t, h, d)); l = rng.standard_normal((h, t)) * 3
        l[0, 1] = -np.inf; o[1, 0] = 0.0
        return o, l
    a, b, c = part(), part(), part()
    empty = (np.zeros((t, h, d)), np.full((h, t), -np.inf))
    for x in (a, b):
        o, l = merge_ref(*x, *empty)
        _close(o, x[0], 0); _close(l, x[1], 0)
        o, l = merge_ref(*empty, *x)
        _close(o, x[0], 0); _close(l, x[1], 0)
    o, l = merge_ref(*empty, *empty)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    ab, ba = merge_ref(*a, *b), merge_ref(*b, *a)
    _close(ab[0], ba[0], 1e-15); _close(ab[1], ba[1], 1e-15)
    ab_c = merge_ref(*merge_ref(*a, *b), *c)
    a_bc = merge_ref(*a, *merge_ref(*b, *c))
    _close(ab_c[0], a_bc[0], 1e-13); _close(ab_c[1], a_bc[1], 1e-13)
    # merged LSE is the log of the summed exponentials
    fin = np.isfinite(a[1]) & np.isfinite(b[1])
    np.testing.assert_allclose(ab[1][fin], np.logaddexp(a[1], b[1])[fin], atol=1e-14)
    # equal LSEs: the plain average, LSE + ln 2
    o, l = merge_ref(a[0], a[1], b[0], a[1])
    fin = np.isfinite(a[1])
    np.testing.assert_allclose(l[fin], (a[1] + math.log(2))[fin], atol=1e-14)
    np.testing.assert_allclose(o.transpose(1, 0, 2)[fin], (0.5 * (a[0] + b[0])).transpose(1, 0, 2)[fin],
                               atol=1e-14)


def test_pack_isolation_and_permutation():
    rng = np.random.default_rng(8)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 4, 20, 4, 2, 8, dtype="fp32", min_len=1)
    o, l = attention_ref(q, k, v, cu_q, cu_k, qo, ko, True)
    for i in range(4):
        oi, li = attention_ref(q[cu_q[i]:cu_q[i + 1]], k[cu_k[i]:cu_k[i + 1]], v[cu_k[i]:cu_k[i + 1]],
                               [0, cu_q[i + 1] - cu_q[i]], [0, cu_k[i + 1] - cu_k[i]], [qo[i]], [ko[i]], True)
        _close(oi, o[cu_q[i]:cu_q[i + 1]], 1e-13)
        _close(li, l[:, cu_q[i]:cu_q[i + 1]], 1e-13)
    perm = [2, 0, 3, 1]
    qr = np.concatenate([q[cu_q[i]:cu_q[i + 1]] for i in perm])
    kr = np.concatenate([k[cu_k[i]:cu_k[i + 1]] for i in perm])
    vr = np.concatenate([v[cu_k[i]:cu_k[i + 1]] for i in perm])
    cq = wl.cu_from_lengths([cu_q[i + 1] - cu_q[i] for i in perm])
    ck = wl.cu_from_lengths([cu_k[i + 1] - cu_k[i] for i in perm])
    op, lp = attention_ref(qr, kr, vr, cq, ck, qo[perm], ko[perm], True)
    _close(op, np.concatenate([o[cu_q[i]:cu_q[i + 1]] for i in perm]), 1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(9)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 2, 16, 8, 2, 8, dtype="fp32", min_len=1)
    o, l = attention_ref(q, k, v, cu_q, cu_k, qo, ko, True)
    k_rep = np.repeat(k, 4, axis=1); v_rep = np.repeat(v, 4, axis=1)      # head h uses kv head h // 4
    o2, l2 = attention_ref(q, k_rep, v_rep, cu_q, cu_k, qo, ko, True)
    _close(o, o2, 1e-13); _close(l, l2, 1e-13)


def test_row_subset_equals_full_rows():
    rng = np.random.default_rng(10)
    q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 3, 30, 4, 1, 8, dtype="fp32", min_len=1)
    o, l = attention_ref(q, k, v, cu_q, cu_k, qo, ko, True)
    rows = np.array(sorted(rng.choice(q.shape[0], size=min(9, q.shape[0]), replace=False)))
    o_s, l_s = attention_ref(q, k, v, cu_q, cu_k, qo, ko, True, rows=rows)
    _close(o_s, o[rows], 1e-13); _close(l_s, l[:, rows], 1e-13)   # BLAS blocking may differ


# ----------------------------------------------------------------------------
# work counting
# ----------------------------------------------------------------------------
def test_visible_pairs_by_brute_enumeration():
    rng = np.random.default_rng(12)
    for _ in range(20):
        q, k, v, cu_q, cu_k, qo, ko = wl.random_pack(rng, 3, 15, 1, 1, 1, dtype="fp32")
        want = 0
        for i in range(3):
            for t in range(cu_q[i + 1] - cu_q[i]):
                for u in range(cu_k[i + 1] - cu_k[i]):
                    want += int(ko[i] + u <= qo[i] + t)
        assert visible_pairs_ref(cu_q, cu_k, qo, ko, True) == want
        assert visible_pairs_ref(cu_q, cu_k, qo, ko, False) == sum(
            (cu_q[i + 1] - cu_q[i]) * (cu_k[i + 1] - cu_k[i]) for i in range(3))
    # a causal diagonal block of n tokens holds n(n+1)/2 pairs
    assert visible_pairs_ref([0, 100], [0, 100]) == 100 * 101 // 2
    assert flops_ref(32896, 2, 64) == 16_842_752          # tiny workload: 16.84 MFLOP


# ----------------------------------------------------------------------------
# backward: gradients of the same function
# ----------------------------------------------------------------------------
from oracle import attention_bwd_ref  # noqa: E402


@pytest.mark.parametrize("seed,hq,hkv,d,causal", [(0, 4, 2, 16, True), (1, 8, 1, 32, True),
                                                   (2, 2, 2, 8, False), (3, 6, 3, 4, True)])
def test_bwd_matches_torch_autograd(seed, hq, hkv, d, causal):
    """torch autograd through scaled_dot_product_attention (float64, explicit mask, its own
    GQA grouping) gives the same dq, dk, dv."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    q, k, v, cu_q, cu_k, qo, ko = _rand_pack(seed, 3, 40, hq, hkv, d, min_len=1)
    ko = np.minimum(ko, qo)           # every query sees at least the sequence's first key
    do = np.random.default_rng(seed + 50).standard_normal(q.shape)
    dq_ref, dk_ref, dv_ref = attention_bwd_ref(q, k, v, do, cu_q, cu_k, qo, ko, causal)
    for i in range(3):
        qs = torch.tensor(np.asarray(q[cu_q[i]:cu_q[i + 1]], np.float64).transpose(1, 0, 2),
                          requires_grad=True)
        ks = torch.tensor(np.asarray(k[cu_k[i]:cu_k[i + 1]], np.float64).transpose(1, 0, 2),
                          requires_grad=True)
        vs = torch.tensor(np.asarray(v[cu_k[i]:cu_k[i + 1]], np.float64).transpose(1, 0, 2),
                          requires_grad=True)
        nq, nk = qs.shape[1], ks.shape[1]
        if causal:
            mask = (int(ko[i]) + torch.arange(nk))[None, :] <= (int(qo[i]) + torch.arange(nq))[:, None]
        else:
            mask = torch.ones(nq, nk, dtype=torch.bool)
        out = F.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask, enable_gqa=True)
        dos = torch.tensor(np.asarray(do[cu_q[i]:cu_q[i + 1]]).transpose(1, 0, 2))
        (out * dos).sum().backward()
        np.testing.assert_allclose(dq_ref[cu_q[i]:cu_q[i + 1]], qs.grad.numpy().transpose(1, 0, 2),
                                   atol=1e-11)
        np.testing.assert_allclose(dk_ref[cu_k[i]:cu_k[i + 1]], ks.grad.numpy().transpose(1, 0, 2),
                                   atol=1e-11)
        np.testing.assert_allclose(dv_ref[cu_k[i]:cu_k[i + 1]], vs.grad.numpy().transpose(1, 0, 2),
                                   atol=1e-11)


def test_bwd_central_differences():
    """Each gradient entry against (L(x + e) - L(x - e)) / 2e of L = sum(O * dO), with O from
    the pinned forward, on a tiny pack with an empty row and a causal diagonal."""
    rng = np.random.default_rng(7)
    cu_q, cu_k = np.array([0, 3, 5]), np.array([0, 4, 7])
    qo, ko = np.array([1, 0]), np.array([0, 1])          # row 0 of sequence 1 sees no key
    hq, hkv, d = 2, 1, 3
    q = rng.standard_normal((5, hq, d)); k = rng.standard_normal((7, hkv, d))
    v = rng.standard_normal((7, hkv, d)); do = rng.standard_normal((5, hq, d))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, cu_q, cu_k, qo, ko, True)

    def loss(q_, k_, v_):
        o, _ = attention_ref(q_, k_, v_, cu_q, cu_k, qo, ko, True)
        return float(np.sum(o * do))

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            ap = [a.copy() for a in args]; am = [a.copy() for a in args]
            pos = "qkv".index(name)
            ap[pos] = xp; am[pos] = xm
            num[idx] = (loss(*ap) - loss(*am)) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, err_msg=name)
    assert np.all(dq[3] == 0.0)                         # the empty row has no gradient


def test_bwd_closed_forms():
    rng = np.random.default_rng(8)
    # one key per sequence: P = 1 for every row that sees it -> dq = dk = 0, dv = sum of dO
    cu_q, cu_k = np.array([0, 4]), np.array([0, 1])
    q = rng.standard_normal((4, 2, 8)); k = rng.standard_normal((1, 1, 8))
    v = rng.standard_normal((1, 1, 8)); do = rng.standard_normal((4, 2, 8))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, cu_q, cu_k, None, None, True)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[0, 0], do.sum(axis=(0, 1)), atol=1e-12)
    # identical value rows: O does not depend on the weights -> dq = dk = 0, dv = P^T dO
    cu_q, cu_k = np.array([0, 6]), np.array([0, 9])
    q = rng.standard_normal((6, 1, 4)); k = rng.standard_normal((9, 1, 4))
    v = np.tile(rng.standard_normal((1, 1, 4)), (9, 1, 1)); do = rng.standard_normal((6, 1, 4))
    dq, dk, dv = attention_bwd_ref(q, k, v, do, cu_q, cu_k, [3], [0], True)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
    # the total dv is the total dO whatever the weights (every row's P sums to 1)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)


def test_bwd_gqa_equals_summed_mha():
    """A kv head's gradient is the sum over its query group of the MHA gradients with the kv
    head repeated."""
    q, k, v, cu_q, cu_k, qo, ko = _rand_pack(21, 3, 30, 6, 2, 8, min_len=1)
    do = np.random.default_rng(22).standard_normal(q.shape)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, cu_q, cu_k, qo, ko, True)
    k_rep = np.repeat(k, 3, axis=1); v_rep = np.repeat(v, 3, axis=1)
    dq_m, dk_m, dv_m = attention_bwd_ref(q, k_rep, v_rep, do, cu_q, cu_k, qo, ko, True)
    _close(dq, dq_m, 1e-12)
    _close(dk, dk_m.reshape(dk.shape[0], 2, 3, 8).sum(axis=2), 1e-12)
    _close(dv, dv_m.reshape(dv.shape[0], 2, 3, 8).sum(axis=2), 1e-12)


# ----------------------------------------------------------------------------
# whole-share wrappers: pinned on a multi-sequence CP share with global offsets
# ----------------------------------------------------------------------------
from oracle import share_bwd_ref  # noqa: E402


@pytest.mark.parametrize("pieces,cp,q_piece,hq,hkv", [([5, 3, 7], 3, 2, 4, 2), ([4, 6], 4, 3, 2, 1),
                                                      ([9], 2, 0, 3, 3)])
def test_share_refs_match_sdpa_over_sequences_rebuilt_from_the_chunks(pieces, cp, q_piece, hq, hkv):
    """share_ref and share_bwd_ref against torch (float64 scaled_dot_product_attention with an
    explicit mask and its own GQA grouping, autograd for the gradients), per sequence, with
    the sequence's keys rebuilt from the chunks' pieces and their positions taken from the
    chunks' offsets: a swapped offset or prefix-sum array in either wrapper changes the
    result.  The share is one CP rank's (its query piece at q_piece x piece length)."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(31 + cp)
    d = 8
    g = wl._even_split_group(rng, pieces, cp, hq, hkv, d, "fp32", q_piece)
    do = rng.standard_normal(g.q.shape)
    o_ref, l_ref = share_ref(g)
    dq_ref, dk_ref, dv_ref = share_bwd_ref(g, do)
    for i, p in enumerate(pieces):
        ks = np.concatenate([c.k[c.cu_k[i]:c.cu_k[i + 1]] for c in g.chunks]).astype(np.float64)
        vs = np.concatenate([c.v[c.cu_k[i]:c.cu_k[i + 1]] for c in g.chunks]).astype(np.float64)
        kpos = np.concatenate([int(c.k_off[i]) + np.arange(c.cu_k[i + 1] - c.cu_k[i])
                               for c in g.chunks])
        assert np.array_equal(kpos, np.arange(cp * p))     # the chunks tile the sequence
        qpos = q_piece * p + np.arange(p)
        mask = torch.tensor(kpos[None, :] <= qpos[:, None])
        Q = torch.tensor(g.q[g.cu_q[i]:g.cu_q[i + 1]].astype(np.float64).transpose(1, 0, 2),
                         requires_grad=True)
        K = torch.tensor(ks.transpose(1, 0, 2), requires_grad=True)
        V = torch.tensor(vs.transpose(1, 0, 2), requires_grad=True)
        out = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, enable_gqa=True)
        scores = (Q @ K.repeat_interleave(hq // hkv, dim=0).transpose(1, 2)) / math.sqrt(d)
        lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)
        rows = slice(int(g.cu_q[i]), int(g.cu_q[i + 1]))
        np.testing.assert_allclose(o_ref[rows], out.detach().numpy().transpose(1, 0, 2), atol=1e-12)
        np.testing.assert_allclose(l_ref[:, rows], lse.detach().numpy(), atol=1e-12)
        (out * torch.tensor(do[rows].transpose(1, 0, 2))).sum().backward()
        keys = slice(int(g.cu_full[i]), int(g.cu_full[i + 1]))
        np.testing.assert_allclose(dq_ref[rows], Q.grad.numpy().transpose(1, 0, 2), atol=1e-11)
        np.testing.assert_allclose(dk_ref[keys], K.grad.numpy().transpose(1, 0, 2), atol=1e-11)
        np.testing.assert_allclose(dv_ref[keys], V.grad.numpy().transpose(1, 0, 2), atol=1e-11)
