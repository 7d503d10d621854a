"""CPU fp64 oracle for chunked causal attention over packed sequences.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this module: only the test suite, the package smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library and it does not
import it.

What it computes (the plain definition that the ring-attention method reaches
exactly, up to rounding order):

  For every packed sequence i, query head h and query token t of that sequence,
  with global query position pq = q_off[i] + t:
    kv head      g = floor(h * Hkv / Hq)                 (contiguous GQA groups)
    visible keys U_t = { u : k_off[i] + u <= pq }   (causal, same sequence only)
                 U_t = { all u of sequence i }        (non-causal)
    scores       s_u = (q_t . k_u) / sqrt(D)
    LSE_t        = m + ln sum_{u in U_t} exp(s_u - m),   m = max_u s_u
    O_t          = sum_{u in U_t} exp(s_u - LSE_t) * v_u
    empty U_t    -> O_t = 0, LSE_t = -inf

  Sources: "Megatron 6D parallelism guide", section 6 (context parallelism):
  the ring loop computes one attention partial per KV chunk, folds each into a
  running result by rescaling both to a common maximum, and normalises at the
  end; that is exactly softmax(QK^T)V over the union of the chunks.  The 1/sqrt(D) scale, the causal mask by global
  position, GQA and the LSE output are not printed on the pages; the readings
  taken are: scale 1/sqrt(D); mask inclusive of the diagonal (k_pos <= q_pos),
  never across sequences; contiguous GQA groups; LSE in natural log.

This is a two-pass softmax over whole rows (max first, then the sum), in row
blocks only to bound memory.  It is not an online softmax and never splits a
row's keys, so it shares neither code nor algorithm with the GPU kernels.

merge_ref is the combination of two normalised partials over disjoint key sets,
written from its definition: the union's LSE is the log of the summed softmax
masses, and its O is the mass-weighted mix of the two sides.

attention_bwd_ref is the gradient of the same function.  The pages train with
context parallelism (a forward-backward pass per micro-batch); they print no
backward of the attention, and the reading taken is the plain one: the gradient
of O = softmax(Q K^T / sqrt(D) + mask) V with respect to Q, K and V for an
upstream gradient dO, written out by the chain rule through the row softmax.  Every function here is pinned by tests/test_oracle.py (brute force,
closed forms, torch's scaled_dot_product_attention, invariants); none is
"parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = ["attention_ref", "attention_bwd_ref", "merge_ref", "share_ref", "share_bwd_ref",
           "visible_pairs_ref", "flops_ref"]

_ROW_BLOCK = 256


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention_ref(q, k, v, cu_q, cu_k, q_off=None, k_off=None, causal: bool = True,
                  rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(Q K^T / sqrt(D) + mask) V per packed sequence, in fp64.

    q: [Tq, Hq, D]; k, v: [Tk, Hkv, D] (any float dtype; read as fp64).
    cu_q, cu_k: int [nseq+1] prefix sums; q_off, k_off: int [nseq] global position
    of each sequence's first query / key (None means zeros).
    rows: optional sorted subset of query rows; then only those rows are computed
    and the result is (O[len(rows), Hq, D], LSE[Hq, len(rows)]).
    Returns O [Tq, Hq, D] and LSE [Hq, Tq] (float64).
    """
    q = np.asarray(q); k = np.asarray(k); v = np.asarray(v)
    cu_q = np.asarray(cu_q, dtype=np.int64); cu_k = np.asarray(cu_k, dtype=np.int64)
    nseq = len(cu_q) - 1
    q_off = np.zeros(nseq, np.int64) if q_off is None else np.asarray(q_off, dtype=np.int64)
    k_off = np.zeros(nseq, np.int64) if k_off is None else np.asarray(k_off, dtype=np.int64)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0, "query heads must be a multiple of kv heads"
    scale = 1.0 / math.sqrt(d)

    want = np.arange(tq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(want), hq, d), dtype=np.float64)
    lse = np.full((hq, len(want)), -np.inf, dtype=np.float64)
    seq_of = np.searchsorted(cu_q, want, side="right") - 1

    for i in range(nseq):
        sel = np.nonzero(seq_of == i)[0]            # positions in `want`
        if sel.size == 0:
            continue
        t_loc = want[sel] - cu_q[i]                 # token index within sequence i
        k_i = _as64(k[cu_k[i]:cu_k[i + 1]])
        v_i = _as64(v[cu_k[i]:cu_k[i + 1]])
        nk = k_i.shape[0]
        u = np.arange(nk)
        for b0 in range(0, sel.size, _ROW_BLOCK):
            bsel = sel[b0:b0 + _ROW_BLOCK]
            bt = t_loc[b0:b0 + _ROW_BLOCK]
            if causal:
                vis = (k_off[i] + u[None, :]) <= (q_off[i] + bt[:, None])
            else:
                vis = np.ones((bt.size, nk), dtype=bool)
            nonempty = vis.any(axis=1)
            for h in range(hq):
                g = (h * hkv) // hq
                qb = _as64(q[want[bsel], h])                 # [b, D]
                s = (qb @ k_i[:, g].T) * scale               # [b, nk]
                s = np.where(vis, s, -np.inf)
                m = np.max(s, axis=1, initial=-np.inf)
                m_safe = np.where(nonempty, m, 0.0)
                e = np.exp(s - m_safe[:, None])              # exp(-inf) = 0 for hidden keys
                l = e.sum(axis=1)
                with np.errstate(divide="ignore"):
                    row_lse = np.where(nonempty, m_safe + np.log(np.where(nonempty, l, 1.0)), -np.inf)
                p = np.exp(s - np.where(nonempty, row_lse, 0.0)[:, None])
                ob = p @ v_i[:, g]
                ob[~nonempty] = 0.0
                o[bsel, h] = ob
                lse[h, bsel] = row_lse
    return o, lse


def attention_bwd_ref(q, k, v, do, cu_q, cu_k, q_off=None, k_off=None,
                      causal: bool = True) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of attention_ref's O with respect to q, k, v for upstream gradient do (fp64).

    Per packed sequence and query head h (kv head g), with S = Q K_g^T / sqrt(D) masked as
    in attention_ref and P its row softmax (rows with no visible key have P = 0):
        dV_g += P^T dO                          (O = P V)
        dP    = dO V_g^T
        dS    = P * (dP - rowsum(P * dP))       (Jacobian of the row softmax)
        dQ_h  = dS K_g / sqrt(D)
        dK_g += dS^T Q_h / sqrt(D)
    A kv head's gradient sums the contributions of every query head of its group.
    Rows are processed in blocks, each row against all its keys (a row's softmax is never
    split).  Returns dq [Tq, Hq, D], dk and dv [Tk, Hkv, D] (float64).
    """
    q = np.asarray(q); k = np.asarray(k); v = np.asarray(v); do = np.asarray(do)
    cu_q = np.asarray(cu_q, dtype=np.int64); cu_k = np.asarray(cu_k, dtype=np.int64)
    nseq = len(cu_q) - 1
    q_off = np.zeros(nseq, np.int64) if q_off is None else np.asarray(q_off, dtype=np.int64)
    k_off = np.zeros(nseq, np.int64) if k_off is None else np.asarray(k_off, dtype=np.int64)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0, "query heads must be a multiple of kv heads"
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros((tq, hq, d), dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for i in range(nseq):
        k_i = _as64(k[cu_k[i]:cu_k[i + 1]])
        v_i = _as64(v[cu_k[i]:cu_k[i + 1]])
        nk = k_i.shape[0]
        u = np.arange(nk)
        for t0 in range(int(cu_q[i]), int(cu_q[i + 1]), _ROW_BLOCK):
            t1 = min(t0 + _ROW_BLOCK, int(cu_q[i + 1]))
            bt = np.arange(t0, t1) - cu_q[i]
            if causal:
                vis = (k_off[i] + u[None, :]) <= (q_off[i] + bt[:, None])
            else:
                vis = np.ones((bt.size, nk), dtype=bool)
            nonempty = vis.any(axis=1)
            for h in range(hq):
                g = (h * hkv) // hq
                qb = _as64(q[t0:t1, h])
                dob = _as64(do[t0:t1, h])
                s = np.where(vis, (qb @ k_i[:, g].T) * scale, -np.inf)
                m = np.where(nonempty, np.max(s, axis=1, initial=-np.inf), 0.0)
                e = np.exp(s - m[:, None])
                l = np.where(nonempty, e.sum(axis=1), 1.0)
                p = e / l[:, None]                                  # 0 on hidden keys and empty rows
                dv[cu_k[i]:cu_k[i + 1], g] += p.T @ dob
                dp = dob @ v_i[:, g].T
                ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
                dq[t0:t1, h] = (ds @ k_i[:, g]) * scale
                dk[cu_k[i]:cu_k[i + 1], g] += (ds.T @ qb) * scale
    return dq, dk, dv


def merge_ref(o_a, lse_a, o_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Merge two partial results over disjoint key sets (fp64).

    Inputs are normalised partials: O [T, H, D] and LSE [H, T].  A normalised partial over
    a key set U has mass exp(LSE) = sum_{u in U} exp(s_u) and O = sum_u exp(s_u) v_u / mass.
    Over the union of two disjoint sets the mass is the sum of the two masses, so
        LSE = ln(exp(lse_a) + exp(lse_b))
        O   = exp(lse_a - LSE) * O_a + exp(lse_b - LSE) * O_b
    (each side weighted by its share of the union's mass).  An empty partial (LSE = -inf,
    mass 0) is the identity; two empty partials give an empty one (O = 0, LSE = -inf),
    never NaN.
    """
    o_a = _as64(o_a); o_b = _as64(o_b)
    la = _as64(lse_a).T[..., None]                  # [T, H, 1]
    lb = _as64(lse_b).T[..., None]
    lse = np.logaddexp(la, lb)                      # -inf only when both sides are empty
    both_empty = np.isneginf(lse)
    lse_safe = np.where(both_empty, 0.0, lse)
    w_a = np.exp(la - lse_safe)                     # exp(-inf) = 0 for an empty side
    w_b = np.exp(lb - lse_safe)
    o = np.where(w_a > 0, w_a * o_a, 0.0) + np.where(w_b > 0, w_b * o_b, 0.0)
    o = np.where(both_empty, 0.0, o)
    return o, lse[..., 0].T.copy()


def share_ref(group, causal: bool = True, rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """A rank's whole share: its Q against every key of its sequences, unsplit."""
    nseq = len(group.cu_q) - 1
    return attention_ref(group.q, group.k_full, group.v_full, group.cu_q, group.cu_full,
                         group.q_off, np.zeros(nseq, np.int64), causal=causal, rows=rows)


def share_bwd_ref(group, do, causal: bool = True) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of a rank's whole share (its Q against every key of its sequences) for the
    upstream gradient do [Tq, Hq, D]: dq [Tq, Hq, D] and dk, dv over the whole sequences'
    keys [Tfull, Hkv, D] (rows of k_full / v_full)."""
    nseq = len(group.cu_q) - 1
    return attention_bwd_ref(group.q, group.k_full, group.v_full, do, group.cu_q, group.cu_full,
                             group.q_off, np.zeros(nseq, np.int64), causal=causal)


def visible_pairs_ref(cu_q, cu_k, q_off=None, k_off=None, causal: bool = True) -> int:
    """Number of visible (query, key) pairs per query head, by enumerating the mask."""
    cu_q = np.asarray(cu_q, dtype=np.int64); cu_k = np.asarray(cu_k, dtype=np.int64)
    nseq = len(cu_q) - 1
    q_off = np.zeros(nseq, np.int64) if q_off is None else np.asarray(q_off, dtype=np.int64)
    k_off = np.zeros(nseq, np.int64) if k_off is None else np.asarray(k_off, dtype=np.int64)
    total = 0
    for i in range(nseq):
        nq = int(cu_q[i + 1] - cu_q[i]); nk = int(cu_k[i + 1] - cu_k[i])
        if not causal:
            total += nq * nk
            continue
        qp = q_off[i] + np.arange(nq)
        kp = k_off[i] + np.arange(nk)
        # per query row: number of keys with position <= its position
        total += int(np.searchsorted(kp, qp, side="right").sum())
    return total


def flops_ref(pairs_per_head: int, hq: int, d: int) -> int:
    """Algorithmic FLOPs: QK^T and PV each cost 2*D per visible pair and head."""
    return 4 * d * hq * int(pairs_per_head)
