"""Seeded synthetic inputs for the chunked-attention path.

This module only draws numbers and lays out packs: sequence lengths, cu_seqlens
prefix sums, per-sequence global position offsets, and Q/K/V values.  It holds
none of the attention arithmetic, so both the CPU oracle (via the tests) and the
GPU path consume the same inputs without sharing any method code.

Workload shapes follow the pages' scenarios:
  * "Dynamic Context Parallelism" (verl docs): a static CP4 run with a 16,384-token
    packed budget has a per-rank limit of 16384 / 4 = 4096 tokens, and DCP picks a
    CP size per micro-batch from the sequence lengths.
  * "Megatron 6D parallelism guide", section 6 (context parallelism): a 128K
    context at CP=4 gives each GPU 32K tokens; each rank holds S/CP of a sequence
    and walks the KV chunks of the whole sequence.

Draw order for every workload (one numpy Generator, `default_rng(seed)`):
  1. sequence lengths, one draw per sequence;
  2. Q rows for the rank's share only, `standard_normal(float32)`;
  3. K for every global token, then V for every global token.
Chunks are slices of the global K/V.  bf16 workloads round every value to the
nearest bfloat16 (round-to-nearest-even) and keep it in a float32 array, so the
GPU converts it to bf16 exactly and the oracle reads the very same numbers.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

__all__ = [
    "Chunk", "Group", "Workload", "round_to_bf16", "make", "CONFIGS",
    "cu_from_lengths", "fill_budget", "lengths_for", "dcp_chunk_count", "random_pack",
]

CONFIGS = ("tiny", "pack", "cp4_share", "ctx128k_share", "dcp_mixed")


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    if len(lengths):
        cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64)).astype(np.int32)
    return cu


def fill_budget(draw, budget: int) -> List[int]:
    """Draw lengths until they reach `budget`; the last one is cut to fit exactly."""
    out: List[int] = []
    total = 0
    while total < budget:
        x = min(int(draw()), budget - total)
        out.append(x)
        total += x
    return out


@dataclass
class Chunk:
    """One KV chunk of a group: THD rows plus per-sequence metadata."""
    k: np.ndarray             # [Tk, Hkv, D] float32
    v: np.ndarray             # [Tk, Hkv, D] float32
    cu_k: np.ndarray          # int32 [nseq+1]
    k_off: np.ndarray         # int32 [nseq], global position of each sequence's first key


@dataclass
class Group:
    """A Q pack and the KV chunks it is computed against (one CP rank's share)."""
    q: np.ndarray             # [Tq, Hq, D] float32
    cu_q: np.ndarray          # int32 [nseq+1]
    q_off: np.ndarray         # int32 [nseq], global position of each sequence's first query
    chunks: List[Chunk]
    k_full: np.ndarray        # [sum of whole-sequence lengths, Hkv, D]: every key of each sequence
    v_full: np.ndarray
    cu_full: np.ndarray       # int32 [nseq+1] over k_full
    sample_ids: List[int] = field(default_factory=list)


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str                # "fp32" or "bf16"
    hq: int
    hkv: int
    d: int
    causal: bool
    lengths: List[int]        # whole-sample lengths in draw order
    groups: List[Group]
    note: str = ""

    @property
    def cp(self) -> int:
        return max(len(g.chunks) for g in self.groups)


def _normal(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def _even_split_group(rng, pieces, cp, hq, hkv, d, dtype, q_piece):
    """Each sequence i is cp pieces of length pieces[i]; Q is piece `q_piece`.

    Global sequence i has cp * pieces[i] tokens.  Chunk c holds piece c of every
    sequence, so all chunks share Q's cu_seqlens (as in a static CP split).
    """
    nseq = len(pieces)
    cu = cu_from_lengths(pieces)
    tq = int(cu[-1])
    q = _normal(rng, (tq, hq, d), dtype)
    glen = [cp * p for p in pieces]
    cu_full = cu_from_lengths(glen)
    tk = int(cu_full[-1])
    k_full = _normal(rng, (tk, hkv, d), dtype)
    v_full = _normal(rng, (tk, hkv, d), dtype)
    chunks = []
    for c in range(cp):
        rows = np.concatenate([np.arange(cu_full[i] + c * pieces[i], cu_full[i] + (c + 1) * pieces[i])
                               for i in range(nseq)]) if nseq else np.zeros(0, np.int64)
        chunks.append(Chunk(k=np.ascontiguousarray(k_full[rows]), v=np.ascontiguousarray(v_full[rows]),
                            cu_k=cu.copy(),
                            k_off=np.array([c * p for p in pieces], dtype=np.int32)))
    q_off = np.array([q_piece * p for p in pieces], dtype=np.int32)
    return Group(q=q, cu_q=cu, q_off=q_off, chunks=chunks, k_full=k_full, v_full=v_full,
                 cu_full=cu_full, sample_ids=list(range(nseq)))


def make_tiny(seed: int = 0) -> Workload:
    """One sequence of 256 tokens, 2 heads, D=64, fp32; KV in two chunks of 128."""
    rng = np.random.default_rng(seed)
    s, h, d = 256, 2, 64
    q = rng.standard_normal(size=(s, h, d), dtype=np.float32)
    k = rng.standard_normal(size=(s, h, d), dtype=np.float32)
    v = rng.standard_normal(size=(s, h, d), dtype=np.float32)
    chunks = [Chunk(k=k[c * 128:(c + 1) * 128].copy(), v=v[c * 128:(c + 1) * 128].copy(),
                    cu_k=np.array([0, 128], np.int32), k_off=np.array([128 * c], np.int32))
              for c in range(2)]
    g = Group(q=q, cu_q=np.array([0, s], np.int32), q_off=np.zeros(1, np.int32), chunks=chunks,
              k_full=k, v_full=v, cu_full=np.array([0, s], np.int32), sample_ids=[0])
    return Workload("tiny", seed, "fp32", h, h, d, True, [s], [g])


def make_pack(seed: int = 0) -> Workload:
    """4,096-token budget of sequences with lengths uniform in [64, 1024]; cp=1."""
    rng = np.random.default_rng(seed)
    lens = fill_budget(lambda: rng.integers(64, 1025), 4096)
    hq, hkv, d = 32, 8, 128
    g = _even_split_group(rng, lens, 1, hq, hkv, d, "bf16", 0)
    return Workload("pack", seed, "bf16", hq, hkv, d, True, lens, [g])


def make_cp4_share(seed: int = 0) -> Workload:
    """The last CP4 rank's share of a 16,384-token packed budget.

    The local pieces are uniform in [512, 4096] and fill 4,096 tokens; each
    sequence is 4 pieces long, Q is its piece 3 and the 4 KV chunks are its
    pieces 0..3 at their global positions.
    """
    rng = np.random.default_rng(seed)
    pieces = fill_budget(lambda: rng.integers(512, 4097), 4096)
    g = _even_split_group(rng, pieces, 4, 32, 8, 128, "bf16", 3)
    return Workload("cp4_share", seed, "bf16", 32, 8, 128, True, [4 * p for p in pieces], [g])


def make_ctx128k_share(seed: int = 0, s_local: int = 32768) -> Workload:
    """The last CP=4 rank of one 131,072-token sequence: 8 q heads / 1 kv head, D=128."""
    rng = np.random.default_rng(seed)
    g = _even_split_group(rng, [s_local], 4, 8, 1, 128, "bf16", 3)
    return Workload("ctx128k_share", seed, "bf16", 8, 1, 128, True, [4 * s_local], [g])


def dcp_chunk_count(length: int, limit: int = 4096) -> int:
    """Smallest power of two cp in {1,2,4,8} with ceil(length/cp) <= limit (8 otherwise)."""
    for cp in (1, 2, 4, 8):
        if -(-length // cp) <= limit:
            return cp
    return 8


def make_dcp_mixed(seed: int = 0, budget: int = 65536) -> Workload:
    """Mixed-length pack; each sample's KV is split into its own number of chunks.

    Lengths are lognormal with median 1,024 (sigma 1 in natural log), rounded and
    clipped to [32, 32768], drawn until the budget is reached (the last one cut).
    Samples are grouped by their chunk count; every group's Q is the whole of its
    samples, and chunk c of a sample of length L is keys [c*p, min((c+1)*p, L))
    with p = ceil(L / cp).
    """
    rng = np.random.default_rng(seed)
    lens = fill_budget(lambda: np.clip(np.round(np.exp(rng.normal(np.log(1024.0), 1.0))), 32, 32768),
                       budget)
    hq, hkv, d = 32, 8, 128
    cu_all = cu_from_lengths(lens)
    T = int(cu_all[-1])
    q_all = _normal(rng, (T, hq, d), "bf16")
    k_all = _normal(rng, (T, hkv, d), "bf16")
    v_all = _normal(rng, (T, hkv, d), "bf16")
    cps = [dcp_chunk_count(L) for L in lens]
    groups = []
    for cp in (1, 2, 4, 8):
        ids = [i for i, c in enumerate(cps) if c == cp]
        if not ids:
            continue
        glens = [lens[i] for i in ids]
        rows = np.concatenate([np.arange(cu_all[i], cu_all[i + 1]) for i in ids])
        q = np.ascontiguousarray(q_all[rows])
        k_full = np.ascontiguousarray(k_all[rows])
        v_full = np.ascontiguousarray(v_all[rows])
        cu_g = cu_from_lengths(glens)
        chunks = []
        for c in range(cp):
            lo = [min(c * -(-L // cp), L) for L in glens]
            hi = [min((c + 1) * -(-L // cp), L) for L in glens]
            crow = np.concatenate([np.arange(cu_g[j] + lo[j], cu_g[j] + hi[j]) for j in range(len(ids))])
            chunks.append(Chunk(k=np.ascontiguousarray(k_full[crow]), v=np.ascontiguousarray(v_full[crow]),
                                cu_k=cu_from_lengths([h - l for l, h in zip(lo, hi)]),
                                k_off=np.array(lo, dtype=np.int32)))
        groups.append(Group(q=q, cu_q=cu_g, q_off=np.zeros(len(ids), np.int32), chunks=chunks,
                            k_full=k_full, v_full=v_full, cu_full=cu_g.copy(), sample_ids=ids))
    return Workload("dcp_mixed", seed, "bf16", hq, hkv, d, True, lens, groups)


def lengths_for(name: str, seed: int = 0) -> List[int]:
    """The length draws of a workload alone (they come first from the generator)."""
    rng = np.random.default_rng(seed)
    if name == "tiny":
        return [256]
    if name == "pack":
        return fill_budget(lambda: rng.integers(64, 1025), 4096)
    if name == "cp4_share":
        return fill_budget(lambda: rng.integers(512, 4097), 4096)   # local pieces
    if name == "ctx128k_share":
        return [32768]                                              # local piece
    if name == "dcp_mixed":
        return fill_budget(lambda: np.clip(np.round(np.exp(rng.normal(np.log(1024.0), 1.0))), 32, 32768),
                           65536)
    raise KeyError(name)


_MAKERS = {
    "tiny": make_tiny,
    "pack": make_pack,
    "cp4_share": make_cp4_share,
    "ctx128k_share": make_ctx128k_share,
    "dcp_mixed": make_dcp_mixed,
}


def make(name: str, seed: int = 0, **kw) -> Workload:
    if name not in _MAKERS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(_MAKERS)}")
    return _MAKERS[name](seed, **kw)


def random_pack(rng: np.random.Generator, nseq: int, max_len: int, hq: int, hkv: int, d: int,
                dtype: str = "bf16", min_len: int = 0, k_extra: Optional[int] = None):
    """A random pack with independent q/k lengths and offsets, for property tests.

    Returns (q, k, v, cu_q, cu_k, q_off, k_off).  Offsets are drawn so that the
    causal diagonal falls anywhere (including before/after the whole chunk).
    """
    lq = rng.integers(min_len, max_len + 1, size=nseq)
    lk = rng.integers(min_len, max_len + 1, size=nseq) if k_extra is None else lq + k_extra
    q_off = rng.integers(0, 2 * max_len + 1, size=nseq).astype(np.int32)
    k_off = rng.integers(0, 2 * max_len + 1, size=nseq).astype(np.int32)
    cu_q = cu_from_lengths(lq)
    cu_k = cu_from_lengths(lk)
    q = _normal(rng, (int(cu_q[-1]), hq, d), dtype)
    k = _normal(rng, (int(cu_k[-1]), hkv, d), dtype)
    v = _normal(rng, (int(cu_k[-1]), hkv, d), dtype)
    return q, k, v, cu_q, cu_k, q_off, k_off
