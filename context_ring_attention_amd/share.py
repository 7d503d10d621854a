"""One rank's share on one GPU: its queries against every KV chunk of the share.

This is the per-rank loop of ring attention ("Megatron 6D parallelism guide",
section 6): for each of the cp steps the rank's queries meet the current KV
chunk and the partial is folded into the running result with the
online-softmax merge.  On one GPU the chunks are already resident, so the
ring's send/recv between steps is absent.  Three schedules of the same
arithmetic are offered:

  "stream"  one cpattn_fwd_chunks launch over all chunks: the running max, sum
            and accumulator of each row are carried across chunks in registers
            (no partial written, no merge pass);
  "accum"   the ring's step order, one cpattn_fwd_chunk per chunk, the later
            ones with cpattn_fwd_chunk_accum folding into the result in the
            kernel epilogue;
  "merge"   the ring's step order with explicit partials: cpattn_fwd_chunk per
            chunk, then cpattn_merge into the running result.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

from ._binding import (cpattn_bwd_chunk, cpattn_bwd_chunks, cpattn_fwd_chunk,
                       cpattn_fwd_chunk_accum, cpattn_fwd_chunks, cpattn_merge,
                       cpattn_workspace_size_chunks)

MODES = ("stream", "accum", "merge")


@dataclass
class ShareBuffers:
    """Device buffers reused across calls: running result, one partial, workspace."""
    o_acc: object
    lse_acc: object
    o_part: object
    lse_part: object
    workspace: object

    @staticmethod
    def allocate(q, hkv: int, cu_seqlens_q, nchunks: int = 1) -> "ShareBuffers":
        import torch
        tq, hq, d = q.shape
        nseq = len(cu_seqlens_q) - 1
        ws = cpattn_workspace_size_chunks(nseq, cu_seqlens_q, hq, hkv, d, max(1, nchunks))
        f32 = dict(dtype=torch.float32, device=q.device)
        return ShareBuffers(torch.empty((tq, hq, d), **f32), torch.empty((hq, tq), **f32),
                            torch.empty((tq, hq, d), **f32), torch.empty((hq, tq), **f32),
                            torch.empty(max(ws, 256), dtype=torch.uint8, device=q.device))


def cpattn_share(q, ks: Sequence, vs: Sequence, cu_seqlens_q, cu_seqlens_ks: Sequence,
                 q_pos_offset=None, k_pos_offsets: Optional[Sequence] = None, causal: bool = True,
                 buffers: Optional[ShareBuffers] = None, stream=None, mode: str = "stream"):
    """Attention of q against the union of the chunks; returns (O, LSE) of the share.

    ks[c], vs[c]: chunk c's keys/values [Tk_c, Hkv, D]; cu_seqlens_ks[c] and
    k_pos_offsets[c]: its host metadata.  The result lives in `buffers.o_acc`
    and `buffers.lse_acc` (allocated if not given; the workspace must cover
    len(ks) chunks for mode "stream").
    """
    if len(ks) == 0:
        raise ValueError("a share needs at least one KV chunk")
    if mode not in MODES:
        raise ValueError(f"mode must be one of {MODES}")
    hkv = ks[0].shape[1]
    if buffers is None:
        buffers = ShareBuffers.allocate(q, hkv, cu_seqlens_q, len(ks))
    k_pos_offsets = k_pos_offsets if k_pos_offsets is not None else [None] * len(ks)
    if mode == "stream":
        cpattn_fwd_chunks(q, ks, vs, cu_seqlens_q, cu_seqlens_ks, q_pos_offset, k_pos_offsets,
                          causal, out=buffers.o_acc, lse=buffers.lse_acc,
                          workspace=buffers.workspace, stream=stream)
        return buffers.o_acc, buffers.lse_acc
    cpattn_fwd_chunk(q, ks[0], vs[0], cu_seqlens_q, cu_seqlens_ks[0], q_pos_offset,
                     k_pos_offsets[0], causal, out=buffers.o_acc, lse=buffers.lse_acc,
                     workspace=buffers.workspace, stream=stream)
    for c in range(1, len(ks)):
        if mode == "accum":
            cpattn_fwd_chunk_accum(q, ks[c], vs[c], cu_seqlens_q, cu_seqlens_ks[c], q_pos_offset,
                                   k_pos_offsets[c], causal, out=buffers.o_acc,
                                   lse=buffers.lse_acc, workspace=buffers.workspace, stream=stream)
            continue
        cpattn_fwd_chunk(q, ks[c], vs[c], cu_seqlens_q, cu_seqlens_ks[c], q_pos_offset,
                         k_pos_offsets[c], causal, out=buffers.o_part, lse=buffers.lse_part,
                         workspace=buffers.workspace, stream=stream)
        cpattn_merge(buffers.o_acc, buffers.lse_acc, buffers.o_part, buffers.lse_part,
                     stream=stream)
    return buffers.o_acc, buffers.lse_acc


def cpattn_share_bwd(q, ks: Sequence, vs: Sequence, o, lse, do, cu_seqlens_q,
                     cu_seqlens_ks: Sequence, q_pos_offset=None,
                     k_pos_offsets: Optional[Sequence] = None, causal: bool = True, stream=None,
                     per_chunk: bool = False):
    """Backward of a rank's share: given the share's forward (o, lse) and the gradient do,
    returns dq [Tq, Hq, D] (summed over the chunks) and per-chunk lists dks, dvs (fp32).

    Default: one cpattn_bwd_chunks pass over all chunks.  per_chunk=True takes the ring's
    backward step order instead, one cpattn_bwd_chunk call per chunk, each adding its dq
    contribution and yielding the gradients of that chunk's keys and values (which a ring
    would send back to their owner).
    """
    import torch
    if len(ks) == 0:
        raise ValueError("a share needs at least one KV chunk")
    if not per_chunk:
        return cpattn_bwd_chunks(q, ks, vs, o, lse, do, cu_seqlens_q, cu_seqlens_ks, q_pos_offset,
                                 k_pos_offsets, causal, stream=stream)
    k_pos_offsets = k_pos_offsets if k_pos_offsets is not None else [None] * len(ks)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    dks, dvs = [], []
    for c in range(len(ks)):
        _, dk, dv = cpattn_bwd_chunk(q, ks[c], vs[c], o, lse, do, cu_seqlens_q, cu_seqlens_ks[c],
                                     q_pos_offset, k_pos_offsets[c], causal, dq=dq, stream=stream)
        dks.append(dk)
        dvs.append(dv)
    return dq, dks, dvs
