"""One rank's share on one GPU: every KV chunk computed, then merged in turn.

This is the per-rank loop of ring attention ("Megatron 6D parallelism guide",
section 6): for each of the cp steps the rank's queries meet the current KV
chunk (cpattn_fwd_chunk) and the partial is folded into the running result
(cpattn_merge).  On one GPU the chunks are already resident, so the ring's
send/recv between steps is absent; the step order is the ring's.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

from ._binding import cpattn_fwd_chunk, cpattn_merge, cpattn_workspace_size


@dataclass
class ShareBuffers:
    """Device buffers reused across calls: running result, one partial, workspace."""
    o_acc: object
    lse_acc: object
    o_part: object
    lse_part: object
    workspace: object

    @staticmethod
    def allocate(q, hkv: int, cu_seqlens_q) -> "ShareBuffers":
        import torch
        tq, hq, d = q.shape
        nseq = len(cu_seqlens_q) - 1
        ws = cpattn_workspace_size(nseq, cu_seqlens_q, hq, hkv, d)
        f32 = dict(dtype=torch.float32, device=q.device)
        return ShareBuffers(torch.empty((tq, hq, d), **f32), torch.empty((hq, tq), **f32),
                            torch.empty((tq, hq, d), **f32), torch.empty((hq, tq), **f32),
                            torch.empty(max(ws, 256), dtype=torch.uint8, device=q.device))


def cpattn_share(q, ks: Sequence, vs: Sequence, cu_seqlens_q, cu_seqlens_ks: Sequence,
                 q_pos_offset=None, k_pos_offsets: Optional[Sequence] = None, causal: bool = True,
                 buffers: Optional[ShareBuffers] = None, stream=None):
    """Attention of q against the union of the chunks; returns (O, LSE) of the share.

    ks[c], vs[c]: chunk c's keys/values [Tk_c, Hkv, D]; cu_seqlens_ks[c] and
    k_pos_offsets[c]: its host metadata.  The result lives in `buffers.o_acc`
    and `buffers.lse_acc` (allocated if not given).
    """
    if len(ks) == 0:
        raise ValueError("a share needs at least one KV chunk")
    hkv = ks[0].shape[1]
    if buffers is None:
        buffers = ShareBuffers.allocate(q, hkv, cu_seqlens_q)
    k_pos_offsets = k_pos_offsets if k_pos_offsets is not None else [None] * len(ks)
    cpattn_fwd_chunk(q, ks[0], vs[0], cu_seqlens_q, cu_seqlens_ks[0], q_pos_offset,
                     k_pos_offsets[0], causal, out=buffers.o_acc, lse=buffers.lse_acc,
                     workspace=buffers.workspace, stream=stream)
    for c in range(1, len(ks)):
        cpattn_fwd_chunk(q, ks[c], vs[c], cu_seqlens_q, cu_seqlens_ks[c], q_pos_offset,
                         k_pos_offsets[c], causal, out=buffers.o_part, lse=buffers.lse_part,
                         workspace=buffers.workspace, stream=stream)
        cpattn_merge(buffers.o_acc, buffers.lse_acc, buffers.o_part, buffers.lse_part,
                     stream=stream)
    return buffers.o_acc, buffers.lse_acc
