"""MI355X-native chunked causal attention for context parallelism (libcpattn).

The C-ABI library (include/cpattn.h, built to libcpattn.so) exports
cpattn_fwd_chunk (one KV chunk -> partial O and LSE), cpattn_fwd_chunk_accum
(the same, folded into a running result in the kernel epilogue),
cpattn_fwd_chunks (all chunks of a share in one launch, merged in registers) and
cpattn_merge (the online-softmax merge of two partials), cpattn_bwd_chunk(s) (the
gradients of the attention) and cpattn_dcp_schedule (the host scheduler of
Dynamic CP: per-sample CP size and micro-batch placement); this package binds them
with the same names and adds `cpattn_share`, the per-rank loop of the ring
method on one GPU.
"""
from ._binding import (  # noqa: F401
    BF16, FP32, EXPORTED, LIB_PATH, MAX_CHUNKS, PLAN_DTYPE, CpattnError, cpattn_bwd_chunk,
    cpattn_bwd_chunks, cpattn_bwd_workspace_size, cpattn_bwd_workspace_size_chunks, cpattn_dcp_schedule,
    cpattn_fwd_chunk,
    cpattn_fwd_chunk_accum, cpattn_fwd_chunks, cpattn_fwd_chunks_noalloc, cpattn_merge,
    cpattn_plan_build, cpattn_plan_build_device,
    cpattn_plan_build_chunks, cpattn_key_plan_build, cpattn_workspace_size,
    cpattn_workspace_size_chunks, load,
)
from .share import MODES, ShareBuffers, cpattn_share, cpattn_share_bwd  # noqa: F401
