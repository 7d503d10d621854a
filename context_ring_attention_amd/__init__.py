"""MI355X-native chunked causal attention for context parallelism (libcpattn).

The C-ABI library (include/cpattn.h, built to libcpattn.so) exports
cpattn_fwd_chunk (one KV chunk -> partial O and LSE) and cpattn_merge (the
online-softmax merge of two partials); this package binds them with the same
names and adds `cpattn_share`, the per-rank loop of the ring method on one GPU
(every KV chunk of a rank's share computed and merged in turn).
"""
from ._binding import (  # noqa: F401
    BF16, FP32, EXPORTED, LIB_PATH, PLAN_DTYPE, CpattnError, cpattn_fwd_chunk, cpattn_merge,
    cpattn_plan_build, cpattn_workspace_size, load,
)
from .share import ShareBuffers, cpattn_share  # noqa: F401
