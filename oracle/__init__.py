"""CPU fp64 oracle (test infrastructure only; see ref.py's header)."""
from .ref import attention_ref, merge_ref, share_ref, visible_pairs_ref, flops_ref  # noqa: F401
