"""CPU fp64 oracle (test infrastructure only; see ref.py's header)."""
from .ref import (attention_bwd_ref, attention_ref, flops_ref, merge_ref, share_bwd_ref,  # noqa: F401
                  share_ref, visible_pairs_ref)
