"""fp64 CPU oracle for blockwise exact attention (test infrastructure only).

This package is the checker, not the product. Only the test suite, the smoke
entry point and the benchmark's CPU-baseline leg may import it; the HIP
library never calls it and it never calls the HIP library.

Sources: the pages "flash_sharding.py" (flash_attn_jax; functions ring_fwd
and ring_bwd) and "picotron/parallel/context_parallel.py" (functions
ring_attention_forward, ring_attention_backward, update_out_and_lse and
RingAttention._repeat_kv).
"""
from .attention import (
    allowed_mask,
    attention_fwd,
    attention_bwd,
    merge,
    merge_sigmoid,
    ring_share,
)

__all__ = [
    "allowed_mask",
    "attention_fwd",
    "attention_bwd",
    "merge",
    "merge_sigmoid",
    "ring_share",
]
