"""MI355X (gfx950) blockwise exact attention.

The compute lives in libattn.so (hand-written HIP kernels behind the C ABI of
include/attn.h).  `attention` is the torch binding; `inputs` and `workloads`
describe the seeded synthetic inputs; `flops` the algorithmic work.
"""
from .attention import (  # noqa: F401
    attn_fwd,
    attn_fwd_acc,
    attn_merge,
    attn_acc_init,
    attn_acc_cast,
    attn_bwd,
    attn_bwd_acc,
    attention_forward,
    attention_backward,
    flash_attention,
    bwd_workspace_bytes,
    ring_share,
    RingShare,
    RingShareBwd,
)
from ._lib import AttnError, lib  # noqa: F401
