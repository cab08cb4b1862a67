"""The five synthetic workloads, as shapes and mask parameters.

C1 tiny fp32 non-causal; C2 causal MHA; C3 one ring rank's share of causal
GQA (rank 7 of 8 over 8192 tokens); C4 causal sliding window (256, 0) at
d = 64; C5 long-context causal forward + backward.  Inputs come from
`inputs.draw_normal` with seed 1000 + the workload number, drawn in the order
q, k, v, dO.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .inputs import draw_normal, round_to_bf16


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    n: int
    l_q: int
    l_k: int
    h: int
    h_kv: int
    d: int
    dtype: str                 # "f32" or "bf16"
    causal: bool
    win_l: int = -1
    win_r: int = -1
    q_offset: int = 0
    k_offset: int = 0
    backward: bool = False
    ring_chunks: int = 0       # > 0: the ring share (q is one chunk of the full sequence)
    ring_rank: int = 0
    scale: float = field(default=0.0)

    @property
    def seed(self):
        return 1000 + self.index

    @property
    def softmax_scale(self):
        return self.scale if self.scale else 1.0 / math.sqrt(self.d)


WORKLOADS = {
    "C1": Workload("tiny-fp32-noncausal", 1, 1, 128, 128, 2, 2, 64, "f32", False),
    "C2": Workload("causal-mha-bf16-n2-l2048-h16-d128", 2, 2, 2048, 2048, 16, 16,
                   128, "bf16", True),
    "C3": Workload("ring-rank7of8-causal-gqa32x8-l8192-d128", 3, 1, 1024, 1024,
                   32, 8, 128, "bf16", True, ring_chunks=8, ring_rank=7),
    "C4": Workload("window256-causal-bf16-n4-l4096-h16-d64", 4, 4, 4096, 4096,
                   16, 16, 64, "bf16", True, win_l=256, win_r=0),
    "C5": Workload("long-causal-fwdbwd-bf16-n1-l16384-h16-d128", 5, 1, 16384,
                   16384, 16, 16, 128, "bf16", True, backward=True),
}


def make_inputs(w: Workload):
    """Synthetic inputs of a workload as float32 numpy arrays (bf16-valued
    when the workload is bf16).

    Returns a dict with q, k, v (and do when the workload has a backward).
    For the ring share, q is the local chunk of the full sequence and
    k_chunks / v_chunks / k_offsets list the chunks in ring order.
    """
    if w.ring_chunks:
        full = w.l_q * w.ring_chunks
        q, k, v = draw_normal(w.seed, [(w.n, full, w.h, w.d),
                                       (w.n, full, w.h_kv, w.d),
                                       (w.n, full, w.h_kv, w.d)])
        if w.dtype == "bf16":
            q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
        c = w.l_q
        r = w.ring_rank
        out = {
            "q": np.ascontiguousarray(q[:, r * c:(r + 1) * c]),
            "q_offset": r * c,
            "k_chunks": [np.ascontiguousarray(k[:, s * c:(s + 1) * c])
                         for s in range(w.ring_chunks)],
            "v_chunks": [np.ascontiguousarray(v[:, s * c:(s + 1) * c])
                         for s in range(w.ring_chunks)],
            "k_offsets": [s * c for s in range(w.ring_chunks)],
            "k_full": k, "v_full": v,
        }
        return out
    shapes = [(w.n, w.l_q, w.h, w.d), (w.n, w.l_k, w.h_kv, w.d),
              (w.n, w.l_k, w.h_kv, w.d)]
    if w.backward:
        shapes.append((w.n, w.l_q, w.h, w.d))
    arrs = draw_normal(w.seed, shapes)
    if w.dtype == "bf16":
        arrs = [round_to_bf16(a) for a in arrs]
    out = {"q": arrs[0], "k": arrs[1], "v": arrs[2]}
    if w.backward:
        out["do"] = arrs[3]
    return out
