"""Algorithmic work of the attention path, for throughput figures.

FLOPs count the work the method must do: 4*d per allowed (query, key) pair
per query head in the forward (two contractions, S = Q K^T and O = P V) and
10*d per pair in the backward (five contractions, including the recompute of
S).  Bytes are the minimal HBM traffic: each input read once, each output
written once.
"""
from __future__ import annotations

import numpy as np


def allowed_pairs(l_q, l_k, causal, win_l=-1, win_r=-1, q_offset=0,
                  k_offset=0):
    """Number of (i, j) with key j allowed for query row i, by rows: row i
    sees j in [i + dlo, i + dhi] intersected with [0, l_k)."""
    delta = int(q_offset) - int(k_offset)
    big = 1 << 62
    hi = big
    if causal:
        hi = delta
    if win_r >= 0:
        hi = min(hi, delta + win_r)
    lo = delta - win_l if win_l >= 0 else -big
    i = np.arange(l_q, dtype=np.int64)
    jlo = np.maximum(0, i + max(lo, -big // 2))
    jhi = np.minimum(l_k - 1, i + min(hi, big // 2))
    return int(np.maximum(0, jhi - jlo + 1).sum())


def fwd_flops(n, h, d, pairs):
    return 4.0 * d * pairs * n * h


def bwd_flops(n, h, d, pairs):
    return 10.0 * d * pairs * n * h


def fwd_bytes(n, l_q, l_k, h, h_kv, d, elem):
    """q read, k and v read, out written (elem bytes each), lse written."""
    return (2 * n * l_q * h * d + 2 * n * l_k * h_kv * d) * elem + 4 * n * h * l_q


def merge_bytes(n, l, h, d, blk_elem):
    """acc read + written (fp32), block read, both LSEs read, LSE written."""
    return n * l * h * d * (8 + blk_elem) + 12 * n * h * l
