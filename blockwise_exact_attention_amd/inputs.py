"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke
check. This module draws random numbers and rounds them to the storage dtype;
it holds none of the attention arithmetic.

Every tensor is i.i.d. N(0, 1) float32 from numpy's PCG64 generator, drawn in
the order the caller lists the shapes (q, k, v, dO), then rounded once to
bfloat16 with round-to-nearest-even when the workload is bf16.  Both the GPU
path and the oracle receive exactly these values.
"""
from __future__ import annotations

import numpy as np


def draw_normal(seed, shapes):
    """Draw float32 N(0,1) arrays of the given shapes, in order, from one
    PCG64(seed) stream."""
    gen = np.random.Generator(np.random.PCG64(int(seed)))
    return [gen.standard_normal(tuple(s), dtype=np.float32) for s in shapes]


def round_to_bf16(x):
    """Round a float32 array to the nearest bfloat16 value (ties to even) and
    return the result as float32 (every bf16 value is exact in float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    # round-to-nearest-even on the 16 dropped mantissa bits; NaN stays NaN
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(x)
    out = (rounded & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    return np.where(nan, x, out)


def bf16_bits(x):
    """uint16 storage bits of a float32 array whose values are already bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(bits):
    """float32 values of an array of bf16 storage bits."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)
