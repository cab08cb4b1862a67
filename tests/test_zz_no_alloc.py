"""attn_bwd_static, the backward for callers that cannot allocate: through
the C ABI it must give attn_bwd's gradients bit for bit (same kernels, the
workspace in the library's static per-device array instead of the
caller's), on consecutive calls that reuse the array with different sizes,
and allocate no device memory."""
import math

import pytest
import torch

from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd._lib import ATTN_BWD_STATIC_MAX_WORKSPACE
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def problem(seed, n, l, h, h_kv, d):
    q, k, v, do = (round_to_bf16(x) for x in draw_normal(
        seed, [(n, l, h, d), (n, l, h_kv, d), (n, l, h_kv, d), (n, l, h, d)]))
    return [dev(x, "bf16") for x in (q, k, v, do)]


CASES = [
    # n, l, h, h_kv, d, causal, window; the first needs split dK/dV partials
    (1, 1000, 8, 2, 128, True, (-1, -1)),
    (2, 300, 4, 4, 64, True, (64, 0)),
]


def test_static_workspace_matches_attn_bwd_on_consecutive_calls():
    # references first (attn_bwd with its own workspace), then the two static
    # calls back to back, the second on smaller sizes than the first
    runs = []
    for i, (n, l, h, h_kv, d, causal, window) in enumerate(CASES):
        need = A.bwd_workspace_bytes(n, l, l, h, h_kv, d)
        assert 0 < need <= ATTN_BWD_STATIC_MAX_WORKSPACE
        tq, tk, tv, tdo = problem(900 + i, n, l, h, h_kv, d)
        scale = 1.0 / math.sqrt(d)
        o, lse = A.attention_forward(tq, tk, tv, scale, causal, window)
        ref = A.attention_backward(tdo, tq, tk, tv, o, lse, scale, causal, window)
        got = tuple(torch.full_like(g, float("nan")) for g in ref)
        runs.append((tdo, tq, tk, tv, o, lse, got, ref, scale, causal, window, need))
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    for i, (tdo, tq, tk, tv, o, lse, got, _, scale, causal, window, need) in enumerate(runs):
        say(f"[no-alloc bwd] call {i}: {CASES[i]}, workspace {need} bytes")
        A.attn_bwd_static(tdo, tq, tk, tv, o, lse, *got, scale, causal, window[0],
                          window[1])
    torch.cuda.synchronize()
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    assert after == before, "the static backward allocated device memory"
    for i, run in enumerate(runs):
        got, ref = run[6], run[7]
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g, r), f"call {i}: {name} differs from attn_bwd"
