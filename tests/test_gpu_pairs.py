"""GPU parity of the paired schedule of the pipelined forward against the
fp64 oracle.  Under a causal mask attn_fwd pairs q tiles r and n-1-r in one
workgroup (r first, then n-1-r, both with two key groups on alternate key
tiles), when the grid is large enough for pairing to pay.  The cases cover an
odd number of q tiles (the middle tile alone), a ragged last tile, grouped and
single key/value heads, d = 64 and 128, keys ahead of the queries, offsets
that leave the first q tiles without any key, and a window (unpaired)."""
import math

import pytest

import oracle
from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from gpu_util import check_o_lse, dev, host, say

pytestmark = pytest.mark.gpu

CASES = [
    # n, l_q, l_k, h, h_kv, d, window, q_offset, k_offset (enough heads that
    # the paired schedule is the one chosen)
    (2, 1664, 1664, 24, 6, 128, (-1, -1), 0, 0),    # 13 q tiles: the middle one alone
    (2, 1500, 1500, 24, 1, 64, (-1, -1), 0, 0),     # ragged last q tile, MQA
    (1, 1536, 1836, 48, 8, 128, (-1, -1), 300, 0),  # keys ahead of the queries
    (1, 1792, 1792, 48, 4, 128, (-1, -1), 0, 200),  # first q tiles without any key
    (1, 2048, 2048, 32, 4, 64, (1500, 0), 0, 0),    # causal window (unpaired)
]


@pytest.mark.parametrize("case", CASES)
def test_paired_schedule(case):
    n, l_q, l_k, h, h_kv, d, window, qo, ko = case
    say(f"[pairs] {case}")
    q, k, v = (round_to_bf16(x) for x in draw_normal(
        301 + l_q + d, [(n, l_q, h, d), (n, l_k, h_kv, d), (n, l_k, h_kv, d)]))
    scale = 1.0 / math.sqrt(d)
    name = A.fwd_kernel_name(n, l_q, l_k, h, h_kv, d, True, window[0], window[1], qo, ko)
    say(f"  kernel {name}")
    tq, tk, tv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o, lse = A.attention_forward(tq, tk, tv, scale, True, window, qo, ko)
    ro, rl = oracle.attention_fwd(q, k, v, scale, True, window[0], window[1], qo, ko)
    check_o_lse(host(o), host(lse), ro, rl, "bf16", f"paired schedule {case}")
    assert name == f"fwd_pipe_kernel<{d}, 2, false, false>"


def test_paired_schedule_repeatable():
    """Two launches give the same bits (the tile order and the key groups'
    merge are fixed by the shape, not by scheduling)."""
    q, k, v = (round_to_bf16(x) for x in draw_normal(
        307, [(2, 2048, 4, 128), (2, 2048, 4, 128), (2, 2048, 4, 128)]))
    tq, tk, tv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o1, l1 = A.attention_forward(tq, tk, tv, None, True)
    o2, l2 = A.attention_forward(tq, tk, tv, None, True)
    assert (o1 == o2).all() and (l1 == l2).all()
