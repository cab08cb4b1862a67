"""GPU parity of the one-launch ring share (attn_fwd_ring) against the fp64
oracle: the share over P chunks must equal attention over the keys of all
chunks together (flash_sharding.py ring_fwd; picotron ring_attention_forward),
whatever the chunk boundaries, their order, empty chunks, ragged lengths,
masks and head layouts.  Also the pipelined kernel on single long chunks
(attn_fwd and the fused step pick it for long key loops)."""
import math

import numpy as np
import pytest
import torch

import oracle
from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd._lib import ATTN_RING_MAX_CHUNKS
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from gpu_util import check_o_lse, dev, host, say

pytestmark = pytest.mark.gpu


def rand(seed, shapes):
    return [round_to_bf16(x) for x in draw_normal(seed, shapes)]


def run_ring(q, k, v, bounds, order, scale, causal, wl, wr, qo, ko):
    """Split k, v at the key indices `bounds` (chunk c = keys
    bounds[c]..bounds[c+1]-1, at absolute offset ko + bounds[c]) and run the
    share with the chunks in `order`."""
    tq = dev(q, "bf16")
    kc = [dev(k[:, bounds[c]:bounds[c + 1]], "bf16") for c in order]
    vc = [dev(v[:, bounds[c]:bounds[c + 1]], "bf16") for c in order]
    offs = [ko + bounds[c] for c in order]
    out = torch.empty_like(tq)
    lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32,
                      device="cuda")
    A.attn_fwd_ring(tq, kc, vc, offs, out, lse, scale, causal, wl, wr, qo)
    torch.cuda.synchronize()
    return host(out), host(lse)


def splits(rng, l_k, n_chunks):
    cuts = sorted(int(x) for x in rng.integers(0, l_k + 1, n_chunks - 1))
    return [0, *cuts, l_k]


SMALL = [
    # n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko
    (1, 200, 333, 4, 2, 128, False, -1, -1, 0, 0),
    (2, 300, 300, 4, 4, 64, True, -1, -1, 0, 0),
    (1, 257, 513, 8, 2, 128, True, -1, -1, 256, 0),
    (1, 130, 700, 3, 1, 64, True, 40, 7, 100, 0),       # MQA + window
    (2, 256, 256, 2, 2, 128, True, 0, 0, 0, 0),         # diagonal only
    (1, 96, 160, 4, 4, 64, True, -1, -1, 0, 64),        # rows 0..63 empty
    (1, 64, 64, 2, 2, 128, True, -1, -1, 0, 1000),      # every row empty
    (1, 1, 300, 2, 1, 128, True, -1, -1, 299, 0),       # single query
    (1, 300, 1, 2, 2, 64, False, -1, -1, 0, 0),         # single key
    (1, 512, 512, 16, 8, 128, True, -1, -1, 0, 0),      # n*h_kv % 8 == 0 path
]


@pytest.mark.parametrize("case", SMALL)
def test_ring_equals_attention_over_all_chunks(case):
    n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko = case
    q, k, v = rand(11 + l_q + l_k + h + d, [(n, l_q, h, d), (n, l_k, h_kv, d),
                                            (n, l_k, h_kv, d)])
    scale = 1.0 / math.sqrt(d)
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal, wl, wr, qo, ko)
    rng = np.random.default_rng(l_q * 7 + l_k)
    layouts = [("one chunk", [0, l_k], [0])]
    for nc in (2, 3, 5):
        b = splits(rng, l_k, nc)
        layouts.append((f"{nc} chunks at {b}", b, list(range(nc))))
    b = splits(rng, l_k, 4)
    layouts.append((f"4 chunks reversed at {b}", b, [3, 2, 1, 0]))
    b = [0, l_k // 2, l_k // 2, l_k]     # an empty chunk in the middle
    layouts.append(("an empty chunk", b, [0, 1, 2]))
    for what, bounds, order in layouts:
        say(f"[ring] {case}: {what}")
        o, lse = run_ring(q, k, v, bounds, order, scale, causal, wl, wr, qo, ko)
        check_o_lse(o, lse, ro, rl, "bf16", f"{case} {what}")


@pytest.mark.parametrize("seed", range(300, 316))
def test_ring_random(seed):
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 128]))
    h_kv = int(r.choice([1, 2, 4]))
    h = h_kv * int(r.choice([1, 2, 4]))
    n = int(r.integers(1, 3))
    l_q = int(r.integers(1, 400))
    l_k = int(r.integers(1, 900))
    nc = int(r.integers(1, ATTN_RING_MAX_CHUNKS + 1))
    causal = bool(r.integers(0, 2))
    wl = int(r.choice([-1, -1, 0, 17, 130]))
    wr = int(r.choice([-1, -1, 0, 9, 70]))
    qo = int(r.integers(-50, 900))
    ko = int(r.integers(-50, 300))
    scale = float(r.choice([1.0 / math.sqrt(d), 0.3, -0.05, 0.0]))
    bounds = splits(r, l_k, nc)
    order = [int(x) for x in r.permutation(nc)]
    case = (n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko, scale, bounds, order)
    say(f"[ring random] seed {seed}: {case}")
    q, k, v = rand(seed, [(n, l_q, h, d), (n, l_k, h_kv, d), (n, l_k, h_kv, d)])
    o, lse = run_ring(q, k, v, bounds, order, scale, causal, wl, wr, qo, ko)
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal, wl, wr, qo, ko)
    check_o_lse(o, lse, ro, rl, "bf16", f"seed {seed}")


@pytest.mark.parametrize("d,h_kv,window", [(128, 2, (-1, -1)), (64, 1, (-1, -1)),
                                           (128, 4, (100, 0))])
def test_small_ring_every_rank(d, h_kv, window):
    """P = 4 ranks, chunks of 160 tokens, causal: each rank's one-launch share,
    with the chunks in ring order, equals its rows of attention over the
    whole sequence."""
    P, c, h = 4, 160, 8
    L = P * c
    q, k, v = rand(51 + d + h_kv, [(1, L, h, d), (1, L, h_kv, d), (1, L, h_kv, d)])
    scale = 1.0 / math.sqrt(d)
    kc = [dev(k[:, s * c:(s + 1) * c], "bf16") for s in range(P)]
    vc = [dev(v[:, s * c:(s + 1) * c], "bf16") for s in range(P)]
    offs = [s * c for s in range(P)]
    ro, rl = oracle.attention_fwd(q, k, v, scale, True, window[0], window[1])
    for r in range(P):
        say(f"[ring ranks] d={d} h_kv={h_kv} window={window} rank {r}")
        tq = dev(q[:, r * c:(r + 1) * c], "bf16")
        # ring order: the rank's own chunk first, then those passed along
        order = [(r - s) % P for s in range(P)]
        share = A.RingShare(tq, scale, True, r * c, window)
        out, lse = share.run([kc[s] for s in order], [vc[s] for s in order],
                             [offs[s] for s in order], one_launch=True)
        torch.cuda.synchronize()
        check_o_lse(host(out), host(lse), ro[:, r * c:(r + 1) * c],
                    rl[:, :, r * c:(r + 1) * c], "bf16", f"rank {r} one launch")


def test_sixteen_chunks_and_the_limit():
    q, k, v = rand(61, [(1, 200, 4, 128), (1, 1000, 2, 128), (1, 1000, 2, 128)])
    bounds = [round(i * 1000 / 16) for i in range(17)]
    o, lse = run_ring(q, k, v, bounds, list(range(16)), 0.09, True, -1, -1, 800, 0)
    ro, rl = oracle.attention_fwd(q, k, v, 0.09, True, -1, -1, 800, 0)
    check_o_lse(o, lse, ro, rl, "bf16", "16 chunks")
    tq = dev(q, "bf16")
    kc = [dev(k[:, :10], "bf16")] * (ATTN_RING_MAX_CHUNKS + 1)
    out = torch.empty_like(tq)
    lse_t = torch.empty((1, 4, 200), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        A.attn_fwd_ring(tq, kc, kc, [0] * len(kc), out, lse_t, 0.09)


def test_ring_without_any_key():
    q, = rand(62, [(2, 70, 4, 64)])
    tq = dev(q, "bf16")
    empty = torch.zeros((2, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(tq, float("nan"))
    lse = torch.zeros((2, 4, 70), dtype=torch.float32, device="cuda")
    A.attn_fwd_ring(tq, [empty, empty], [empty, empty], [0, 5], out, lse, 0.1, True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("d,h,h_kv,causal,window", [
    (128, 4, 2, True, (-1, -1)),
    (64, 2, 1, False, (-1, -1)),
    (128, 2, 2, True, (6000, 0)),
])
def test_pipelined_kernel_on_long_chunks(d, h, h_kv, causal, window):
    """Key loops long enough (12 and more key tiles per 128-row q tile on
    average) that attn_fwd and the fused step run the pipelined kernel: its plain and
    accumulating epilogues against the oracle, ragged lengths, and the
    one-chunk share (always the pipelined kernel) bit-equal to attn_fwd."""
    l_q, l_k = 333, 9001
    qo = l_k - l_q
    q, k, v = rand(71 + d + h, [(1, l_q, h, d), (1, l_k, h_kv, d), (1, l_k, h_kv, d)])
    scale = 1.0 / math.sqrt(d)
    say(f"[pipe long] d={d} h={h} h_kv={h_kv} causal={causal} window={window}")
    tq, tk, tv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o, lse = A.attention_forward(tq, tk, tv, scale, causal, window, qo, 0)
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal, window[0], window[1], qo, 0)
    torch.cuda.synchronize()
    check_o_lse(host(o), host(lse), ro, rl, "bf16", "attn_fwd, long chunk")
    o1 = torch.empty_like(tq)
    l1 = torch.empty_like(lse)
    A.attn_fwd_ring(tq, [tk], [tv], [0], o1, l1, scale, causal, window[0], window[1], qo)
    torch.cuda.synchronize()
    assert torch.equal(o1, o) and torch.equal(l1, lse)
    # fused step into a random accumulator, a third of its rows empty
    rng = np.random.default_rng(d + h)
    acc0 = rng.standard_normal((1, l_q, h, d)).astype(np.float32)
    lse0 = (rng.standard_normal((1, h, l_q)) * 2).astype(np.float32)
    lse0[rng.random((1, h, l_q)) < 0.33] = -np.inf
    acc = torch.from_numpy(acc0).cuda()
    lacc = torch.from_numpy(lse0).cuda()
    A.attn_fwd_acc(tq, tk, tv, acc, lacc, scale, causal, window[0], window[1], qo, 0)
    torch.cuda.synchronize()
    mo, ml = oracle.merge(acc0, lse0, ro, rl)
    check_o_lse(host(acc), host(lacc), mo, ml, "bf16", "fused step, long chunk")
