"""GPU parity of the forward pass, the merge and the ring share against the
fp64 oracle, through the C ABI (blockwise_exact_attention_amd.attention).

Sizes: the five workloads at their full shapes (the oracle computes every
output where that takes seconds, and sampled heads or rows otherwise), plus
small cases that span several tiles, ragged tails, every mask mode, grouped
and multi-query heads and the degenerate cases (one key, one query, empty
rows, zero and negative scale)."""
import math

import numpy as np
import pytest
import torch

import oracle
from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from blockwise_exact_attention_amd.workloads import WORKLOADS, make_inputs
from gpu_util import check_o_lse, dev, host, say

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, dtype, scale, causal=False, wl=-1, wr=-1, qo=0, ko=0):
    tq, tk, tv = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    o, lse = A.attention_forward(tq, tk, tv, scale, causal, (wl, wr), qo, ko)
    torch.cuda.synchronize()
    return host(o), host(lse)


def rand_inputs(seed, n, l_q, l_k, h, h_kv, d, dtype):
    q, k, v = draw_normal(seed, [(n, l_q, h, d), (n, l_k, h_kv, d),
                                 (n, l_k, h_kv, d)])
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


# ---------------------------------------------------------------- workloads

def test_c1_tiny_fp32():
    w = WORKLOADS["C1"]
    say(f"[C1] {w}")
    x = make_inputs(w)
    o, lse = run_fwd(x["q"], x["k"], x["v"], "f32", w.softmax_scale, w.causal)
    ro, rl = oracle.attention_fwd(x["q"], x["k"], x["v"], w.softmax_scale,
                                  w.causal)
    check_o_lse(o, lse, ro, rl, "f32", "C1")


def test_c2_causal_mha_full():
    w = WORKLOADS["C2"]
    say(f"[C2] {w}")
    x = make_inputs(w)
    o, lse = run_fwd(x["q"], x["k"], x["v"], "bf16", w.softmax_scale, True)
    ro, rl = oracle.attention_fwd(x["q"], x["k"], x["v"], w.softmax_scale, True)
    check_o_lse(o, lse, ro, rl, "bf16", "C2")


def test_mqa_at_the_c2_shape_full():
    """The multi-query variant the benchmark also times (2 x 2048 tokens, 16
    query heads reading one key/value head, d = 128, causal): every head and
    row against the oracle."""
    q, k, v = (round_to_bf16(x) for x in draw_normal(
        203, [(2, 2048, 16, 128), (2, 2048, 1, 128), (2, 2048, 1, 128)]))
    scale = 1.0 / math.sqrt(128)
    o, lse = run_fwd(q, k, v, "bf16", scale, True)
    ro, rl = oracle.attention_fwd(q, k, v, scale, True)
    check_o_lse(o, lse, ro, rl, "bf16", "MQA at the C2 shape")


def test_c3_ring_share():
    """Rank 7 of 8: the merged share equals rows 7168..8191 of causal
    attention over the full 8192-token sequence, on every head and row."""
    w = WORKLOADS["C3"]
    say(f"[C3] {w}")
    x = make_inputs(w)
    tq = dev(x["q"], "bf16")
    kc = [dev(c, "bf16") for c in x["k_chunks"]]
    vc = [dev(c, "bf16") for c in x["v_chunks"]]
    share = A.RingShare(tq, w.softmax_scale, True, x["q_offset"])
    heads = None  # all 32
    q_full_rows = x["q"]
    ro, rl = oracle.attention_fwd(q_full_rows, x["k_full"], x["v_full"],
                                  w.softmax_scale, True, -1, -1,
                                  x["q_offset"], 0, heads=heads, block=1024)
    for fused, one in ((False, False), (True, False), (False, True)):
        out, lse_acc = share.run(kc, vc, x["k_offsets"], fused=fused, one_launch=one)
        torch.cuda.synchronize()
        o, lse = host(out), host(lse_acc)
        check_o_lse(o, lse, ro, rl, "bf16",
                    f"C3 ring share (fused={fused}, one launch={one}) vs full-sequence rows")
    # the all-gather form: the chunks side by side, one call with the offset
    o, lse = run_fwd(x["q"], x["k_full"], x["v_full"], "bf16", w.softmax_scale,
                     True, -1, -1, x["q_offset"], 0)
    check_o_lse(o, lse, ro, rl, "bf16", "C3 share, all-gathered K/V in one call")
    # the single steps too: step 0 (wholly in the past) and step 7 (diagonal)
    for s in (0, 7):
        ob, lb = run_fwd(x["q"], x["k_chunks"][s], x["v_chunks"][s], "bf16",
                         w.softmax_scale, True, -1, -1, x["q_offset"],
                         x["k_offsets"][s])
        rob, rlb = oracle.attention_fwd(x["q"], x["k_chunks"][s],
                                        x["v_chunks"][s], w.softmax_scale,
                                        True, -1, -1, x["q_offset"],
                                        x["k_offsets"][s], heads=heads)
        check_o_lse(ob, lb, rob, rlb, "bf16", f"C3 step {s}")


def test_c4_sliding_window_full():
    w = WORKLOADS["C4"]
    say(f"[C4] {w}")
    x = make_inputs(w)
    o, lse = run_fwd(x["q"], x["k"], x["v"], "bf16", w.softmax_scale, True,
                     w.win_l, w.win_r)
    ro, rl = oracle.attention_fwd(x["q"], x["k"], x["v"], w.softmax_scale,
                                  True, w.win_l, w.win_r, block=256)
    check_o_lse(o, lse, ro, rl, "bf16", "C4")


def test_c5_forward_full():
    """The 16384-token causal workload at full size, every head and row (the
    oracle goes head by head, about two seconds each on a 16-thread host)."""
    w = WORKLOADS["C5"]
    say(f"[C5 fwd] {w}")
    x = make_inputs(w)
    o, lse = run_fwd(x["q"], x["k"], x["v"], "bf16", w.softmax_scale, True)
    for hq in range(w.h):
        ro, rl = oracle.attention_fwd(x["q"], x["k"], x["v"], w.softmax_scale,
                                      True, heads=[(0, hq)], block=1024)
        check_o_lse(o, lse, ro, rl, "bf16", f"C5 forward head {hq}")


# ---------------------------------------------------------------- small cases

SMALL = [
    # n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko
    (1, 200, 333, 4, 2, 128, False, -1, -1, 0, 0),
    (2, 300, 300, 4, 4, 64, True, -1, -1, 0, 0),
    (1, 257, 513, 8, 2, 128, True, -1, -1, 256, 0),     # bottom-right-ish
    (1, 130, 700, 3, 1, 64, True, 40, 7, 100, 0),       # MQA + window
    (2, 256, 256, 2, 2, 128, True, 0, 0, 0, 0),         # diagonal only
    (1, 190, 190, 2, 1, 128, False, 31, 31, 0, 0),
    (1, 96, 160, 4, 4, 64, True, -1, -1, 0, 64),        # rows 0..63 empty
    (1, 64, 64, 2, 2, 128, True, -1, -1, 0, 1000),      # every row empty
    (1, 1, 1, 1, 1, 64, False, -1, -1, 0, 0),
    (1, 1, 300, 2, 1, 128, True, -1, -1, 299, 0),       # single query, last
    (1, 300, 1, 2, 2, 64, False, -1, -1, 0, 0),         # single key
    (2, 129, 129, 8, 1, 64, False, -1, 5, 0, 0),        # right window only
    (1, 512, 512, 16, 8, 128, True, -1, -1, 0, 0),      # n*h_kv % 8 == 0 path
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", SMALL)
def test_small_cases(case, dtype):
    n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko = case
    say(f"[small] {case} {dtype}")
    q, k, v = rand_inputs(7 + l_q + l_k + h + d, n, l_q, l_k, h, h_kv, d, dtype)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_fwd(q, k, v, dtype, scale, causal, wl, wr, qo, ko)
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal, wl, wr, qo, ko)
    check_o_lse(o, lse, ro, rl, dtype, str(case))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [0.0, -0.09, 0.4])
def test_scale_values(scale, dtype):
    q, k, v = rand_inputs(99, 1, 160, 200, 2, 2, 128, dtype)
    o, lse = run_fwd(q, k, v, dtype, scale, True, -1, -1, 40, 0)
    ro, rl = oracle.attention_fwd(q, k, v, scale, True, -1, -1, 40, 0)
    check_o_lse(o, lse, ro, rl, dtype, f"scale={scale}")


def test_forward_is_deterministic():
    q, k, v = rand_inputs(3, 1, 1024, 1024, 8, 2, 128, "bf16")
    tq, tk, tv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o1, l1 = A.attention_forward(tq, tk, tv, 0.088, True)
    o2, l2 = A.attention_forward(tq, tk, tv, 0.088, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_large_offsets():
    q, k, v = rand_inputs(4, 1, 100, 100, 2, 2, 64, "bf16")
    for qo, ko in [(2**40 + 50, 2**40), (-(2**50), -(2**50) + 30),
                   (2**62, -(2**62)), (-(2**62), 2**62)]:
        o, lse = run_fwd(q, k, v, "bf16", 0.125, True, -1, -1, qo, ko)
        dq = max(min(qo - ko, 10**6), -10**6)
        ro, rl = oracle.attention_fwd(q, k, v, 0.125, True, -1, -1, dq, 0)
        check_o_lse(o, lse, ro, rl, "bf16", f"offsets {qo},{ko}")


@pytest.mark.parametrize("case", [
    # n, l_q, l_k, h, h_kv, d, causal, q_offset, rows checked (None = all)
    (1, 65536, 65536, 1, 1, 64, True, 0, [0, 1, 127, 128, 4095, 32768, 65534, 65535]),
    (300, 17, 17, 3, 1, 128, False, 0, None),
    (1, 1, 65536, 4, 2, 128, True, 65535, None),      # one query at the end (decode-like)
    (1, 65536, 1, 2, 2, 64, True, 0, [0, 1, 2, 65535]),  # one key
    (2, 129, 40000, 4, 1, 128, True, 39871, None),  # chunk at the end of a long key range
])
def test_shape_extremes(case):
    """Very long and very short sequences, many tiny heads and batches, a
    single query or key: grid mapping, tile bounds and tails."""
    n, l_q, l_k, h, h_kv, d, causal, qo, rows = case
    say(f"[extremes] {case[:8]}")
    q, k, v = rand_inputs(77, n, l_q, l_k, h, h_kv, d, "bf16")
    o, lse = run_fwd(q, k, v, "bf16", 0.11, causal, -1, -1, qo, 0)
    heads = None if rows is None else [(0, 0), (n - 1, h - 1)]
    ro, rl = oracle.attention_fwd(q, k, v, 0.11, causal, -1, -1, qo, 0, heads=heads,
                                  rows=rows)
    check_o_lse(o, lse, ro, rl, "bf16", f"extremes {case[:8]}")


# ---------------------------------------------------------------- merge

def _partial(rng, n, l, h, d, p_empty):
    o = rng.standard_normal((n, l, h, d)).astype(np.float32)
    lse = (rng.standard_normal((n, h, l)) * 4).astype(np.float32)
    empty = rng.random((n, h, l)) < p_empty
    lse[empty] = -np.inf
    o[np.transpose(empty, (0, 2, 1))] = 0.0
    return o, lse


@pytest.mark.parametrize("d", [128, 64, 256, 5])
@pytest.mark.parametrize("blk_dtype", ["bf16", "f32"])
def test_merge_parity(d, blk_dtype):
    rng = np.random.default_rng(d)
    n, l, h = 2, 77, 3
    oa, la = _partial(rng, n, l, h, d, 0.2)
    ob, lb = _partial(rng, n, l, h, d, 0.2)
    if blk_dtype == "bf16":
        ob = round_to_bf16(ob)
    acc = torch.from_numpy(oa).cuda()
    lacc = torch.from_numpy(la).cuda()
    # an accumulator row with LSE -inf must be overwritten, whatever it holds
    acc_np_nan = oa.copy()
    acc_np_nan[np.transpose(np.isneginf(la), (0, 2, 1))] = np.nan
    acc.copy_(torch.from_numpy(acc_np_nan))
    A.attn_merge(acc, lacc, dev(ob, blk_dtype),
                 torch.from_numpy(lb).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.merge(oa, la, ob, lb)
    go, gl = host(acc), host(lacc)
    # every row, the both-empty ones included (there the merge gives O = 0,
    # whatever the accumulator held: NaN above)
    both = np.isneginf(la) & np.isneginf(lb)
    assert both.any()
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.max(np.abs(gl[fin] - rl[fin])) < 2e-6
    assert np.all(np.isfinite(go))
    assert np.max(np.abs(go - ro)) < 2e-5


def test_acc_init_and_cast():
    n, l, h, d = 1, 33, 3, 64
    acc = torch.full((n, l, h, d), 7.0, device="cuda")
    lse = torch.zeros((n, h, l), device="cuda")
    A.attn_acc_init(acc, lse)
    torch.cuda.synchronize()
    assert torch.all(acc == 0) and torch.all(torch.isneginf(lse))
    x = torch.randn((n, l, h, d), device="cuda") * 3
    out = torch.empty((n, l, h, d), dtype=torch.bfloat16, device="cuda")
    A.attn_acc_cast(x, out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), x.cpu().to(torch.bfloat16))
    out32 = torch.empty((n, l, h, d), dtype=torch.float32, device="cuda")
    A.attn_acc_cast(x, out32)
    torch.cuda.synchronize()
    assert torch.equal(out32, x)
    # an accumulator 4 bytes past a 16-byte boundary, with a ragged size: the
    # scalar stores cover it all and nothing beyond it
    buf = torch.full((1 + 5 * 3 * 7 + 1,), 7.0, device="cuda")
    acc_u = buf[1:-1].view(1, 5, 3, 7)
    lse_u = torch.zeros((1, 3, 5), device="cuda")
    A.attn_acc_init(acc_u, lse_u)
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[1:-1] == 0) and b[0] == 7.0 and b[-1] == 7.0
    assert torch.all(torch.isneginf(lse_u))


@pytest.mark.parametrize("d,fused", [(128, False), (128, True), (64, True)])
def test_small_ring_share_gqa(d, fused):
    """A small ring (P = 4 chunks of 96) on every rank, against causal
    attention over the whole sequence; separate and fused ring steps."""
    P, c, h, h_kv = 4, 96, 8, 2
    q, k, v = rand_inputs(21, 1, P * c, P * c, h, h_kv, d, "bf16")
    ro, rl = oracle.attention_fwd(q, k, v, 0.1, True)
    kc = [dev(k[:, s * c:(s + 1) * c], "bf16") for s in range(P)]
    vc = [dev(v[:, s * c:(s + 1) * c], "bf16") for s in range(P)]
    for r in range(P):
        tq = dev(q[:, r * c:(r + 1) * c], "bf16")
        out, lse = A.ring_share(tq, kc, vc, [s * c for s in range(P)], r * c,
                                0.1, True, fused=fused)
        torch.cuda.synchronize()
        check_o_lse(host(out), host(lse), ro[:, r * c:(r + 1) * c],
                    rl[:, :, r * c:(r + 1) * c], "bf16", f"ring rank {r}")



@pytest.mark.parametrize("d,h_kv,causal,window,fused", [
    (128, 1, True, (100, 0), False),
    (64, 1, True, (100, 0), True),
    (128, 2, False, (50, 30), True),
])
def test_ring_share_sliding_window(d, h_kv, causal, window, fused):
    """Sliding-window attention in ring mode (P = 4 chunks of 96, multi-query
    and grouped heads): each rank's share equals its rows of windowed
    attention over the whole sequence; chunks wholly outside a rank's window
    are empty steps that must leave the accumulator alone."""
    P, c, h = 4, 96, 8
    q, k, v = rand_inputs(23 + d + h_kv, 1, P * c, P * c, h, h_kv, d, "bf16")
    scale = 1.0 / math.sqrt(d)
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal, window[0], window[1])
    kc = [dev(k[:, s * c:(s + 1) * c], "bf16") for s in range(P)]
    vc = [dev(v[:, s * c:(s + 1) * c], "bf16") for s in range(P)]
    for r in range(P):
        tq = dev(q[:, r * c:(r + 1) * c], "bf16")
        out, lse = A.ring_share(tq, kc, vc, [s * c for s in range(P)], r * c,
                                scale, causal, fused=fused, window=window)
        torch.cuda.synchronize()
        check_o_lse(host(out), host(lse), ro[:, r * c:(r + 1) * c],
                    rl[:, :, r * c:(r + 1) * c], "bf16", f"window ring rank {r}")

FWD_ACC_CASES = [
    # n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko
    (1, 300, 257, 8, 2, 128, True, -1, -1, 0, 100),   # rows 0..99 see no key
    (2, 190, 333, 4, 4, 64, True, 40, 7, 120, 0),     # window, ragged tiles
    (1, 1024, 512, 64, 8, 128, False, -1, -1, 0, 0),  # one 4-wave group per tile
    (1, 128, 1024, 2, 1, 128, True, -1, -1, 896, 0),  # two key groups per tile
]


@pytest.mark.parametrize("case", FWD_ACC_CASES)
def test_fwd_acc_merges_into_accumulator(case):
    """attn_fwd_acc on an accumulator holding a previous partial result (some
    rows empty, with NaN in their O) equals the fp64 merge of that
    accumulator with the oracle's attention over this chunk."""
    n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko = case
    say(f"[fwd_acc] {case}")
    q, k, v = rand_inputs(31 + l_q + d, n, l_q, l_k, h, h_kv, d, "bf16")
    rng = np.random.default_rng(l_q + l_k)
    acc0 = rng.standard_normal((n, l_q, h, d)).astype(np.float32)
    lse0 = (rng.standard_normal((n, h, l_q)) * 3).astype(np.float32)
    empty = rng.random((n, h, l_q)) < 0.25
    lse0[empty] = -np.inf
    acc_in = acc0.copy()
    acc_in[np.transpose(empty, (0, 2, 1))] = np.nan
    heads = [(b, hq) for b in range(n) for hq in sorted({0, h // 2, h - 1})]
    scale = 1.0 / math.sqrt(d)
    ob, lb = oracle.attention_fwd(q, k, v, scale, causal, wl, wr, qo, ko,
                                  heads=heads)
    sel = ~np.isnan(lb)
    # rows outside the sampled heads: keep them out of the reference merge
    lb_m = np.where(sel, lb, -np.inf)
    ob_m = np.where(np.isnan(ob), 0.0, ob)
    acc0_clean = np.where(np.isnan(acc_in), 0.0, acc_in)
    ro, rl = oracle.merge(acc0_clean, lse0, ob_m, lb_m)
    # every sampled row against the merge (where the accumulator row is
    # empty its NaN content must not leak: the merge there is the block, or
    # O = 0 when this chunk gives the row no key either); besides, a row
    # with a result and no allowed key in this chunk is left bit for bit
    keep = sel & np.isneginf(lb) & ~empty
    cleared = sel & np.isneginf(lb) & empty
    ro = np.where(np.transpose(sel, (0, 2, 1))[..., None], ro, np.nan)
    rl = np.where(sel, rl, np.nan)
    acc = torch.from_numpy(acc_in).cuda()
    lse_acc = torch.from_numpy(lse0).cuda()
    A.attn_fwd_acc(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), acc, lse_acc,
                   scale, causal, wl, wr, qo, ko)
    torch.cuda.synchronize()
    go, gl = acc.cpu().numpy(), lse_acc.cpu().numpy()
    check_o_lse(go.astype(np.float64), gl.astype(np.float64), ro, rl, "bf16",
                str(case))
    kr = np.transpose(keep, (0, 2, 1))
    assert np.array_equal(go[kr], acc_in[kr])
    assert np.array_equal(gl[keep], lse0[keep])
    cr = np.transpose(cleared, (0, 2, 1))
    assert np.all(go[cr] == 0.0) and np.all(np.isneginf(gl[cleared]))
