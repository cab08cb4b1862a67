"""GPU parity of the backward pass (dQ, dK, dV) against the fp64 oracle,
through the C ABI.  The GPU backward consumes the GPU forward's bf16 O and
fp32 LSE, as the ring backward on the pages does with the saved out and
softmax_lse; the oracle recomputes everything in fp64 from q, k, v and dO.

Tolerance (the pages give none for gradients): max |g - g_ref| <=
2e-2 * max(1, max |g_ref|) per gradient, the forward's bf16 bound scaled to
the gradient's magnitude; the relative Frobenius error is printed too."""
import math

import numpy as np
import pytest
import torch

import oracle
from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from blockwise_exact_attention_amd.workloads import WORKLOADS, make_inputs
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def check_grad(g, ref, name):
    sel = ~np.isnan(ref)
    assert np.all(np.isfinite(g[sel])), f"{name}: non-finite"
    scale = max(1.0, float(np.max(np.abs(ref[sel]), initial=0.0)))
    err = float(np.max(np.abs(g[sel] - ref[sel]), initial=0.0))
    fro = float(np.linalg.norm(g[sel] - ref[sel]) /
                max(np.linalg.norm(ref[sel]), 1e-30))
    say(f"  {name}: max|err| = {err:.3e} (tol {2e-2 * scale:.3e}), "
        f"rel fro = {fro:.3e}")
    assert err <= 2e-2 * scale, f"{name}: {err} > {2e-2 * scale}"
    return err


def run_fwd_bwd(q, k, v, do, scale, causal, wl=-1, wr=-1, qo=0, ko=0):
    tq, tk, tv, tdo = (dev(x, "bf16") for x in (q, k, v, do))
    o, lse = A.attention_forward(tq, tk, tv, scale, causal, (wl, wr), qo, ko)
    dq, dk, dv = A.attention_backward(tdo, tq, tk, tv, o, lse, scale, causal,
                                      (wl, wr), qo, ko)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


CASES = [
    # n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko
    (1, 256, 256, 2, 2, 128, True, -1, -1, 0, 0),
    (2, 200, 333, 4, 2, 128, False, -1, -1, 0, 0),
    (1, 300, 300, 4, 4, 64, True, -1, -1, 0, 0),
    (1, 257, 513, 8, 2, 128, True, -1, -1, 256, 0),
    (1, 130, 700, 3, 1, 64, True, 40, 7, 100, 0),
    (1, 96, 160, 4, 4, 64, True, -1, -1, 0, 64),       # empty rows
    (1, 64, 64, 2, 2, 128, True, -1, -1, 0, 1000),     # every row empty
    (1, 1, 300, 2, 1, 128, True, -1, -1, 299, 0),
    (1, 300, 1, 2, 2, 64, False, -1, -1, 0, 0),
    (2, 129, 129, 8, 1, 64, False, -1, 5, 0, 0),
    (1, 512, 384, 8, 2, 128, True, 100, 0, 0, 0),
]


@pytest.mark.parametrize("case", CASES)
def test_backward_small(case):
    n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko = case
    say(f"[bwd] {case}")
    q, k, v, do = draw_normal(11 + l_q + l_k + h, [(n, l_q, h, d),
                                                  (n, l_k, h_kv, d),
                                                  (n, l_k, h_kv, d),
                                                  (n, l_q, h, d)])
    q, k, v, do = (round_to_bf16(x) for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = run_fwd_bwd(q, k, v, do, scale, causal, wl, wr, qo, ko)
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, scale, causal, wl, wr, qo,
                                      ko)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


def test_backward_negative_scale():
    q, k, v, do = draw_normal(5, [(1, 200, 2, 128), (1, 200, 1, 128),
                                  (1, 200, 1, 128), (1, 200, 2, 128)])
    q, k, v, do = (round_to_bf16(x) for x in (q, k, v, do))
    dq, dk, dv = run_fwd_bwd(q, k, v, do, -0.07, True)
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, -0.07, True)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


@pytest.mark.parametrize("d,window", [(64, (100, 0)), (128, (-1, -1))])
def test_backward_zero_scale(d, window):
    # scale 0: every allowed key has the same weight, and dQ = scale dS K,
    # dK = scale dS^T Q vanish exactly
    q, k, v, do = draw_normal(7 + d, [(1, 200, 2, d), (1, 200, 1, d),
                                      (1, 200, 1, d), (1, 200, 2, d)])
    q, k, v, do = (round_to_bf16(x) for x in (q, k, v, do))
    dq, dk, dv = run_fwd_bwd(q, k, v, do, 0.0, True, *window)
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, 0.0, True, *window)
    assert not np.any(dq) and not np.any(dk)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


def test_backward_is_deterministic():
    q, k, v, do = draw_normal(6, [(1, 512, 4, 128), (1, 512, 2, 128),
                                  (1, 512, 2, 128), (1, 512, 4, 128)])
    tq, tk, tv, tdo = (dev(round_to_bf16(x), "bf16") for x in (q, k, v, do))
    o, lse = A.attention_forward(tq, tk, tv, 0.088, True)
    a = A.attention_backward(tdo, tq, tk, tv, o, lse, 0.088, True)
    b = A.attention_backward(tdo, tq, tk, tv, o, lse, 0.088, True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_wide_dq_ragged_grouped():
    """A backward whose dQ runs the wide form (eight waves over 256 query
    rows, d = 128, at least one 256-row workgroup per CU): ragged length
    (2200 = 8 x 256 + 152), grouped heads 32/8, causal with a query offset;
    three whole key/value groups (their 12 query heads) against the oracle."""
    n, l_q, l_k, h, h_kv, d = 1, 2200, 2300, 32, 8, 128
    q, k, v, do = draw_normal(17, [(n, l_q, h, d), (n, l_k, h_kv, d), (n, l_k, h_kv, d),
                                   (n, l_q, h, d)])
    q, k, v, do = (round_to_bf16(x) for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = run_fwd_bwd(q, k, v, do, scale, True, qo=100)
    for g in (0, 5, 7):
        rq, rk, rv = oracle.attention_bwd(q, k, v, do, scale, True, -1, -1, 100, 0,
                                          kv_heads=[(0, g)], block=1024)
        check_grad(dq, rq, f"group {g} dq")
        check_grad(dk, rk, f"group {g} dk")
        check_grad(dv, rv, f"group {g} dv")


def test_c5_backward_full():
    """Long-context workload at full size (l = 16384, 16 heads): every
    gradient of every head against the oracle (head by head, about three
    seconds each on a 16-thread host)."""
    w = WORKLOADS["C5"]
    say(f"[C5 bwd] {w}")
    x = make_inputs(w)
    dq, dk, dv = run_fwd_bwd(x["q"], x["k"], x["v"], x["do"], w.softmax_scale,
                             True)
    for g in range(w.h_kv):
        rq, rk, rv = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"],
                                          w.softmax_scale, True, kv_heads=[(0, g)],
                                          block=1024)
        check_grad(dq, rq, f"C5 head {g} dq")
        check_grad(dk, rk, f"C5 head {g} dk")
        check_grad(dv, rv, f"C5 head {g} dv")


def test_fp32_one_launch_ring_backward_without_keys():
    """The float32 three-launch ring share with only empty chunks: dQ = 0 and
    the accumulators untouched (the float32 forms run on tests/test_gpu_f32.py)."""
    q = torch.randn((1, 64, 2, 64), device="cuda")
    lse = torch.zeros((1, 2, 64), device="cuda")
    kc = [torch.zeros((1, 0, 1, 64), device="cuda")]
    acc = [torch.ones((1, 0, 1, 64), device="cuda")]
    dq = torch.full_like(q, float("nan"))
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    A.attn_bwd_ring(q, q, q, lse, kc, kc, [0], acc, [a.clone() for a in acc], dq, 0.1, True,
                    workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


@pytest.mark.parametrize("d,h_kv,window,fused,one_launch", [
    (128, 2, (-1, -1), True, False),
    (64, 1, (-1, -1), False, False),
    (128, 2, (100, 0), True, False),
    (128, 2, (-1, -1), True, True),
    (64, 1, (-1, -1), False, True),
    (128, 4, (100, 0), True, True),
])
def test_ring_share_backward(d, h_kv, window, fused, one_launch):
    """The ring backward as each of P = 4 ranks sees it (chunks of 96, causal):
    forward ring share for the rank's queries, then one attn_bwd_acc per
    chunk with the share's final (O, LSE).  dQ must equal the rank's rows of
    the full-sequence gradient, and each chunk's (dK, dV) accumulator the
    contribution of the rank's queries to that chunk's keys - the oracle's
    backward of the rank's query block against the whole sequence."""
    P, c, h = 4, 96, 8
    L = P * c
    q, k, v, do = draw_normal(41 + d + h_kv, [(1, L, h, d), (1, L, h_kv, d),
                                              (1, L, h_kv, d), (1, L, h, d)])
    q, k, v, do = (round_to_bf16(x) for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(d)
    kc = [dev(k[:, s * c:(s + 1) * c], "bf16") for s in range(P)]
    vc = [dev(v[:, s * c:(s + 1) * c], "bf16") for s in range(P)]
    offs = [s * c for s in range(P)]
    for r in range(P):
        say(f"[ring bwd] d={d} h_kv={h_kv} window={window} one_launch={one_launch} rank {r}")
        qr, dor = q[:, r * c:(r + 1) * c], do[:, r * c:(r + 1) * c]
        tq, tdo = dev(qr, "bf16"), dev(dor, "bf16")
        out, lse = A.ring_share(tq, kc, vc, offs, r * c, scale, True,
                                fused=fused, window=window)
        share = A.RingShareBwd(tq, out.clone(), lse.clone(), tdo, scale, True,
                               r * c, window)
        dq, dk_acc, dv_acc = share.run(kc, vc, offs, one_launch=one_launch)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.attention_bwd(qr, k, v, dor, scale, True, window[0],
                                          window[1], r * c, 0)
        check_grad(host(dq), rq, f"rank {r} dq")
        for s in range(P):
            check_grad(host(dk_acc[s]), rk[:, s * c:(s + 1) * c],
                       f"rank {r} chunk {s} dk")
            check_grad(host(dv_acc[s]), rv[:, s * c:(s + 1) * c],
                       f"rank {r} chunk {s} dv")


@pytest.mark.parametrize("seed", range(400, 406))
def test_ring_backward_one_launch_random(seed):
    """attn_bwd_ring on random chunk boundaries, orders (an empty chunk among
    them), masks and head layouts: dq against the oracle's backward of the
    query block over all keys, and each chunk's accumulator (which starts
    from a random value) against that value plus the chunk's slice of the
    oracle's dK, dV."""
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 128]))
    h_kv = int(r.choice([1, 2, 4]))
    h = h_kv * int(r.choice([1, 2]))
    l_q = int(r.integers(1, 300))
    l_k = int(r.integers(1, 700))
    nc = int(r.integers(1, 7))
    cuts = sorted(int(x) for x in r.integers(0, l_k + 1, nc - 1))
    bounds = [0, *cuts, l_k]
    order = [int(x) for x in r.permutation(nc)]
    causal = bool(r.integers(0, 2))
    wl = int(r.choice([-1, -1, 60]))
    wr = int(r.choice([-1, 0, 30]))
    qo = int(r.integers(0, 700))
    scale = float(r.choice([1.0 / math.sqrt(d), -0.07]))
    say(f"[ring bwd one launch] seed {seed}: d={d} h={h} h_kv={h_kv} l_q={l_q} l_k={l_k} "
        f"bounds={bounds} order={order} causal={causal} window=({wl},{wr}) qo={qo}")
    q, k, v, do = (round_to_bf16(x) for x in draw_normal(
        seed, [(1, l_q, h, d), (1, l_k, h_kv, d), (1, l_k, h_kv, d), (1, l_q, h, d)]))
    tq, tk, tv, tdo = (dev(x, "bf16") for x in (q, k, v, do))
    o, lse = A.attention_forward(tq, tk, tv, scale, causal, (wl, wr), qo, 0)
    kc = [dev(k[:, bounds[c]:bounds[c + 1]], "bf16") for c in order]
    vc = [dev(v[:, bounds[c]:bounds[c + 1]], "bf16") for c in order]
    offs = [bounds[c] for c in order]
    init = [r.standard_normal((1, bounds[c + 1] - bounds[c], h_kv, d)).astype(np.float32)
            for c in order]
    dka = [torch.from_numpy(x.copy()).cuda() for x in init]
    init_v = [r.standard_normal(x.shape).astype(np.float32) for x in init]
    dva = [torch.from_numpy(x.copy()).cuda() for x in init_v]
    dq = torch.empty_like(tq)
    A.attn_bwd_ring(tdo, tq, o, lse, kc, vc, offs, dka, dva, dq, scale, causal, wl, wr, qo)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, scale, causal, wl, wr, qo, 0)
    check_grad(host(dq), rq, "dq")
    for i, c in enumerate(order):
        sl = slice(bounds[c], bounds[c + 1])
        check_grad(host(dka[i]) - init[i], rk[:, sl], f"chunk {c} dk")
        check_grad(host(dva[i]) - init_v[i], rv[:, sl], f"chunk {c} dv")


def test_ring_backward_without_keys():
    """Chunks without keys: dq = 0, their (empty) accumulators untouched."""
    q, do = (round_to_bf16(x) for x in draw_normal(71, [(1, 90, 4, 64), (1, 90, 4, 64)]))
    tq, tdo = dev(q, "bf16"), dev(do, "bf16")
    out = torch.zeros_like(tq)
    lse = torch.full((1, 4, 90), float("-inf"), device="cuda")
    empty = torch.zeros((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    eacc = torch.zeros((1, 0, 2, 64), dtype=torch.float32, device="cuda")
    dq = torch.full_like(tq, float("nan"))
    A.attn_bwd_ring(tdo, tq, out, lse, [empty, empty], [empty, empty], [0, 5],
                    [eacc, eacc.clone()], [eacc.clone(), eacc.clone()], dq, 0.1, True)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


def test_prepared_ring_steps_equal_unprepared():
    """The share's backward with D and the LSE prepared once
    (attn_bwd_prepare + attn_bwd_acc_prepared, as RingShareBwd runs it)
    equals per-chunk attn_bwd_acc, which prepares them itself, bit for bit;
    and a second run on the same share object gives the same again."""
    P, c, h, h_kv, d = 3, 200, 8, 2, 128
    L = P * c
    q, k, v, do = (round_to_bf16(x) for x in draw_normal(
        57, [(1, L, h, d), (1, L, h_kv, d), (1, L, h_kv, d), (1, L, h, d)]))
    scale = 1.0 / math.sqrt(d)
    kc = [dev(k[:, s * c:(s + 1) * c], "bf16") for s in range(P)]
    vc = [dev(v[:, s * c:(s + 1) * c], "bf16") for s in range(P)]
    offs = [s * c for s in range(P)]
    r = P - 1
    tq, tdo = dev(q[:, r * c:], "bf16"), dev(do[:, r * c:], "bf16")
    out, lse = A.ring_share(tq, kc, vc, offs, r * c, scale, True, one_launch=True)
    out, lse = out.clone(), lse.clone()
    share = A.RingShareBwd(tq, out, lse, tdo, scale, True, r * c)
    dq1, dk1, dv1 = share.run(kc, vc, offs)
    dq1, dk1, dv1 = dq1.clone(), [t.clone() for t in dk1], [t.clone() for t in dv1]
    dq_acc = torch.zeros(tq.shape, dtype=torch.float32, device="cuda")
    for s in range(P):
        dka = torch.zeros(kc[s].shape, dtype=torch.float32, device="cuda")
        dva = torch.zeros_like(dka)
        A.attn_bwd_acc(tdo, tq, kc[s], vc[s], out, lse, dq_acc, dka, dva, scale, True,
                       -1, -1, r * c, offs[s])
        torch.cuda.synchronize()
        assert torch.equal(dka, dk1[s]) and torch.equal(dva, dv1[s]), f"chunk {s}"
    dq_ref = A.attn_acc_cast(dq_acc, torch.empty_like(tq))
    torch.cuda.synchronize()
    assert torch.equal(dq_ref, dq1)
    dq2, dk2, dv2 = share.run(kc, vc, offs)
    torch.cuda.synchronize()
    assert torch.equal(dq2, dq1) and all(torch.equal(a, b) for a, b in zip(dk2, dk1))


def test_c3_ring_share_backward():
    """The ring backward share of rank 7 at the ring workload's full size
    (1024 query rows, 8 chunks of 1024 keys, GQA 32/8), every key/value
    group: dQ and every chunk's (dK, dV) accumulators against the oracle's
    backward of rank 7's queries over the whole 8192-token sequence."""
    w = WORKLOADS["C3"]
    say(f"[C3 ring bwd] {w}")
    x = make_inputs(w)
    rng = np.random.default_rng(77)
    do = round_to_bf16(rng.standard_normal(x["q"].shape).astype(np.float32))
    tq, tdo = dev(x["q"], "bf16"), dev(do, "bf16")
    kc = [dev(cc, "bf16") for cc in x["k_chunks"]]
    vc = [dev(cc, "bf16") for cc in x["v_chunks"]]
    out, lse = A.ring_share(tq, kc, vc, x["k_offsets"], x["q_offset"],
                            w.softmax_scale, True, fused=True)
    share = A.RingShareBwd(tq, out.clone(), lse.clone(), tdo, w.softmax_scale,
                           True, x["q_offset"])
    rq, rk, rv = oracle.attention_bwd(x["q"], x["k_full"], x["v_full"], do,
                                      w.softmax_scale, True, -1, -1,
                                      x["q_offset"], 0, block=1024)
    c = w.l_k
    for one in (False, True):
        dq, dk_acc, dv_acc = share.run(kc, vc, x["k_offsets"], one_launch=one)
        torch.cuda.synchronize()
        check_grad(host(dq), rq, f"C3 rank 7 dq (one launch {one})")
        for s in range(8):
            check_grad(host(dk_acc[s]), rk[:, s * c:(s + 1) * c], f"C3 chunk {s} dk ({one})")
            check_grad(host(dv_acc[s]), rv[:, s * c:(s + 1) * c], f"C3 chunk {s} dv ({one})")


@pytest.mark.parametrize("causal,window,h_kv", [(True, (-1, -1), 2), (True, (40, 0), 1),
                                                (False, (-1, -1), 4)])
def test_flash_attention_autograd(causal, window, h_kv):
    """flash_attention under torch autograd: the forward equals attn_fwd, the
    gradients torch computes through the node equal attn_bwd's bit for bit,
    and both match the oracle."""
    q, k, v, do = (round_to_bf16(x) for x in draw_normal(
        811, [(1, 200, 4, 128), (1, 230, h_kv, 128), (1, 230, h_kv, 128),
              (1, 200, 4, 128)]))
    tq, tk, tv, tdo = (dev(x, "bf16") for x in (q, k, v, do))
    for t in (tq, tk, tv):
        t.requires_grad_(True)
    o = A.flash_attention(tq, tk, tv, 0.09, causal, window)
    (o.float() * tdo.float()).sum().backward()
    with torch.no_grad():
        o_ref, lse_ref = A.attention_forward(tq, tk, tv, 0.09, causal, window)
        g_ref = A.attention_backward(tdo, tq, tk, tv, o_ref, lse_ref, 0.09, causal,
                                     window)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for g, r in zip((tq.grad, tk.grad, tv.grad), g_ref):
        assert torch.equal(g, r)
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, 0.09, causal, window[0],
                                      window[1])
    check_grad(host(tq.grad), rq, "autograd dq")
    check_grad(host(tk.grad), rk, "autograd dk")
    check_grad(host(tv.grad), rv, "autograd dv")


@pytest.mark.parametrize("case", [
    # n, l_q, l_k, h, h_kv, d, causal, q_offset
    (300, 17, 17, 3, 1, 128, False, 0),
    (1, 1, 65536, 4, 2, 128, True, 65535),    # one query against a long key range
    (1, 20000, 1, 2, 2, 64, True, 0),         # one key seen by every row
    (2, 129, 40000, 4, 1, 128, True, 39871),  # a short chunk at the end of the keys
])
def test_backward_shape_extremes(case):
    """The backward at shape extremes (many tiny batches, one query, one key,
    a short query block against a long key range), whole gradients against
    the oracle."""
    n, l_q, l_k, h, h_kv, d, causal, qo = case
    say(f"[bwd extremes] {case}")
    q, k, v, do = (round_to_bf16(x) for x in draw_normal(
        91, [(n, l_q, h, d), (n, l_k, h_kv, d), (n, l_k, h_kv, d), (n, l_q, h, d)]))
    dq, dk, dv = run_fwd_bwd(q, k, v, do, 0.11, causal, -1, -1, qo, 0)
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, 0.11, causal, -1, -1, qo, 0)
    check_grad(dq, rq, f"{case} dq")
    check_grad(dk, rk, f"{case} dk")
    check_grad(dv, rv, f"{case} dv")
