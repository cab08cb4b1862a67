"""Seeded random configurations against the fp64 oracle: forward (and the
fused ring step on a random accumulator) and backward over small shapes drawn
across head dims, grouped-head ratios, causal / window / offset masks, ragged
lengths and scales.  Each case is printed before it runs."""
import math

import numpy as np
import pytest
import torch

import oracle
from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from gpu_util import check_o_lse, dev, host, say

pytestmark = pytest.mark.gpu


def draw_case(seed):
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 128]))
    h_kv = int(r.choice([1, 2, 4]))
    h = h_kv * int(r.choice([1, 2, 4]))
    n = int(r.integers(1, 3))
    l_q = int(r.integers(1, 400))
    l_k = int(r.integers(1, 400))
    causal = bool(r.integers(0, 2))
    wl = int(r.choice([-1, -1, 0, 17, 130]))
    wr = int(r.choice([-1, -1, 0, 9, 70]))
    qo = int(r.integers(-50, 300))
    ko = int(r.integers(-50, 300))
    scale = float(r.choice([1.0 / math.sqrt(d), 0.3, -0.05]))
    return n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko, scale


SEEDS = list(range(100, 124))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_forward_and_fused_step(seed):
    n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko, scale = case = draw_case(seed)
    say(f"[random fwd] seed {seed}: {case}")
    q, k, v = (round_to_bf16(x) for x in draw_normal(
        seed, [(n, l_q, h, d), (n, l_k, h_kv, d), (n, l_k, h_kv, d)]))
    tq, tk, tv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    o, lse = A.attention_forward(tq, tk, tv, scale, causal, (wl, wr), qo, ko)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal, wl, wr, qo, ko)
    check_o_lse(host(o), host(lse), ro, rl, "bf16", f"seed {seed}")
    # the fused ring step on a random accumulator (a third of its rows empty,
    # holding garbage: an empty accumulator row's O must not leak, and where
    # this chunk gives the row no key either the merge gives O = 0)
    rng = np.random.default_rng(seed + 1)
    acc0 = rng.standard_normal((n, l_q, h, d)).astype(np.float32)
    lse0 = (rng.standard_normal((n, h, l_q)) * 2).astype(np.float32)
    empty0 = rng.random((n, h, l_q)) < 0.33
    lse0[empty0] = -np.inf
    acc_in = acc0.copy()
    acc_in[np.transpose(empty0, (0, 2, 1))] = 1e30
    acc = torch.from_numpy(acc_in).cuda()
    lacc = torch.from_numpy(lse0).cuda()
    A.attn_fwd_acc(tq, tk, tv, acc, lacc, scale, causal, wl, wr, qo, ko)
    torch.cuda.synchronize()
    mo, ml = oracle.merge(acc0, lse0, ro, rl)
    check_o_lse(host(acc), host(lacc), mo, ml, "bf16", f"seed {seed} fused")


@pytest.mark.parametrize("seed", SEEDS[:12])
def test_random_backward(seed):
    n, l_q, l_k, h, h_kv, d, causal, wl, wr, qo, ko, scale = case = draw_case(seed)
    say(f"[random bwd] seed {seed}: {case}")
    q, k, v, do = (round_to_bf16(x) for x in draw_normal(
        seed, [(n, l_q, h, d), (n, l_k, h_kv, d), (n, l_k, h_kv, d), (n, l_q, h, d)]))
    tq, tk, tv, tdo = (dev(x, "bf16") for x in (q, k, v, do))
    o, lse = A.attention_forward(tq, tk, tv, scale, causal, (wl, wr), qo, ko)
    dq, dk, dv = A.attention_backward(tdo, tq, tk, tv, o, lse, scale, causal,
                                      (wl, wr), qo, ko)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, scale, causal, wl, wr, qo, ko)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = host(g)
        tol = 2e-2 * max(1.0, float(np.max(np.abs(r), initial=0.0)))
        err = float(np.max(np.abs(g - r), initial=0.0))
        say(f"  {name}: max|err| = {err:.3e} (tol {tol:.3e})")
        assert np.all(np.isfinite(g)) and err <= tol, (name, err, tol)
