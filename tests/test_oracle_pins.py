"""Pins for the fp64 oracle: each test checks it against something other than
itself (hand-derived worked examples, brute force, closed forms, library
routines, invariants, finite differences), chosen so that a dropped term, a
wrong sign or index, or a transposed operand fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from brute_force import brute_attention

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _arr(x):
    def conv(v):
        if isinstance(v, list):
            return [conv(u) for u in v]
        return -math.inf if v == "-inf" else float(v)
    return np.array(conv(x), dtype=np.float64)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


MASKS = [
    # (causal, win_l, win_r, q_offset, k_offset)
    (False, -1, -1, 0, 0),
    (True, -1, -1, 0, 0),
    (True, 2, 0, 0, 0),
    (False, 1, 2, 0, 0),
    (True, -1, -1, 3, 0),     # bottom-right style alignment, l_q < l_k
    (True, -1, -1, 0, 4),     # some rows fully masked
    (False, 0, 0, 0, 0),      # diagonal only
    (True, 3, -1, 5, 2),
    (False, -1, 1, 0, 3),
]


# ---------------------------------------------------------------- worked examples

def test_worked_examples_attention():
    cases = json.load(open(GOLD))["attention"]
    for c in cases:
        o, lse = oracle.attention_fwd(_arr(c["q"]), _arr(c["k"]), _arr(c["v"]),
                                      c["scale"], c["causal"], c["win_l"],
                                      c["win_r"], c["q_offset"], c["k_offset"])
        np.testing.assert_allclose(o, _arr(c["o"]), rtol=0, atol=1e-14,
                                   err_msg=c["name"])
        exp_lse = _arr(c["lse"])
        assert np.array_equal(np.isneginf(lse), np.isneginf(exp_lse)), c["name"]
        fin = np.isfinite(exp_lse)
        np.testing.assert_allclose(lse[fin], exp_lse[fin], rtol=0, atol=1e-14,
                                   err_msg=c["name"])


def test_worked_examples_merge():
    for c in json.load(open(GOLD))["merge"]:
        for fn in (oracle.merge, oracle.merge_sigmoid):
            o, lse = fn(_arr(c["o1"]), _arr(c["lse1"]), _arr(c["o2"]),
                        _arr(c["lse2"]))
            np.testing.assert_allclose(o, _arr(c["o"]), rtol=0, atol=1e-14,
                                       err_msg=c["name"])
            np.testing.assert_allclose(lse, _arr(c["lse"]), rtol=0, atol=1e-14,
                                       err_msg=c["name"])


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("h_kv", [1, 2, 4])
def test_brute_force_tiny(mask, h_kv):
    causal, wl, wr, qo, ko = mask
    rng = np.random.default_rng(hash((mask, h_kv)) % 2**32)
    n, l_q, l_k, h, d = 2, 7, 9, 4, 5
    q = _rand(rng, n, l_q, h, d)
    k = _rand(rng, n, l_k, h_kv, d)
    v = _rand(rng, n, l_k, h_kv, d)
    scale = 0.7
    o, lse = oracle.attention_fwd(q, k, v, scale, causal, wl, wr, qo, ko)
    bo, blse = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale,
                               causal, wl, wr, qo, ko)
    bo, blse = np.array(bo), np.array(blse)
    assert np.array_equal(np.isneginf(lse), np.isneginf(blse))
    fin = np.isfinite(blse)
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)


def test_brute_force_ragged_and_single_key():
    rng = np.random.default_rng(7)
    for (l_q, l_k) in [(1, 1), (1, 5), (5, 1), (3, 8), (8, 3)]:
        q = _rand(rng, 1, l_q, 2, 3)
        k = _rand(rng, 1, l_k, 1, 3)
        v = _rand(rng, 1, l_k, 1, 3)
        for causal in (False, True):
            o, lse = oracle.attention_fwd(q, k, v, 1.3, causal)
            bo, blse = brute_attention(q.tolist(), k.tolist(), v.tolist(), 1.3,
                                       causal)
            np.testing.assert_allclose(o, np.array(bo), atol=1e-12, rtol=0)
            fin = np.isfinite(np.array(blse))
            np.testing.assert_allclose(lse[fin], np.array(blse)[fin],
                                       atol=1e-12, rtol=0)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("mask", MASKS)
def test_zero_query_closed_form(mask):
    """q = 0: every allowed key gets weight 1/|A_i|, so LSE_i = ln|A_i| and
    O_i is the mean of v over A_i."""
    causal, wl, wr, qo, ko = mask
    rng = np.random.default_rng(3)
    l_q, l_k = 11, 13
    q = np.zeros((1, l_q, 2, 4))
    k = _rand(rng, 1, l_k, 2, 4)
    v = _rand(rng, 1, l_k, 2, 4)
    o, lse = oracle.attention_fwd(q, k, v, 0.9, causal, wl, wr, qo, ko)
    for i in range(l_q):
        qp = qo + i
        a = [j for j in range(l_k)
             if (not causal or ko + j <= qp)
             and (wl < 0 or ko + j >= qp - wl)
             and (wr < 0 or ko + j <= qp + wr)]
        for hq in range(2):
            if not a:
                assert lse[0, hq, i] == -np.inf
                assert np.all(o[0, i, hq] == 0.0)
            else:
                assert abs(lse[0, hq, i] - math.log(len(a))) < 1e-13
                np.testing.assert_allclose(o[0, i, hq],
                                           v[0, a, hq].mean(axis=0),
                                           atol=1e-13, rtol=0)


def test_window_256_steady_state_is_ln257():
    """Causal window (256, 0) at the sliding-window workload's sizes: a
    steady-state row sees 257 keys (inclusive bounds), so with q = 0 its LSE
    is ln 257; row i < 256 sees i + 1 keys."""
    l = 600
    q = np.zeros((1, l, 1, 2))
    k = np.ones((1, l, 1, 2))
    v = np.ones((1, l, 1, 2))
    _, lse = oracle.attention_fwd(q, k, v, 0.125, True, 256, 0)
    assert abs(lse[0, 0, 400] - 5.549076) < 1e-6
    assert abs(lse[0, 0, 400] - math.log(257)) < 1e-13
    for i in (0, 1, 100, 255, 256, 599):
        assert abs(lse[0, 0, i] - math.log(min(i, 256) + 1)) < 1e-13


def test_lse_is_scipy_logsumexp():
    rng = np.random.default_rng(11)
    q = _rand(rng, 2, 9, 4, 6)
    k = _rand(rng, 2, 12, 2, 6)
    v = _rand(rng, 2, 12, 2, 6)
    for causal, wl, wr, qo, ko in MASKS:
        _, lse = oracle.attention_fwd(q, k, v, 0.4, causal, wl, wr, qo, ko)
        for b in range(2):
            for hq in range(4):
                g = hq // 2
                for i in range(9):
                    a = oracle.allowed_mask([i], np.arange(12), causal, wl, wr,
                                            qo, ko)[0]
                    if not a.any():
                        assert lse[b, hq, i] == -np.inf
                        continue
                    s = 0.4 * (k[b, a, g] @ q[b, i, hq])
                    ref = scipy.special.logsumexp(s)
                    assert abs(lse[b, hq, i] - ref) < 1e-12


def test_constant_v_gives_constant_o():
    rng = np.random.default_rng(12)
    q = _rand(rng, 1, 10, 2, 8)
    k = _rand(rng, 1, 10, 2, 8)
    c = rng.standard_normal(8)
    v = np.broadcast_to(c, (1, 10, 2, 8)).copy()
    for causal, wl, wr, qo, ko in MASKS:
        o, lse = oracle.attention_fwd(q, k, v, 1.1, causal, wl, wr, qo, ko)
        for i in range(10):
            for hq in range(2):
                if np.isfinite(lse[0, hq, i]):
                    np.testing.assert_allclose(o[0, i, hq], c, atol=1e-13)


def test_single_key_and_diagonal_window():
    rng = np.random.default_rng(13)
    q = _rand(rng, 1, 6, 2, 5)
    k = _rand(rng, 1, 1, 2, 5)
    v = _rand(rng, 1, 1, 2, 5)
    o, lse = oracle.attention_fwd(q, k, v, 0.3)
    for i in range(6):
        for hq in range(2):
            np.testing.assert_allclose(o[0, i, hq], v[0, 0, hq], atol=1e-14)
            assert abs(lse[0, hq, i] - 0.3 * q[0, i, hq] @ k[0, 0, hq]) < 1e-13
    k = _rand(rng, 1, 6, 2, 5)
    v = _rand(rng, 1, 6, 2, 5)
    o, lse = oracle.attention_fwd(q, k, v, 0.3, False, 0, 0)
    for i in range(6):
        for hq in range(2):
            np.testing.assert_allclose(o[0, i, hq], v[0, i, hq], atol=1e-14)
            assert abs(lse[0, hq, i] - 0.3 * q[0, i, hq] @ k[0, i, hq]) < 1e-13


def test_matches_torch_sdpa_fp64():
    """Library routine: torch's scaled_dot_product_attention in fp64 on the
    CPU, with the boolean mask spelled out and K/V repeated for grouped heads
    as RingAttention._repeat_kv does."""
    rng = np.random.default_rng(14)
    n, l_q, l_k, h, h_kv, d = 2, 13, 17, 6, 2, 8
    q = _rand(rng, n, l_q, h, d)
    k = _rand(rng, n, l_k, h_kv, d)
    v = _rand(rng, n, l_k, h_kv, d)
    for causal, wl, wr, qo, ko in MASKS:
        o, lse = oracle.attention_fwd(q, k, v, 0.35, causal, wl, wr, qo, ko)
        mask = oracle.allowed_mask(np.arange(l_q), np.arange(l_k), causal, wl,
                                   wr, qo, ko)
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(np.repeat(k, h // h_kv, axis=2)).permute(0, 2, 1, 3)
        tv = torch.from_numpy(np.repeat(v, h // h_kv, axis=2)).permute(0, 2, 1, 3)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=0.35)
        ref = ref.permute(0, 2, 1, 3).numpy()
        rows = mask.any(axis=1)
        np.testing.assert_allclose(o[:, rows], ref[:, rows], atol=1e-12)
        assert np.all(o[:, ~rows] == 0.0)


# ---------------------------------------------------------------- invariants

def test_key_shift_invariance():
    """K <- K + 1 b^T leaves O unchanged and shifts LSE_i by scale q_i . b."""
    rng = np.random.default_rng(15)
    q = _rand(rng, 1, 8, 2, 4)
    k = _rand(rng, 1, 8, 1, 4)
    v = _rand(rng, 1, 8, 1, 4)
    bvec = rng.standard_normal(4)
    for causal, wl, wr, qo, ko in MASKS:
        o1, l1 = oracle.attention_fwd(q, k, v, 0.8, causal, wl, wr, qo, ko)
        o2, l2 = oracle.attention_fwd(q, k + bvec, v, 0.8, causal, wl, wr, qo,
                                      ko)
        np.testing.assert_allclose(o1, o2, atol=1e-12)
        shift = 0.8 * np.einsum("nlhd,d->nhl", q, bvec)
        fin = np.isfinite(l1)
        np.testing.assert_allclose(l2[fin], (l1 + shift)[fin], atol=1e-12)


def test_offset_shift_invariance():
    rng = np.random.default_rng(16)
    q = _rand(rng, 1, 9, 2, 4)
    k = _rand(rng, 1, 11, 2, 4)
    v = _rand(rng, 1, 11, 2, 4)
    for causal, wl, wr, qo, ko in MASKS:
        o1, l1 = oracle.attention_fwd(q, k, v, 0.8, causal, wl, wr, qo, ko)
        o2, l2 = oracle.attention_fwd(q, k, v, 0.8, causal, wl, wr,
                                      qo + 1000, ko + 1000)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(17)
    q = _rand(rng, 2, 7, 6, 4)
    k = _rand(rng, 2, 9, 3, 4)
    v = _rand(rng, 2, 9, 3, 4)
    kr = np.repeat(k, 2, axis=2)
    vr = np.repeat(v, 2, axis=2)
    for causal, wl, wr, qo, ko in MASKS:
        o1, l1 = oracle.attention_fwd(q, k, v, 0.6, causal, wl, wr, qo, ko)
        o2, l2 = oracle.attention_fwd(q, kr, vr, 0.6, causal, wl, wr, qo, ko)
        np.testing.assert_allclose(o1, o2, atol=1e-14)
        np.testing.assert_array_equal(np.isneginf(l1), np.isneginf(l2))


def test_key_permutation_invariance_noncausal():
    rng = np.random.default_rng(18)
    q = _rand(rng, 1, 5, 2, 4)
    k = _rand(rng, 1, 12, 2, 4)
    v = _rand(rng, 1, 12, 2, 4)
    perm = rng.permutation(12)
    o1, l1 = oracle.attention_fwd(q, k, v, 0.9)
    o2, l2 = oracle.attention_fwd(q, k[:, perm], v[:, perm], 0.9)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_fully_masked_rows():
    rng = np.random.default_rng(19)
    q = _rand(rng, 1, 4, 2, 3)
    k = _rand(rng, 1, 4, 2, 3)
    v = _rand(rng, 1, 4, 2, 3)
    o, lse = oracle.attention_fwd(q, k, v, 1.0, True, -1, -1, 0, 10)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))
    o, lse = oracle.attention_fwd(q, k, v, 1.0, False, 1, -1, 50, 0)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- merge and ring

def _rand_partial(rng, n, l, h, d, p_empty=0.2):
    o = _rand(rng, n, l, h, d)
    lse = rng.standard_normal((n, h, l)) * 3
    empty = rng.random((n, h, l)) < p_empty
    lse = np.where(empty, -np.inf, lse)
    o = np.where(np.transpose(empty, (0, 2, 1))[..., None], 0.0, o)
    return o, lse


def test_merge_log1p_equals_sigmoid_form():
    rng = np.random.default_rng(20)
    o1, l1 = _rand_partial(rng, 2, 9, 3, 4)
    o2, l2 = _rand_partial(rng, 2, 9, 3, 4)
    a = oracle.merge(o1, l1, o2, l2)
    b = oracle.merge_sigmoid(o1, l1, o2, l2)
    np.testing.assert_allclose(a[0], b[0], atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_merge_identity_commutative_associative():
    rng = np.random.default_rng(21)
    parts = [_rand_partial(rng, 1, 8, 2, 3) for _ in range(3)]
    zero = (np.zeros((1, 8, 2, 3)), np.full((1, 2, 8), -np.inf))
    for o, l in parts:
        mo, ml = oracle.merge(zero[0], zero[1], o, l)
        np.testing.assert_array_equal(mo, o)
        np.testing.assert_array_equal(ml, l)
        mo, ml = oracle.merge(o, l, zero[0], zero[1])
        np.testing.assert_array_equal(mo, o)
        np.testing.assert_array_equal(ml, l)
    (a, la), (b, lb), (c, lc) = parts
    ab = oracle.merge(a, la, b, lb)
    ba = oracle.merge(b, lb, a, la)
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-13)
    np.testing.assert_allclose(ab[1], ba[1], atol=1e-13)
    left = oracle.merge(*ab, c, lc)
    bc = oracle.merge(b, lb, c, lc)
    right = oracle.merge(a, la, *bc)
    np.testing.assert_allclose(left[0], right[0], atol=1e-12)
    np.testing.assert_allclose(left[1], right[1], atol=1e-12)


@pytest.mark.parametrize("mask", MASKS)
def test_chunked_merge_equals_unchunked(mask):
    """Attention over the whole key set equals the merge of attention over
    any split of it into chunks, merged in any order."""
    causal, wl, wr, qo, ko = mask
    rng = np.random.default_rng(22)
    l_k = 23
    q = _rand(rng, 1, 10, 4, 5)
    k = _rand(rng, 1, l_k, 2, 5)
    v = _rand(rng, 1, l_k, 2, 5)
    o_ref, l_ref = oracle.attention_fwd(q, k, v, 0.5, causal, wl, wr, qo, ko)
    cuts = [0, 4, 5, 13, 23]
    chunks = list(zip(cuts[:-1], cuts[1:]))
    for order in (chunks, chunks[::-1], [chunks[2], chunks[0], chunks[3],
                                         chunks[1]]):
        o = np.zeros(q.shape)
        lse = np.full((1, 4, 10), -np.inf)
        for a, b in order:
            ob, lb = oracle.attention_fwd(q, k[:, a:b], v[:, a:b], 0.5, causal,
                                          wl, wr, qo, ko + a)
            o, lse = oracle.merge(o, lse, ob, lb)
        np.testing.assert_allclose(o, o_ref, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(l_ref))
        fin = np.isfinite(l_ref)
        np.testing.assert_allclose(lse[fin], l_ref[fin], atol=1e-12)


def test_ring_share_equals_full_rows():
    """One rank's ring share over P chunks equals the rank's rows of causal
    attention over the full sequence (flash_sharding.py ring_fwd)."""
    rng = np.random.default_rng(23)
    P, c, h, h_kv, d = 4, 6, 4, 2, 5
    q = _rand(rng, 1, P * c, h, d)
    k = _rand(rng, 1, P * c, h_kv, d)
    v = _rand(rng, 1, P * c, h_kv, d)
    o_full, l_full = oracle.attention_fwd(q, k, v, 0.45, True)
    for r in range(P):
        qr = q[:, r * c:(r + 1) * c]
        kc = [k[:, s * c:(s + 1) * c] for s in range(P)]
        vc = [v[:, s * c:(s + 1) * c] for s in range(P)]
        o, lse = oracle.ring_share(qr, kc, vc, 0.45, True, r * c,
                                   [s * c for s in range(P)])
        np.testing.assert_allclose(o, o_full[:, r * c:(r + 1) * c], atol=1e-12)
        np.testing.assert_allclose(lse, l_full[:, :, r * c:(r + 1) * c],
                                   atol=1e-12)


# ---------------------------------------------------------------- backward

def _loss_grad_fd(q, k, v, do, scale, mask, eps=1e-6):
    """Central finite differences of L = sum(dO * O) in every input entry."""
    causal, wl, wr, qo, ko = mask
    grads = []
    for which in range(3):
        base = [q, k, v]
        x = base[which]
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy()
            xm = x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = list(base)
            args_m = list(base)
            args_p[which] = xp
            args_m[which] = xm
            op, _ = oracle.attention_fwd(*args_p, scale, causal, wl, wr, qo, ko)
            om, _ = oracle.attention_fwd(*args_m, scale, causal, wl, wr, qo, ko)
            g[idx] = (np.sum(do * op) - np.sum(do * om)) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("mask", [MASKS[0], MASKS[1], MASKS[2], MASKS[5],
                                  MASKS[7]])
def test_backward_finite_differences(mask):
    causal, wl, wr, qo, ko = mask
    rng = np.random.default_rng(24)
    q = _rand(rng, 1, 5, 4, 3)
    k = _rand(rng, 1, 6, 2, 3)
    v = _rand(rng, 1, 6, 2, 3)
    do = _rand(rng, 1, 5, 4, 3)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.6, causal, wl, wr, qo, ko)
    fq, fk, fv = _loss_grad_fd(q, k, v, do, 0.6, mask)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, atol=2e-7, rtol=1e-6)


def test_backward_matches_torch_autograd():
    """torch.autograd in fp64 through the dense definition (masked softmax on
    K/V expanded to every query head)."""
    rng = np.random.default_rng(25)
    n, l_q, l_k, h, h_kv, d = 2, 9, 11, 4, 2, 6
    for causal, wl, wr, qo, ko in MASKS:
        q = _rand(rng, n, l_q, h, d)
        k = _rand(rng, n, l_k, h_kv, d)
        v = _rand(rng, n, l_k, h_kv, d)
        do = _rand(rng, n, l_q, h, d)
        mask = oracle.allowed_mask(np.arange(l_q), np.arange(l_k), causal, wl,
                                   wr, qo, ko)
        rows = mask.any(axis=1)
        do[:, ~rows] = 0.0  # empty rows have no defined softmax in torch
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        kk = tk.repeat_interleave(h // h_kv, dim=2)
        vv = tv.repeat_interleave(h // h_kv, dim=2)
        s = torch.einsum("nihd,njhd->nhij", tq, kk) * 0.55
        tm = torch.from_numpy(mask)
        s = s.masked_fill(~tm, float("-inf"))
        s = s.masked_fill(~tm.any(dim=1)[:, None].expand_as(tm), 0.0)
        p = torch.softmax(s, dim=-1) * tm.any(dim=1)[:, None]
        o = torch.einsum("nhij,njhd->nihd", p, vv)
        (o * torch.from_numpy(do)).sum().backward()
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.55, causal, wl, wr,
                                          qo, ko)
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_backward_gqa_is_group_sum_of_mha():
    rng = np.random.default_rng(26)
    q = _rand(rng, 1, 8, 6, 4)
    k = _rand(rng, 1, 8, 2, 4)
    v = _rand(rng, 1, 8, 2, 4)
    do = _rand(rng, 1, 8, 6, 4)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.7, True)
    dq2, dk2, dv2 = oracle.attention_bwd(q, np.repeat(k, 3, axis=2),
                                         np.repeat(v, 3, axis=2), do, 0.7, True)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(1, 8, 2, 3, 4).sum(axis=3),
                               atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(1, 8, 2, 3, 4).sum(axis=3),
                               atol=1e-13)


def test_backward_fully_masked_rows_have_zero_grads():
    rng = np.random.default_rng(27)
    q = _rand(rng, 1, 4, 2, 3)
    k = _rand(rng, 1, 4, 2, 3)
    v = _rand(rng, 1, 4, 2, 3)
    do = _rand(rng, 1, 4, 2, 3)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 1.0, True, -1, -1, 0, 2)
    # rows 0 and 1 see nothing
    assert np.all(dq[:, :2] == 0.0)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 1.0, True, -1, -1, 0, 10)
    assert np.all(dq == 0.0) and np.all(dk == 0.0) and np.all(dv == 0.0)


def test_empty_sequences():
    """No keys: every row is fully masked (O = 0, LSE = -inf, dQ = 0); no
    query rows: dK = dV = 0; and a chunk with no keys merges as a no-op, so
    the ring share is unchanged by it."""
    rng = np.random.default_rng(31)
    q = _rand(rng, 1, 5, 2, 3)
    do = _rand(rng, 1, 5, 2, 3)
    k0 = np.zeros((1, 0, 2, 3))
    o, lse = oracle.attention_fwd(q, k0, k0, 1.0, True)
    assert o.shape == q.shape and np.all(o == 0.0) and np.all(np.isneginf(lse))
    dq, dk, dv = oracle.attention_bwd(q, k0, k0, do, 1.0, True)
    assert np.all(dq == 0.0) and dk.shape == (1, 0, 2, 3)
    k = _rand(rng, 1, 6, 2, 3)
    v = _rand(rng, 1, 6, 2, 3)
    q0 = np.zeros((1, 0, 2, 3))
    dq, dk, dv = oracle.attention_bwd(q0, k, v, q0, 1.0, True)
    assert np.all(dk == 0.0) and np.all(dv == 0.0)
    full = oracle.ring_share(q, [k[:, :3], k[:, 3:]], [v[:, :3], v[:, 3:]], 1.0,
                             True, 3, [0, 3])
    with_empty = oracle.ring_share(q, [k[:, :3], k0, k[:, 3:]],
                                   [v[:, :3], k0, v[:, 3:]], 1.0, True, 3,
                                   [0, 3, 3])
    for a, b in zip(full, with_empty):
        assert np.array_equal(a, b)
    ref_o, ref_l = brute_attention(q, k, v, 1.0, True, -1, -1, 3, 0)
    assert np.allclose(full[0], ref_o, atol=1e-12)


# ---------------------------------------------------------------- pins bite

def test_pins_catch_planted_mistakes():
    """Plant plausible mistakes in oracle calls (swapped window sides, an
    off-by-one offset, a missing scale, the wrong grouped-head mapping) and
    check that the brute-force pin disagrees with each one."""
    rng = np.random.default_rng(28)
    q = _rand(rng, 1, 6, 4, 3)
    k = _rand(rng, 1, 8, 2, 3)
    v = _rand(rng, 1, 8, 2, 3)
    bo, blse = brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.5, True,
                               2, 1, 3, 0)
    bo = np.array(bo)
    good, _ = oracle.attention_fwd(q, k, v, 0.5, True, 2, 1, 3, 0)
    assert np.allclose(good, bo, atol=1e-12)
    mutants = [
        oracle.attention_fwd(q, k, v, 0.5, True, 1, 2, 3, 0)[0],     # sides
        oracle.attention_fwd(q, k, v, 0.5, True, 2, 1, 3, 1)[0],     # offset
        oracle.attention_fwd(q, k, v, 1.0, True, 2, 1, 3, 0)[0],     # scale
        oracle.attention_fwd(q, k[:, :, ::-1], v[:, :, ::-1], 0.5, True, 2, 1,
                             3, 0)[0],                               # heads
        oracle.attention_fwd(q, k, v, 0.5, False, 2, 1, 3, 0)[0],    # causal
    ]
    for m in mutants:
        assert not np.allclose(m, bo, atol=1e-6)


# ---------------------------------------------------------------- row blocks and sampling

@pytest.mark.parametrize("mask", MASKS)
def test_brute_force_across_row_blocks(mask):
    """The oracle's row blocks do not change the result: with block=2 (four
    or five blocks over 7-9 rows, the last one ragged) the forward still
    equals the pure-Python brute force, and the backward equals its own
    one-block result and torch autograd through the dense definition."""
    causal, wl, wr, qo, ko = mask
    rng = np.random.default_rng(abs(hash(("blocks", mask))) % 2**32)
    n, l_q, l_k, h, h_kv, d = 2, 9, 8, 4, 2, 5
    q = _rand(rng, n, l_q, h, d)
    k = _rand(rng, n, l_k, h_kv, d)
    v = _rand(rng, n, l_k, h_kv, d)
    do = _rand(rng, n, l_q, h, d)
    o, lse = oracle.attention_fwd(q, k, v, 0.8, causal, wl, wr, qo, ko, block=2)
    bo, blse = brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.8, causal,
                               wl, wr, qo, ko)
    bo, blse = np.array(bo), np.array(blse)
    assert np.array_equal(np.isneginf(lse), np.isneginf(blse))
    fin = np.isfinite(blse)
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    g2 = oracle.attention_bwd(q, k, v, do, 0.8, causal, wl, wr, qo, ko, block=2)
    g1 = oracle.attention_bwd(q, k, v, do, 0.8, causal, wl, wr, qo, ko, block=64)
    for a, b in zip(g2, g1):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # autograd through the dense masked softmax, independent of the blocks
    m = oracle.allowed_mask(np.arange(l_q), np.arange(l_k), causal, wl, wr, qo, ko)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.repeat_interleave(h // h_kv, dim=2)
    vv = tv.repeat_interleave(h // h_kv, dim=2)
    s = torch.einsum("nihd,njhd->nhij", tq, kk) * 0.8
    tm = torch.from_numpy(m)
    rows = tm.any(dim=1)
    s = s.masked_fill(~tm, float("-inf")).masked_fill(~rows[:, None].expand_as(tm), 0.0)
    p = torch.softmax(s, dim=-1) * rows[:, None]
    (torch.einsum("nhij,njhd->nihd", p, vv) * torch.from_numpy(do)).sum().backward()
    for a, t in zip(g2, (tq, tk, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=0, atol=1e-12)


def test_sampling_arguments_select_without_changing_values():
    """heads= and rows= (forward) and kv_heads= (backward) compute exactly the
    entries of the full call and leave every other entry NaN; the GPU checks
    at full size rely on these samples."""
    rng = np.random.default_rng(31)
    n, l_q, l_k, h, h_kv, d = 2, 13, 11, 6, 3, 4
    q = _rand(rng, n, l_q, h, d)
    k = _rand(rng, n, l_k, h_kv, d)
    v = _rand(rng, n, l_k, h_kv, d)
    do = _rand(rng, n, l_q, h, d)
    args = (0.6, True, 5, -1, 2, 0)
    o, lse = oracle.attention_fwd(q, k, v, *args, block=3)
    heads = [(1, 4), (0, 0), (1, 1)]
    rows = [12, 0, 5, 6, 7]
    so, sl = oracle.attention_fwd(q, k, v, *args, heads=heads, rows=rows, block=2)
    sel_o = np.zeros(o.shape, bool)
    sel_l = np.zeros(lse.shape, bool)
    for b, hq in heads:
        sel_o[b, rows, hq, :] = True
        sel_l[b, hq, rows] = True
    assert np.all(np.isnan(so[~sel_o])) and np.all(np.isnan(sl[~sel_l]))
    # (different row blocks keep different key columns: rounding-level
    # differences only)
    np.testing.assert_allclose(so[sel_o], o[sel_o], rtol=0, atol=1e-13)
    np.testing.assert_allclose(sl[sel_l], lse[sel_l], rtol=0, atol=1e-13)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, *args)
    kvh = [(1, 2), (0, 1)]
    sq, sk, sv = oracle.attention_bwd(q, k, v, do, *args, kv_heads=kvh, block=4)
    sel_q = np.zeros(dq.shape, bool)
    sel_k = np.zeros(dk.shape, bool)
    for b, g in kvh:
        sel_q[b, :, 2 * g:2 * g + 2, :] = True   # the group's query heads
        sel_k[b, :, g, :] = True
    for full, samp, sel in ((dq, sq, sel_q), (dk, sk, sel_k), (dv, sv, sel_k)):
        assert np.all(np.isnan(samp[~sel]))
        np.testing.assert_allclose(samp[sel], full[sel], rtol=0, atol=1e-13)


def test_ring_share_head_sample_equals_full_rows():
    """ring_share(heads=...) merges exactly the sampled heads: their rows equal
    full-sequence attention; the other heads stay at the empty result."""
    rng = np.random.default_rng(32)
    P, c, h, h_kv, d = 4, 5, 6, 2, 3
    q = _rand(rng, 2, P * c, h, d)
    k = _rand(rng, 2, P * c, h_kv, d)
    v = _rand(rng, 2, P * c, h_kv, d)
    o_full, l_full = oracle.attention_fwd(q, k, v, 0.5, True)
    heads = [(0, 5), (1, 0), (1, 3)]
    r = 2
    kc = [k[:, s * c:(s + 1) * c] for s in range(P)]
    vc = [v[:, s * c:(s + 1) * c] for s in range(P)]
    o, lse = oracle.ring_share(q[:, r * c:(r + 1) * c], kc, vc, 0.5, True, r * c,
                               [s * c for s in range(P)], heads=heads)
    for b in range(2):
        for hq in range(h):
            if (b, hq) in heads:
                np.testing.assert_allclose(o[b, :, hq], o_full[b, r * c:(r + 1) * c, hq],
                                           atol=1e-12)
                np.testing.assert_allclose(lse[b, hq], l_full[b, hq, r * c:(r + 1) * c],
                                           atol=1e-12)
            else:
                assert np.all(o[b, :, hq] == 0.0) and np.all(np.isneginf(lse[b, hq]))
