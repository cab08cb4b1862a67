"""Empty inputs through the C ABI on the GPU: no keys (every row empty: O = 0,
LSE = -inf, dQ = 0; a fused ring step or a merge of the empty block keeps
the accumulator rows that hold a result and clears those at -inf to O = 0;
an accumulating backward step leaves its accumulators alone), no query rows
(dK = dV = 0), zero batch, and a ring share with an empty chunk among its
chunks.  Expected values are the oracle's (fully-masked rows, its merge) or
the untouched inputs."""
import numpy as np
import pytest
import torch

import oracle
from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from gpu_util import check_o_lse, dev, host, say

pytestmark = pytest.mark.gpu


def rand(seed, shapes, dtype="bf16"):
    xs = draw_normal(seed, shapes)
    return [round_to_bf16(x) if dtype == "bf16" else x for x in xs]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_forward_without_keys(dtype, d):
    say(f"[empty] forward l_k = 0, {dtype}, d={d}")
    (q,) = rand(601, [(2, 70, 4, d)], dtype)
    k = np.zeros((2, 0, 2, d), np.float32)
    tq, tk, tv = dev(q, dtype), dev(k, dtype), dev(k, dtype)
    out = torch.full_like(tq, 7.0)
    lse = torch.full((2, 4, 70), 7.0, device="cuda")
    A.attn_fwd(tq, tk, tv, out, lse, 0.1, True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(q, k, k, 0.1, True)
    check_o_lse(host(out), host(lse), ro, rl, dtype, "l_k = 0")
    assert torch.count_nonzero(out).item() == 0


def test_forward_without_rows_or_batch():
    for shape in ((0, 64, 2, 128), (1, 0, 2, 128)):
        q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        k = torch.zeros((shape[0], 64, 2, 128), dtype=torch.bfloat16, device="cuda")
        o, lse = A.attention_forward(q, k, k, 0.1, True)
        torch.cuda.synchronize()
        assert o.numel() == 0 and lse.numel() == 0


def test_fused_step_and_merge_of_an_empty_chunk():
    (q, acc, lacc) = rand(602, [(1, 50, 4, 128), (1, 50, 4, 128), (1, 4, 50)], "f32")
    q = round_to_bf16(q)
    tq = dev(q, "bf16")
    tk = torch.zeros((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    # a fifth of the accumulator rows empty, holding garbage
    empty = np.random.default_rng(602).random((1, 4, 50)) < 0.2
    assert empty.any() and not empty.all()
    lacc = lacc.copy()
    lacc[empty] = -np.inf
    ref_o, ref_l = oracle.merge(acc, lacc, np.zeros_like(acc),
                                np.full_like(lacc, -np.inf))
    acc = acc.copy()
    acc[np.transpose(empty, (0, 2, 1))] = np.nan
    tacc = torch.from_numpy(acc).cuda()
    tl = torch.from_numpy(lacc).cuda()
    A.attn_fwd_acc(tq, tk, tk, tacc, tl, 0.1, True)
    torch.cuda.synchronize()
    assert np.array_equal(host(tacc), ref_o) and np.array_equal(host(tl), ref_l)
    a0, l0 = tacc.clone(), tl.clone()
    # the unfused ring step: forward of the empty chunk, then the merge
    blk, lblk = A.attention_forward(tq, tk, tk, 0.1, True)
    A.attn_merge(tacc, tl, blk, lblk)
    e = torch.zeros((1, 0, 4, 128), device="cuda")
    A.attn_merge(e, torch.zeros((1, 4, 0), device="cuda"),
                 e.to(torch.bfloat16), torch.zeros((1, 4, 0), device="cuda"))
    A.attn_acc_init(e, torch.zeros((1, 4, 0), device="cuda"))
    A.attn_acc_cast(e, e.to(torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(tacc, a0) and torch.equal(tl, l0)


@pytest.mark.parametrize("fused", [True, False])
def test_ring_share_with_an_empty_chunk(fused):
    q, k, v = rand(603, [(1, 96, 4, 64), (1, 192, 2, 64), (1, 192, 2, 64)])
    tq = dev(q, "bf16")
    kc = [dev(k[:, :96], "bf16"), dev(k[:, 96:], "bf16")]
    vc = [dev(v[:, :96], "bf16"), dev(v[:, 96:], "bf16")]
    empty = torch.zeros((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    o1, l1 = A.ring_share(tq, kc, vc, [0, 96], 96, 0.125, True, fused=fused)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = A.ring_share(tq, [kc[0], empty, kc[1]], [vc[0], empty, vc[1]],
                          [0, 96, 96], 96, 0.125, True, fused=fused)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ro, rl = oracle.attention_fwd(q, k, v, 0.125, True, -1, -1, 96, 0)
    check_o_lse(host(o2), host(l2), ro, rl, "bf16", "ring share with an empty chunk")


def test_backward_without_keys_or_rows():
    q, k, do = rand(604, [(1, 80, 4, 128), (1, 90, 2, 128), (1, 80, 4, 128)])
    tq, tk, tdo = dev(q, "bf16"), dev(k, "bf16"), dev(do, "bf16")
    # no keys: dQ = 0
    k0 = torch.zeros((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = A.attention_forward(tq, k0, k0, 0.1, True)
    dq = torch.full_like(tq, 3.0)
    dk = torch.empty_like(k0)
    A.attn_bwd(tdo, tq, k0, k0, o, lse, dq, dk, dk.clone(), 0.1, True)
    torch.cuda.synchronize()
    rq, _, _ = oracle.attention_bwd(q, np.zeros((1, 0, 2, 128), np.float32),
                                    np.zeros((1, 0, 2, 128), np.float32), do, 0.1, True)
    assert np.array_equal(host(dq), rq)
    # no query rows: dK = dV = 0
    q0 = torch.zeros((1, 0, 4, 128), dtype=torch.bfloat16, device="cuda")
    o0, l0 = A.attention_forward(q0, tk, tk, 0.1, True)
    dk = torch.full_like(tk, 3.0)
    dv = torch.full_like(tk, 3.0)
    A.attn_bwd(q0, q0, tk, tk, o0, l0, torch.empty_like(q0), dk, dv, 0.1, True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0
    # accumulating form: nothing added
    acc = [torch.full(t.shape, 2.5, device="cuda") for t in (tq, k0, k0)]
    A.attn_bwd_acc(tdo, tq, k0, k0, o, lse, *acc, 0.1, True)
    acc2 = [torch.full(t.shape, 2.5, device="cuda") for t in (q0, tk, tk)]
    A.attn_bwd_acc(q0, q0, tk, tk, o0, l0, *acc2, 0.1, True)
    torch.cuda.synchronize()
    for t in acc + acc2:
        assert bool((t == 2.5).all())


def test_hbm_copy_reference_copies():
    """The bandwidth reference of the merge is a plain copy: dst equals src
    bit for bit, and nothing past dst's end is touched."""
    src = torch.randn(3 * 4096 + 4, device="cuda")
    buf = torch.full((3 * 4096 + 4 + 64,), 7.0, device="cuda")
    A.hbm_copy(src, buf[:src.numel()])
    torch.cuda.synchronize()
    assert torch.equal(buf[:src.numel()], src)
    assert torch.all(buf[src.numel():] == 7.0)
