"""Tensors of more than 2^31 elements: q, k, v, O, dO and the gradients are
[3, 2^20, 8, 128] bf16 (3 * 2^30 elements, 6.4 GB each) and the float32
accumulators twice that.  The rows of the last batch start at element
offset 2^31 (byte offset 2^32), so 32-bit index arithmetic anywhere in the
forward, the merge, the fused ring step, the accumulator cast or the
backward would read or write the wrong rows there.

Every tensor is zero except a seeded block of 768 rows (all heads) at the
end of the last batch.  The mask is causal with a 256-key window, so the
last 512 rows see only keys of the block and the block's last 512 keys are
seen only by queries of the block: the oracle, run on the 768-row block
alone, gives exact O, LSE, dQ, dK and dV for them.  A misplaced read lands
on zeros (or on other rows of the block) and changes those values.  Rows
of the zero region have the closed form O = 0, LSE = ln(number of keys in
the window).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from gpu_util import check_o_lse, dev, host, say

pytestmark = pytest.mark.gpu

N, L, H, D = 3, 1 << 20, 8, 128
WL, WR = 255, 0            # causal, 256 keys per row
BLK, CHK = 768, 512        # seeded block, checked rows at its end
SCALE = 1.0 / math.sqrt(D)


def grad_close(g, ref, name):
    scale = max(1.0, float(np.max(np.abs(ref))))
    err = float(np.max(np.abs(g - ref)))
    say(f"  {name}: max|err| = {err:.3e} (tol {2e-2 * scale:.3e})")
    assert np.all(np.isfinite(g)), f"{name}: non-finite"
    assert err <= 2e-2 * scale, f"{name}: {err} > {2e-2 * scale}"


def test_tensors_beyond_2_31_elements():
    need = 110 << 30
    free, _ = torch.cuda.mem_get_info()
    if free < need:
        pytest.skip(f"needs {need >> 30} GiB of free device memory, {free >> 30} free")
    assert N * L * H * D > 2 ** 31
    say(f"[large] n={N} l={L} h={H} d={D} window=({WL},{WR}) causal")
    q_b, k_b, v_b, do_b = (round_to_bf16(x) for x in draw_normal(
        2031, [(1, BLK, H, D)] * 4))
    shape = (N, L, H, D)
    q, k, v, do = (torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
                   for _ in range(4))
    for big, blk in ((q, q_b), (k, k_b), (v, v_b), (do, do_b)):
        big[N - 1, L - BLK:] = dev(blk, "bf16")[0]
    rows = slice(L - CHK, L)

    o_ref, lse_ref = oracle.attention_fwd(q_b, k_b, v_b, SCALE, True, WL, WR)
    o_ref, lse_ref = o_ref[:, BLK - CHK:], lse_ref[:, :, BLK - CHK:]

    # ---- forward
    o, lse = A.attention_forward(q, k, v, SCALE, True, (WL, WR))
    torch.cuda.synchronize()
    check_o_lse(host(o[N - 1:, rows]), host(lse[N - 1:, :, rows]), o_ref,
                lse_ref, "bf16", "forward, last rows of the last batch")
    # zero region: first row sees one key, a later row a full window
    for b, i, n_keys in ((0, 0, 1), (N - 1, 0, 1), (N - 1, 1000, WL + 1),
                         (1, L - 1, WL + 1), (N - 1, L - BLK - 300, WL + 1)):
        assert torch.count_nonzero(o[b, i]).item() == 0, (b, i)
        got = lse[b, :, i].cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got - math.log(n_keys))) <= 1e-5, (b, i, got)

    # ---- merge: an empty accumulator takes the block, a second merge of
    # the same block keeps O and adds ln 2 to the LSE
    acc = torch.empty(shape, dtype=torch.float32, device="cuda")
    lacc = torch.empty((N, H, L), dtype=torch.float32, device="cuda")
    A.attn_acc_init(acc, lacc)
    A.attn_merge(acc, lacc, o, lse)
    torch.cuda.synchronize()
    assert torch.equal(acc[N - 1, rows], o[N - 1, rows].float())
    assert torch.equal(lacc[N - 1, :, rows], lse[N - 1, :, rows])
    A.attn_merge(acc, lacc, o, lse)
    torch.cuda.synchronize()
    d_o = (acc[N - 1, rows] - o[N - 1, rows].float()).abs().max().item()
    d_l = (lacc[N - 1, :, rows] - lse[N - 1, :, rows] - math.log(2.0)).abs().max().item()
    say(f"  merge twice: max|dO| = {d_o:.2e}, max|dLSE - ln2| = {d_l:.2e}")
    assert d_o <= 1e-5 and d_l <= 1e-5

    # ---- fused ring step into a fresh accumulator, then the cast
    A.attn_acc_init(acc, lacc)
    A.attn_fwd_acc(q, k, v, acc, lacc, SCALE, True, WL, WR)
    torch.cuda.synchronize()
    check_o_lse(host(acc[N - 1:, rows]), host(lacc[N - 1:, :, rows]), o_ref,
                lse_ref, "bf16", "fused step, last rows of the last batch")
    cast = torch.empty_like(o)
    A.attn_acc_cast(acc, cast)
    torch.cuda.synchronize()
    d_c = (cast[N - 1, rows].float() - o[N - 1, rows].float()).abs().max().item()
    say(f"  cast vs forward: max|d| = {d_c:.2e}")
    assert d_c <= 2e-2
    del acc, lacc, cast

    # ---- backward
    dq_ref, dk_ref, dv_ref = oracle.attention_bwd(q_b, k_b, v_b, do_b, SCALE,
                                                  True, WL, WR)
    dq_ref, dk_ref, dv_ref = (x[0, BLK - CHK:] for x in (dq_ref, dk_ref, dv_ref))
    dq, dk, dv = A.attention_backward(do, q, k, v, o, lse, SCALE, True, (WL, WR))
    torch.cuda.synchronize()
    grad_close(host(dq[N - 1, rows]), dq_ref, "dq")
    grad_close(host(dk[N - 1, rows]), dk_ref, "dk")
    grad_close(host(dv[N - 1, rows]), dv_ref, "dv")
    for g in (dq, dk, dv):
        assert torch.count_nonzero(g[: N - 1]).item() == 0
    del dq, dk, dv

    # ---- backward into float32 accumulators (the ring backward's step)
    dq_a, dk_a, dv_a = (torch.zeros(shape, dtype=torch.float32, device="cuda")
                        for _ in range(3))
    ws = torch.empty(A.bwd_workspace_bytes(N, L, L, H, H, D), dtype=torch.uint8,
                     device="cuda")
    A.attn_bwd_acc(do, q, k, v, o, lse, dq_a, dk_a, dv_a, SCALE, True, WL, WR,
                   0, 0, ws)
    torch.cuda.synchronize()
    grad_close(host(dq_a[N - 1, rows]), dq_ref, "dq (fp32 accumulator)")
    grad_close(host(dk_a[N - 1, rows]), dk_ref, "dk (fp32 accumulator)")
    grad_close(host(dv_a[N - 1, rows]), dv_ref, "dv (fp32 accumulator)")
    del dq_a, dk_a, dv_a, ws, q, k, v, do, o, lse
    torch.cuda.empty_cache()
