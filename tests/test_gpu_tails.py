"""Rows past the end of a tensor are never used.  The kernels load whole
64-row tiles and rely on the buffer range check to return zeros for rows
past a tensor's end; here every input is the front of a larger allocation
whose remainder (more than a tile of rows) is NaN, so a tail row that were
fetched from memory instead would turn the results NaN.  All reads stay
inside the allocation either way."""
import math

import numpy as np
import pytest
import torch

import oracle
from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from gpu_util import check_o_lse, host, say

pytestmark = pytest.mark.gpu


def nan_padded(x, dtype=torch.bfloat16, extra=512):
    """Device tensor holding x, followed in memory by `extra` rows of NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    row = int(np.prod(x.shape[2:])) if x.ndim > 2 else 1
    buf = torch.full((x.size + extra * row,), float("nan"), dtype=dtype, device="cuda")
    buf[:x.size] = torch.from_numpy(x.reshape(-1)).to(dtype).cuda()
    return buf[:x.size].view(x.shape)


def inputs(seed, l_q, l_k, h, h_kv, d):
    return [round_to_bf16(a) for a in draw_normal(
        seed, [(1, l_q, h, d), (1, l_k, h_kv, d), (1, l_k, h_kv, d), (1, l_q, h, d)])]


@pytest.mark.parametrize("l_q,l_k,h,h_kv,d,causal,qo", [
    (100, 77, 2, 1, 128, False, 0),
    (70, 130, 4, 2, 64, True, 60),
    (130, 8999, 2, 1, 128, False, 0),      # long key loop: the pipelined kernel
    (200, 9001, 2, 2, 64, True, 8801),
])
def test_forward_tails(l_q, l_k, h, h_kv, d, causal, qo):
    say(f"[tails fwd] l_q={l_q} l_k={l_k} h={h} h_kv={h_kv} d={d} causal={causal}")
    q, k, v, _ = inputs(81 + l_q, l_q, l_k, h, h_kv, d)
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv = nan_padded(q), nan_padded(k), nan_padded(v)
    ro, rl = oracle.attention_fwd(q, k, v, scale, causal, -1, -1, qo, 0)
    o, lse = A.attention_forward(tq, tk, tv, scale, causal, (-1, -1), qo, 0)
    torch.cuda.synchronize()
    check_o_lse(host(o), host(lse), ro, rl, "bf16", "attn_fwd")
    # the fused step into an empty accumulator gives the same result
    acc = torch.zeros((1, l_q, h, d), dtype=torch.float32, device="cuda")
    lacc = torch.full((1, h, l_q), float("-inf"), dtype=torch.float32, device="cuda")
    A.attn_fwd_acc(tq, tk, tv, acc, lacc, scale, causal, -1, -1, qo, 0)
    torch.cuda.synchronize()
    check_o_lse(host(acc), host(lacc), ro, rl, "bf16", "attn_fwd_acc")
    # the one-launch share over three ragged chunks, each followed by NaN
    b = [0, l_k // 3 + 5, 2 * l_k // 3 + 1, l_k]
    kc = [nan_padded(k[:, b[c]:b[c + 1]]) for c in range(3)]
    vc = [nan_padded(v[:, b[c]:b[c + 1]]) for c in range(3)]
    o3 = torch.empty_like(tq)
    l3 = torch.empty_like(lse)
    A.attn_fwd_ring(tq, kc, vc, b[:3], o3, l3, scale, causal, -1, -1, qo)
    torch.cuda.synchronize()
    check_o_lse(host(o3), host(l3), ro, rl, "bf16", "attn_fwd_ring")


@pytest.mark.parametrize("l_q,l_k,h,h_kv,d,causal", [
    (100, 77, 2, 1, 128, False),
    (77, 150, 4, 2, 64, True),
])
def test_backward_tails(l_q, l_k, h, h_kv, d, causal):
    say(f"[tails bwd] l_q={l_q} l_k={l_k} h={h} h_kv={h_kv} d={d} causal={causal}")
    q, k, v, do = inputs(91 + l_q, l_q, l_k, h, h_kv, d)
    scale = 1.0 / math.sqrt(d)
    qo = l_k - l_q if causal else 0
    tq, tk, tv, tdo = nan_padded(q), nan_padded(k), nan_padded(v), nan_padded(do)
    o, lse = A.attention_forward(tq, tk, tv, scale, causal, (-1, -1), qo, 0)
    torch.cuda.synchronize()
    to = nan_padded(host(o))
    tl = nan_padded(host(lse), torch.float32)
    dq, dk, dv = A.attention_backward(tdo, tq, tk, tv, to, tl, scale, causal, (-1, -1),
                                      qo, 0)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, scale, causal, -1, -1, qo, 0)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = host(g)
        tol = 2e-2 * max(1.0, float(np.max(np.abs(r), initial=0.0)))
        err = float(np.max(np.abs(g - r), initial=0.0))
        say(f"  {name}: max|err| = {err:.3e} (tol {tol:.3e})")
        assert np.all(np.isfinite(g)) and err <= tol, (name, err, tol)
