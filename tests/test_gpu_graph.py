"""The ring shares recorded into HIP graphs (RingShare.capture,
RingShareBwd.capture): every replay must give exactly what an eager run on
the same buffer contents gives (bit for bit: the same kernels on the same
inputs), with eager launches and synchronisations between replays, and with
the input buffers rewritten in place between replays (a replay reads what
the buffers hold then).  The eager results are checked against the fp64
oracle as well."""
import numpy as np
import pytest
import torch

import oracle
from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from gpu_util import check_o_lse, dev, host, say

pytestmark = pytest.mark.gpu

P, C, H, HKV, D = 4, 192, 8, 2, 128   # 4 chunks of 192 keys, GQA 8/2
RANK = 2
SCALE = 0.0883883


def draw(seed):
    q, k, v, do = (round_to_bf16(x) for x in draw_normal(
        seed, [(1, C, H, D), (1, P * C, HKV, D), (1, P * C, HKV, D),
               (1, C, H, D)]))
    return q, k, v, do


def chunks(t):
    return [t[:, s * C:(s + 1) * C].contiguous() for s in range(P)]


def fill(dst, src):
    dst.copy_(dev(src, "bf16"))


@pytest.mark.parametrize("fused", [True, False])
def test_ring_share_graph_replays(fused):
    say(f"[graph fwd] P={P} chunk={C} h={H}/{HKV} d={D} rank={RANK} fused={fused}")
    q, k, v, _ = draw(501)
    tq = dev(q, "bf16")
    kc, vc = chunks(dev(k, "bf16")), chunks(dev(v, "bf16"))
    offs = [s * C for s in range(P)]
    share = A.RingShare(tq, SCALE, True, RANK * C)
    ref = A.RingShare(tq, SCALE, True, RANK * C)   # eager twin
    graph = share.capture(kc, vc, offs, fused=fused)
    for rep in range(3):
        if rep == 2:
            # new contents in q and one chunk, written in place
            q, k, v, _ = draw(502)
            fill(tq, q)
            fill(kc[1], k[:, C:2 * C])
            fill(vc[1], v[:, C:2 * C])
            torch.cuda.synchronize()
        # eager work of the program between replays
        o_e, l_e = ref.run(kc, vc, offs, fused=fused)
        torch.cuda.synchronize()
        o_e, l_e = o_e.clone(), l_e.clone()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(share.out, o_e), f"replay {rep}: O differs"
        assert torch.equal(share.lse_acc, l_e), f"replay {rep}: LSE differs"
        kk = np.concatenate([host(c) for c in kc], axis=1)
        vv = np.concatenate([host(c) for c in vc], axis=1)
        ro, rl = oracle.attention_fwd(host(tq), kk, vv, SCALE, True, -1, -1,
                                      RANK * C, 0)
        check_o_lse(host(o_e), host(l_e), ro, rl, "bf16", f"replay {rep}")


def test_ring_share_bwd_graph_replays():
    say(f"[graph bwd] P={P} chunk={C} h={H}/{HKV} d={D} rank={RANK}")
    q, k, v, do = draw(503)
    tq, tdo = dev(q, "bf16"), dev(do, "bf16")
    kc, vc = chunks(dev(k, "bf16")), chunks(dev(v, "bf16"))
    offs = [s * C for s in range(P)]
    out, lse = A.RingShare(tq, SCALE, True, RANK * C).run(kc, vc, offs,
                                                          fused=True)
    out, lse = out.clone(), lse.clone()
    bshare = A.RingShareBwd(tq, out, lse, tdo, SCALE, True, RANK * C)
    ref = A.RingShareBwd(tq, out, lse, tdo, SCALE, True, RANK * C)
    graph = bshare.capture(kc, vc, offs)
    for rep in range(3):
        if rep == 2:
            _, _, _, do2 = draw(504)
            fill(tdo, do2)
            torch.cuda.synchronize()
        dq_e, dk_e, dv_e = ref.run(kc, vc, offs)
        torch.cuda.synchronize()
        dq_e = dq_e.clone()
        dk_e = [t.clone() for t in dk_e]
        dv_e = [t.clone() for t in dv_e]
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bshare.dq, dq_e), f"replay {rep}: dQ differs"
        for s in range(P):
            assert torch.equal(bshare.dk_acc[s], dk_e[s]), f"replay {rep}: dK {s}"
            assert torch.equal(bshare.dv_acc[s], dv_e[s]), f"replay {rep}: dV {s}"
    # the last eager result against the oracle (q rows of this rank against
    # the whole key sequence)
    kk = np.concatenate([host(c) for c in kc], axis=1)
    vv = np.concatenate([host(c) for c in vc], axis=1)
    rq, rk, rv = oracle.attention_bwd(host(tq), kk, vv, host(tdo), SCALE, True,
                                      -1, -1, RANK * C, 0)
    g_dq = host(dq_e)
    g_dk = np.concatenate([host(t) for t in dk_e], axis=1)
    g_dv = np.concatenate([host(t) for t in dv_e], axis=1)
    for g, r, name in ((g_dq, rq, "dq"), (g_dk, rk, "dk"), (g_dv, rv, "dv")):
        tol = 2e-2 * max(1.0, float(np.max(np.abs(r))))
        err = float(np.max(np.abs(g - r)))
        say(f"  {name}: max|err| = {err:.3e} (tol {tol:.3e})")
        assert err <= tol
