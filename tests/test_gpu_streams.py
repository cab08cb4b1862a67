"""Stream semantics of the C ABI: every call enqueues on the stream it is
given and nothing else, so (1) results on a side stream equal those on the
default stream bit for bit, (2) work enqueued earlier on the same stream (an
in-place rewrite of q) is seen without any synchronisation, and (3) calls
from two host threads on two streams, interleaved, give each thread exactly
its single-threaded results (the library keeps no global state)."""
import threading

import pytest
import torch

from blockwise_exact_attention_amd import attention as A
from blockwise_exact_attention_amd.inputs import draw_normal, round_to_bf16
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def inputs(seed, n=1, l=300, h=4, h_kv=2, d=128):
    q, k, v = (round_to_bf16(x) for x in draw_normal(
        seed, [(n, l, h, d), (n, l, h_kv, d), (n, l, h_kv, d)]))
    return dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")


def test_side_stream_and_same_stream_ordering():
    say("[streams] side stream, in-stream ordering")
    q, k, v = inputs(701)
    q2, _, _ = inputs(702)
    o_ref, l_ref = A.attention_forward(q, k, v, 0.1, True)
    o2_ref, l2_ref = A.attention_forward(q2, k, v, 0.1, True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    qs = q.clone()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = A.attention_forward(qs, k, v, 0.1, True)
        o_a, l_a = o.clone(), lse.clone()
        qs.copy_(q2)                      # enqueued on s, before the next call
        o, lse = A.attention_forward(qs, k, v, 0.1, True)
        dq, dk, dv = A.attention_backward(o, qs, k, v, o, lse, 0.1, True)
    s.synchronize()
    assert torch.equal(o_a, o_ref) and torch.equal(l_a, l_ref)
    assert torch.equal(o, o2_ref) and torch.equal(lse, l2_ref)
    dq_ref, dk_ref, dv_ref = A.attention_backward(o2_ref, q2, k, v, o2_ref, l2_ref,
                                                  0.1, True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq_ref) and torch.equal(dk, dk_ref) and torch.equal(dv, dv_ref)


def test_two_host_threads_two_streams():
    say("[streams] two host threads")
    probs = [inputs(703, l=257, h=8, h_kv=2), inputs(704, l=400, h=4, h_kv=4, d=64)]
    refs = []
    for q, k, v in probs:
        o, lse = A.attention_forward(q, k, v, 0.2, True)
        refs.append((o.clone(), lse.clone()))
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            q, k, v = probs[i]
            s = torch.cuda.Stream()
            outs = []
            with torch.cuda.stream(s):
                for _ in range(20):
                    outs.append(A.attention_forward(q, k, v, 0.2, True))
            s.synchronize()
            for o, lse in outs:
                if not (torch.equal(o, refs[i][0]) and torch.equal(lse, refs[i][1])):
                    errors.append(f"thread {i}: result differs")
                    break
        except Exception as e:  # surfaced in the main thread
            errors.append(f"thread {i}: {e!r}")

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in ts), "a worker thread did not finish"
    assert not errors, errors


def test_backward_on_a_side_stream_while_another_is_current():
    """stream= names a stream other than the current one: the wrapper's
    workspace and outputs belong to that stream, so memory the current
    stream allocates and fills right after the call (before any
    synchronisation) cannot be the workspace the backward is still reading."""
    say("[streams] backward with stream= a side stream, the default stream current")
    q, k, v = inputs(705, l=1024, h=8, h_kv=2)
    do, _, _ = inputs(706, l=1024, h=8, h_kv=2)
    o, lse = A.attention_forward(q, k, v, 0.1, True)
    ref = A.attention_backward(do, q, k, v, o, lse, 0.1, True)
    # 1024 keys of 2 key/value heads give the dK/dV kernel few workgroups,
    # so the workspace also holds split partials; then the same call on a
    # side stream
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for rep in range(3):
        got = A.attention_backward(do, q, k, v, o, lse, 0.1, True, stream=s)
        # the current (default) stream grabs memory and overwrites it at once
        junk = [torch.full((1 << 22,), float(rep + 1), device="cuda") for _ in range(8)]
        s.synchronize()
        torch.cuda.synchronize()
        for g, r in zip(got, ref):
            assert torch.equal(g, r), f"repetition {rep}: gradients differ"
        del junk, got
