"""Benchmark of the blockwise exact-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--no-extras] [--no-cpu]
    python bench.py --workload {c3-steps,c3-fused,c3-share,c3-bwd,c3-bwd-one,c4,c5-fwd,c5-bwd,mqa-c2,mqa-c5}

Workload: causal multi-head attention, n=2, l=2048, h=h_kv=16, d=128, bf16,
scale 1/sqrt(128), synthetic N(0,1) inputs resident in HBM.  A step is one
attn_fwd call over that batch (through the C ABI).  Prints one JSON line:
forward TFLOP/s (algorithmic FLOPs: 4*d per allowed query/key pair per head),
the roofline of the forward kernel, the other targeted figures under
"extras" (the rank-7 ring share as per-chunk forwards, fused steps, one
launch and backward; the sliding window; the 16k-token forward and backward;
the merge's bandwidth warm and cold on both shapes against a plain streaming
copy), and the fp64 CPU oracle's rate on a bounded sample of the headline
workload.  --workload times one workload's call alone (for profiler runs);
--merge-only runs just the merge figures.  Every timed loop is preceded by
--settle-ms (default 100) of the same calls back to back and then its warmup
calls: the GPU reaches its sustained shader clock only after some 30 ms of
continuous work.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4 SIMD x 1024 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
SETTLE_MS = 100.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="milliseconds of back-to-back calls before each timed "
                         "loop's warmup, so that the loop runs at the clock the "
                         "GPU holds under sustained work (0: none)")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline workload (and the CPU baseline)")
    ap.add_argument("--workload", default="c2",
                    choices=("c2", "c3-steps", "c3-fused", "c3-share", "c3-bwd", "c3-bwd-one",
                             "mqa-c2", "mqa-c5",
                             "c4", "c5-fwd", "c5-bwd"),
                    help="time only this workload's call (for profiler runs); c2 "
                         "is the default full run")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--oracle-times", action="store_true",
                    help="only time the fp64 oracle on every workload at its "
                         "full size on the host cores and print the times")
    ap.add_argument("--merge-only", action="store_true",
                    help="only run the merge measurements (warm, cold, full "
                         "sequence) and print them")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 10 times "
                         "(reference for the HBM byte counters) and exit")
    return ap.parse_args()


def settle(fn, torch, ms=None):
    """Call fn() back to back for `ms` milliseconds of wall time (checked
    every 8 calls).  The GPU raises its shader clock only after tens of
    milliseconds of sustained work and lowers it again within milliseconds of
    idling, so every timed loop starts with this, then its warmup calls.
    Returns the number of calls made."""
    ms = SETTLE_MS if ms is None else ms
    calls = 0
    if ms <= 0:
        return calls
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn()
        calls += 8
        torch.cuda.synchronize()
    return calls


def timed(fn, steps, warmup, torch):
    """Mean GPU time per call (ms) of fn(), called `steps` times back to back
    between one event pair on the current stream (the one every library call
    is launched on), so that the events' own cost is spread over the calls.
    The calls run at the settled clock (settle() first)."""
    settle(fn, torch)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def cpu_baseline(x, w, seconds):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    whole (batch, head) pairs of the same inputs, cycling through the batch,
    until about `seconds` of CPU work is done."""
    import oracle
    from blockwise_exact_attention_amd.flops import allowed_pairs, fwd_flops
    cores = os.cpu_count() or 1
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] or [cores])
    except Exception:
        pass
    pairs = allowed_pairs(w.l_q, w.l_k, True)
    heads_all = [(b, hq) for b in range(w.n) for hq in range(w.h)]
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        oracle.attention_fwd(x["q"], x["k"], x["v"], w.softmax_scale, True,
                             heads=[heads_all[done % len(heads_all)]])
        done += 1
    dt = time.perf_counter() - t0
    flops = fwd_flops(1, done, w.d, pairs)
    host = _host_description()
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{done} (batch, head) forward passes of this workload "
                      f"({done / len(heads_all):.2f} x the whole batch), fp64 "
                      f"numpy with {cores} BLAS threads, {dt:.1f} s; host "
                      f"{host['model']}, {host['logical_cpus']} logical CPUs, "
                      f"{host['usable_cpus']} usable"}


def kernel_sources(kernel):
    """The source files that define a forward kernel's code."""
    main = "fwd_pipe.hip" if kernel.startswith("fwd_pipe") else "fwd.hip"
    return (main, "tile.hpp", "common.hpp")


def kernel_sources_sha256(kernel):
    """sha256 over a forward kernel's source files, in a fixed order."""
    import hashlib
    h = hashlib.sha256()
    for name in kernel_sources(kernel):
        with open(os.path.join(ROOT, "blockwise_exact_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


COUNTERS_JSON = "fwd_causal_mha_n2_l2048_h16_d128_counters.json"


def counted_traffic(kernel):
    """HBM bytes per forward launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy of known size), or
    None when that summary is of another kernel or the kernel's sources
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", COUNTERS_JSON)
    try:
        rec = json.load(open(path))
        sha = kernel_sources_sha256(kernel)
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("kernel_sources_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def merge_measurements(A, torch, merge_bytes, steps):
    """attn_merge bandwidth on the ring-share shape [1,1024,32,128] (bf16
    block), warm and cold, and on the full-sequence shape [1,8192,32,128],
    cold.  Cold: the calls rotate over enough separate buffer sets (403 MB
    and 606 MB of distinct memory) that each call's data has left the 256 MB
    Infinity Cache and the L2s since its set was last used, and one event
    pair spans all the calls (a per-call event pair adds microseconds).
    Warm: one buffer set, merged into again and again.  The library's plain
    streaming copy of the same byte count (attn_hbm_copy), cold the same way,
    is timed beside each as the reference for what a read-and-write stream
    reaches on this GPU (torch's copy for context)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)

    def buffers(n, l, h, d):
        acc = torch.randn((n, l, h, d), generator=gen, device=dev)
        lacc = torch.randn((n, h, l), generator=gen, device=dev)
        blk = torch.randn((n, l, h, d), generator=gen, device=dev).to(torch.bfloat16)
        lblk = torch.randn((n, h, l), generator=gen, device=dev)
        return acc, lacc, blk, lblk

    def rotating(sets):
        it = [0]

        def f():
            A.attn_merge(*sets[it[0] % len(sets)])
            it[0] += 1
        return f

    res = {}
    for name, shape, n_sets, warm in (("ring_block_1x1024x32x128", (1, 1024, 32, 128), 16, True),
                                      ("full_sequence_1x8192x32x128", (1, 8192, 32, 128), 3, False)):
        sets = [buffers(*shape) for _ in range(n_sets)]
        nbytes = merge_bytes(*shape, 2)
        r = {"bytes": nbytes}
        if warm:
            ms = timed(rotating(sets[:1]), steps, 5, torch)
            r["warm_ms"] = round(ms, 5)
            r["warm_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        ms = timed(rotating(sets), max(2 * n_sets, steps // n_sets * n_sets),
                   n_sets, torch)
        r["cold_ms"] = round(ms, 5)
        r["cold_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        r["cold_frac_of_hbm"] = round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        res[name] = r
        del sets
    # reference: the library's plain streaming copy (attn_hbm_copy) of the
    # same number of bytes as each merge moves, cold the same way; torch's
    # copy beside it for context
    for name, n_sets in (("ring_block_1x1024x32x128", 16), ("full_sequence_1x8192x32x128", 3)):
        nb = res[name]["bytes"] // 2 // 16 * 16      # copied once: read nb, write nb
        sets = [(torch.ones(nb // 4, device=dev), torch.empty(nb // 4, device=dev))
                for _ in range(n_sets)]
        for kind in ("hbm_copy", "torch_copy"):
            it = [0]

            def copy():
                src, dst = sets[it[0] % n_sets]
                if kind == "hbm_copy":
                    A.hbm_copy(src, dst)
                else:
                    dst.copy_(src)
                it[0] += 1
            ms = timed(copy, max(4 * n_sets, 32), n_sets, torch)
            res[name][f"{kind}_cold_gbs"] = round(2 * nb / (ms * 1e-3) / 1e9, 1)
        res[name]["merge_frac_of_hbm_copy"] = round(
            res[name]["cold_gbs"] / res[name]["hbm_copy_cold_gbs"], 4)
        del sets
    torch.cuda.empty_cache()
    return res


def oracle_times():
    """Wall time of the fp64 oracle (as it stands) on each workload at full
    size on this host's cores: best of 3 for the small ones, one run for the
    causal 2048- and 16384-token ones (forward, and forward plus backward for
    the latter).  Input generation is not timed."""
    import oracle
    from blockwise_exact_attention_amd.flops import (allowed_pairs, bwd_flops,
                                                     fwd_flops)
    from blockwise_exact_attention_amd.workloads import WORKLOADS, make_inputs
    res = {"cpu": _host_description()}
    for name, w in WORKLOADS.items():
        x = make_inputs(w)
        reps = 1 if name in ("C2", "C5") else 3
        if w.ring_chunks:
            def fwd():
                oracle.ring_share(x["q"], x["k_chunks"], x["v_chunks"],
                                  w.softmax_scale, True, x["q_offset"],
                                  x["k_offsets"])
            pairs = sum(allowed_pairs(w.l_q, w.l_k, True, -1, -1, x["q_offset"], ko)
                        for ko in x["k_offsets"])
        else:
            def fwd():
                oracle.attention_fwd(x["q"], x["k"], x["v"], w.softmax_scale,
                                     w.causal, w.win_l, w.win_r)
            pairs = allowed_pairs(w.l_q, w.l_k, w.causal, w.win_l, w.win_r)
        best = math.inf
        for _ in range(reps):
            if w.backward:
                # the long workload head by head (the oracle treats heads
                # independently), with a progress line per head
                t = 0.0
                for hq in range(w.h):
                    t0 = time.perf_counter()
                    oracle.attention_fwd(x["q"], x["k"], x["v"], w.softmax_scale,
                                         w.causal, w.win_l, w.win_r,
                                         heads=[(b, hq) for b in range(w.n)])
                    t += time.perf_counter() - t0
                    print(f"{name} forward head {hq}: {t:.1f} s", file=sys.stderr,
                          flush=True)
            else:
                t0 = time.perf_counter()
                fwd()
                t = time.perf_counter() - t0
            best = min(best, t)
        r = {"fwd_s": round(best, 3), "runs": reps,
             "fwd_tflops": round(fwd_flops(w.n, w.h, w.d, pairs) / best / 1e12, 5)}
        if w.backward:
            tb = 0.0
            for g in range(w.h_kv):
                t0 = time.perf_counter()
                oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], w.softmax_scale,
                                     w.causal, w.win_l, w.win_r,
                                     kv_heads=[(b, g) for b in range(w.n)])
                tb += time.perf_counter() - t0
                print(f"{name} backward head {g}: {tb:.1f} s", file=sys.stderr,
                      flush=True)
            r["bwd_s"] = round(tb, 3)
            r["bwd_tflops"] = round(bwd_flops(w.n, w.h, w.d, pairs) / tb / 1e12, 5)
        res[name] = r
        print(json.dumps({name: r}), file=sys.stderr, flush=True)
    return res


def _host_description():
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = os.cpu_count() or 1
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [threads])
    except Exception:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else threads
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable,
            "blas_threads": threads}


def copy_calibration(nbytes):
    """A plain device-to-device copy of nbytes, ten times: the reference that
    the FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": int(src.numel() * 4), "copies": 10}))


def main():
    global SETTLE_MS
    args = parse()
    SETTLE_MS = args.settle_ms
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): the "
              "path runs on one GPU's share; its multi-GPU form is not provided",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.oracle_times:
        print(json.dumps({"oracle_times": oracle_times()}), flush=True)
        return
    import torch
    from blockwise_exact_attention_amd import attention as A
    from blockwise_exact_attention_amd.flops import (allowed_pairs, fwd_flops,
                                                     fwd_bytes, bwd_flops,
                                                     merge_bytes)
    from blockwise_exact_attention_amd.workloads import WORKLOADS, make_inputs
    if args.merge_only:
        print(json.dumps({"merge": merge_measurements(A, torch, merge_bytes,
                                                      args.steps)}), flush=True)
        return
    if args.workload != "c2":
        # one workload's timed loop alone (for profiler runs)
        fn, flops, what = single_workload(args.workload, A, torch, allowed_pairs,
                                          fwd_flops, bwd_flops, WORKLOADS, make_inputs)
        ms = timed(fn, args.steps, args.warmup, torch)
        print(json.dumps({"workload": args.workload, "what": what, "steps": args.steps,
                          "ms": round(ms, 5),
                          "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                          "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12
                                                     / PEAK_BF16_TFLOPS, 4)}), flush=True)
        return

    w = WORKLOADS["C2"]
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x[s]).to(torch.bfloat16).to(dev)
                  for s in ("q", "k", "v"))
    out = torch.empty_like(tq)
    lse = torch.empty((w.n, w.h, w.l_q), dtype=torch.float32, device=dev)
    pairs = allowed_pairs(w.l_q, w.l_k, True)
    flops = fwd_flops(w.n, w.h, w.d, pairs)
    kernel = A.fwd_kernel_name(w.n, w.l_q, w.l_k, w.h, w.h_kv, w.d, True)

    def step():
        A.attn_fwd(tq, tk, tv, out, lse, w.softmax_scale, True)

    settle_calls = settle(step, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed region: K launches back to back on the launch stream.  One
    # event pair around them gives the GPU time per launch (the host queues
    # launches faster than they run); the host clock gives time per step.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    kern_ms = start.elapsed_time(end) / args.steps
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12

    rec = {
        "metric": "attention fwd TFLOP/s (causal bf16, d=128) and % of MFMA bf16 peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "settle_calls": settle_calls,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "n": w.n, "l": w.l_q, "h": w.h,
                   "h_kv": w.h_kv, "d": w.d, "causal": True,
                   "allowed_pairs_per_head": pairs,
                   "algorithmic_gflop": round(flops / 1e9, 3)},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": counted_traffic(kernel),
                     "kernel": kernel,
                     "kernel_ms_per_launch": round(kern_ms, 5),
                     "algorithmic_bytes": fwd_bytes(w.n, w.l_q, w.l_k, w.h,
                                                    w.h_kv, w.d, 2)},
    }
    del tq, tk, tv, out, lse

    if not args.no_extras:
        rec["extras"] = extras(A, torch, args, allowed_pairs, fwd_flops,
                               bwd_flops, merge_bytes, WORKLOADS, make_inputs)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(x, w, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def _frac(tflops):
    return round(tflops / PEAK_BF16_TFLOPS, 4)


def _dev_bf16(torch, a):
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.device("cuda:0"))


def single_workload(name, A, torch, allowed_pairs, fwd_flops, bwd_flops, WORKLOADS,
                    make_inputs):
    """(callable, algorithmic FLOPs per call, description) of one workload's
    timed call, inputs resident on the GPU."""
    t = lambda a: _dev_bf16(torch, a)
    dev = torch.device("cuda:0")
    if name.startswith("c3"):
        w = WORKLOADS["C3"]
        x = make_inputs(w)
        tq = t(x["q"])
        kc = [t(c) for c in x["k_chunks"]]
        vc = [t(c) for c in x["v_chunks"]]
        offs = x["k_offsets"]
        pairs = sum(allowed_pairs(1024, 1024, True, -1, -1, x["q_offset"], ko) for ko in offs)
        share = A.RingShare(tq, w.softmax_scale, True, x["q_offset"])
        if name == "c3-steps":
            def fn():
                for s in range(8):
                    A.attn_fwd(tq, kc[s], vc[s], share.blk, share.lse_blk, w.softmax_scale,
                               True, -1, -1, x["q_offset"], offs[s])
            return fn, fwd_flops(1, 32, 128, pairs), "the 8 per-chunk forwards of the rank-7 share"
        if name == "c3-fused":
            return (lambda: share.run(kc, vc, offs, fused=True), fwd_flops(1, 32, 128, pairs),
                    "rank-7 share as 8 fused steps (init, 8 x attn_fwd_acc, cast)")
        if name == "c3-share":
            return (lambda: share.run(kc, vc, offs, one_launch=True),
                    fwd_flops(1, 32, 128, pairs), "rank-7 share in one attn_fwd_ring launch")
        if name in ("c3-bwd", "c3-bwd-one"):
            tdo = t(np.random.default_rng(77).standard_normal(x["q"].shape).astype(np.float32))
            o, l = share.run(kc, vc, offs, one_launch=True)
            b = A.RingShareBwd(tq, o.clone(), l.clone(), tdo, w.softmax_scale, True,
                               x["q_offset"])
            one = name == "c3-bwd-one"
            return (lambda: b.run(kc, vc, offs, one_launch=one), bwd_flops(1, 32, 128, pairs),
                    "rank-7 ring backward share" + (" in three launches" if one else ""))
    if name == "c4":
        w = WORKLOADS["C4"]
        x = make_inputs(w)
        tq, tk, tv = t(x["q"]), t(x["k"]), t(x["v"])
        o = torch.empty_like(tq)
        lse = torch.empty((w.n, w.h, w.l_q), dtype=torch.float32, device=dev)
        pairs = allowed_pairs(w.l_q, w.l_k, True, w.win_l, w.win_r)
        return (lambda: A.attn_fwd(tq, tk, tv, o, lse, w.softmax_scale, True, w.win_l,
                                   w.win_r), fwd_flops(w.n, w.h, w.d, pairs),
                "sliding-window forward")
    if name.startswith("c5"):
        w = WORKLOADS["C5"]
        x = make_inputs(w)
        tq, tk, tv = t(x["q"]), t(x["k"]), t(x["v"])
        o = torch.empty_like(tq)
        lse = torch.empty((w.n, w.h, w.l_q), dtype=torch.float32, device=dev)
        pairs = allowed_pairs(w.l_q, w.l_k, True)
        if name == "c5-fwd":
            return (lambda: A.attn_fwd(tq, tk, tv, o, lse, w.softmax_scale, True),
                    fwd_flops(w.n, w.h, w.d, pairs), "16k-token causal forward")
        tdo = t(x["do"])
        A.attn_fwd(tq, tk, tv, o, lse, w.softmax_scale, True)
        dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
        ws = torch.empty(A.bwd_workspace_bytes(w.n, w.l_q, w.l_k, w.h, w.h_kv, w.d),
                         dtype=torch.uint8, device=dev)
        return (lambda: A.attn_bwd(tdo, tq, tk, tv, o, lse, dq, dk, dv, w.softmax_scale,
                                   True, workspace=ws), bwd_flops(w.n, w.h, w.d, pairs),
                "16k-token causal backward")
    if name.startswith("mqa"):
        # the headline and 16k-token causal forwards with one key/value head
        # (multi-query): the first K/V head of the same inputs
        w = WORKLOADS["C2" if name == "mqa-c2" else "C5"]
        x = make_inputs(w)
        tq = t(x["q"])
        tk = t(np.ascontiguousarray(x["k"][:, :, :1]))
        tv = t(np.ascontiguousarray(x["v"][:, :, :1]))
        o = torch.empty_like(tq)
        lse = torch.empty((w.n, w.h, w.l_q), dtype=torch.float32, device=dev)
        pairs = allowed_pairs(w.l_q, w.l_k, True)
        return (lambda: A.attn_fwd(tq, tk, tv, o, lse, w.softmax_scale, True),
                fwd_flops(w.n, w.h, w.d, pairs),
                f"causal MQA forward n={w.n} l={w.l_q} h={w.h} h_kv=1 d={w.d}")
    raise ValueError(f"unknown workload {name}")


def extras(A, torch, args, allowed_pairs, fwd_flops, bwd_flops, merge_bytes,
           WORKLOADS, make_inputs):
    """Every other targeted figure, each timed on its own: the rank-7 ring
    share (per-chunk forwards, fused steps, one launch, all-gathered keys,
    backward), the sliding window, the 16k-token forward and backward, and
    the merge's bandwidth warm and cold."""
    dev = torch.device("cuda:0")
    res = {}
    steps = max(10, args.steps // 4)
    t = lambda a: _dev_bf16(torch, a)

    w = WORKLOADS["C3"]
    x = make_inputs(w)
    tq = t(x["q"])
    kc = [t(c) for c in x["k_chunks"]]
    vc = [t(c) for c in x["v_chunks"]]
    offs = x["k_offsets"]
    share = A.RingShare(tq, w.softmax_scale, True, x["q_offset"])
    pairs = sum(allowed_pairs(1024, 1024, True, -1, -1, 7168, ko) for ko in offs)
    fl = fwd_flops(1, 32, 128, pairs)
    fwd_ms = []
    for s in range(8):
        def f(s=s):
            A.attn_fwd(tq, kc[s], vc[s], share.blk, share.lse_blk,
                       w.softmax_scale, True, -1, -1, x["q_offset"], offs[s])
        fwd_ms.append(timed(f, steps, 5, torch))
    A.attn_acc_init(share.acc, share.lse_acc)
    merge_ms = timed(lambda: A.attn_merge(share.acc, share.lse_acc, share.blk,
                                          share.lse_blk), steps, 5, torch)
    e2e = timed(lambda: share.run(kc, vc, offs), steps, 3, torch)
    e2e_fused = timed(lambda: share.run(kc, vc, offs, fused=True), steps, 3, torch)
    e2e_one = timed(lambda: share.run(kc, vc, offs, one_launch=True), steps, 3, torch)
    # the all-gather form of the same share: the 8 chunks side by side, one
    # attn_fwd with the share's absolute query offset
    kf, vf = t(x["k_full"]), t(x["v_full"])
    ag_out = torch.empty_like(tq)
    ag_lse = torch.empty((1, 32, 1024), dtype=torch.float32, device=dev)
    ag_ms = timed(lambda: A.attn_fwd(tq, kf, vf, ag_out, ag_lse, w.softmax_scale, True,
                                     -1, -1, x["q_offset"], 0), steps, 3, torch)
    # the ring backward share of the same rank (dO drawn like the inputs)
    tdo = t(np.random.default_rng(77).standard_normal(x["q"].shape).astype(np.float32))
    out, lse = share.run(kc, vc, offs, one_launch=True)
    bshare = A.RingShareBwd(tq, out.clone(), lse.clone(), tdo, w.softmax_scale,
                            True, x["q_offset"])
    bwd_ms = timed(lambda: bshare.run(kc, vc, offs), max(5, steps // 4), 2, torch)
    bwd_one_ms = timed(lambda: bshare.run(kc, vc, offs, one_launch=True), max(5, steps // 4),
                       2, torch)
    mb = merge_bytes(1, 1024, 32, 128, 2)
    tf = lambda ms, f=fl: round(f / (ms * 1e-3) / 1e12, 2)
    bfl = bwd_flops(1, 32, 128, pairs)
    res["ring_share_rank7"] = {
        "algorithmic_gflop": round(fl / 1e9, 3),
        "step_kernel": A.fwd_kernel_name(1, 1024, 1024, 32, 8, 128, True,
                                         q_offset=7168, k_offset=0),
        "fwd_ms_per_step": [round(v, 4) for v in fwd_ms],
        "fwd_ms_sum_of_8": round(sum(fwd_ms), 4),
        "fwd_tflops_sum_of_8": tf(sum(fwd_ms)),
        "fwd_frac_sum_of_8": _frac(tf(sum(fwd_ms))),
        "merge_ms": round(merge_ms, 4),
        "merge_gbs_warm": round(mb / (merge_ms * 1e-3) / 1e9, 1),
        "unfused_ms": round(e2e, 4),
        "unfused_tflops": tf(e2e),
        "fused_steps_ms": round(e2e_fused, 4),
        "fused_steps_tflops": tf(e2e_fused),
        "fused_steps_frac": _frac(tf(e2e_fused)),
        "one_launch_kernel": "fwd_pipe_kernel (8 chunks)",
        "one_launch_ms": round(e2e_one, 4),
        "one_launch_tflops": tf(e2e_one),
        "one_launch_frac": _frac(tf(e2e_one)),
        "all_gather_ms": round(ag_ms, 4),
        "all_gather_tflops": tf(ag_ms),
        "backward_share_ms": round(bwd_ms, 4),
        "backward_share_tflops": tf(bwd_ms, bfl),
        "backward_share_frac": _frac(tf(bwd_ms, bfl)),
        "backward_share_one_launch_ms": round(bwd_one_ms, 4),
        "backward_share_one_launch_tflops": tf(bwd_one_ms, bfl),
        "backward_share_one_launch_frac": _frac(tf(bwd_one_ms, bfl))}
    del bshare, tdo, kf, vf, ag_out, ag_lse, share, kc, vc, tq

    for key, name in (("window_256", "c4"), ("long_16k_fwd", "c5-fwd"),
                      ("long_16k_bwd", "c5-bwd"), ("mqa_c2", "mqa-c2"),
                      ("mqa_16k_fwd", "mqa-c5")):
        fn, flops, what = single_workload(name, A, torch, allowed_pairs, fwd_flops,
                                          bwd_flops, WORKLOADS, make_inputs)
        n_steps = steps if name in ("c4", "mqa-c2") else max(5, steps // 8)
        ms = timed(fn, n_steps, 3, torch)
        r = {"what": what, "ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
             "frac": _frac(flops / (ms * 1e-3) / 1e12)}
        if name == "c4":
            r["kernel"] = A.fwd_kernel_name(4, 4096, 4096, 16, 16, 64, True, 256, 0)
        if name == "c5-fwd":
            r["kernel"] = A.fwd_kernel_name(1, 16384, 16384, 16, 16, 128, True)
        if name == "mqa-c2":
            r["kernel"] = A.fwd_kernel_name(2, 2048, 2048, 16, 1, 128, True)
        if name == "mqa-c5":
            r["kernel"] = A.fwd_kernel_name(1, 16384, 16384, 16, 1, 128, True)
        res[key] = r
        del fn
        torch.cuda.empty_cache()
    res["merge"] = merge_measurements(A, torch, merge_bytes, steps)
    return res


if __name__ == "__main__":
    main()
