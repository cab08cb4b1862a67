"""Host-side pieces of bench.py (no GPU): the multi-GPU refusal, the
counter-traffic lookup that only reports bytes taken on the current kernel
sources, and the algorithmic work and byte counts the bench line uses."""
import json
import os
import subprocess
import sys

import bench
from blockwise_exact_attention_amd.flops import (allowed_pairs, bwd_flops,
                                                 fwd_bytes, fwd_flops,
                                                 merge_bytes)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counted_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    """Bytes are reported only from a counter summary of the same kernel whose
    recorded sha256 equals that of the kernel's current sources."""
    os.symlink(os.path.join(ROOT, "blockwise_exact_attention_amd"),
               tmp_path / "blockwise_exact_attention_amd")
    (tmp_path / "profiles").mkdir()
    path = tmp_path / "profiles" / bench.COUNTERS_JSON
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    kern = "fwd_bf16_kernel<128, 64, 2, false>"
    assert bench.counted_traffic(kern) is None          # no summary at all
    sha = bench.kernel_sources_sha256(kern)
    path.write_text(json.dumps({"kernel": kern, "kernel_sources_sha256": sha,
                                "hbm_bytes_per_launch": 12345}))
    assert bench.counted_traffic(kern) == 12345
    # another kernel, or the other kernel file's sources
    assert bench.counted_traffic("fwd_bf16_kernel<128, 64, 1, false>") is None
    assert bench.kernel_sources_sha256("fwd_pipe_kernel<128, 2, false, false>") != sha
    path.write_text(json.dumps({"kernel": kern, "kernel_sources_sha256": "0" * 64,
                                "hbm_bytes_per_launch": 12345}))
    assert bench.counted_traffic(kern) is None


def test_workload_counts():
    # C2: 2 x 16 heads of causal 2048 x 2048, d = 128
    pairs = allowed_pairs(2048, 2048, True)
    assert pairs == 2048 * 2049 // 2
    assert fwd_flops(2, 16, 128, pairs) == 4 * 128 * pairs * 32
    assert bwd_flops(2, 16, 128, pairs) == 2.5 * fwd_flops(2, 16, 128, pairs)
    # q, k, v read once, O (bf16) and LSE written once
    assert fwd_bytes(2, 2048, 2048, 16, 16, 128, 2) == 4 * 2 * 2048 * 16 * 128 * 2 + 2 * 16 * 2048 * 4
    # merge: fp32 accumulator read and written, bf16 block read, three LSE vectors
    assert merge_bytes(1, 1024, 32, 128, 2) == 1024 * 32 * 128 * 10 + 3 * 32 * 1024 * 4
