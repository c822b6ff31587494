"""Host logic of bench.py on the CPU: the one-GPU refusal, the algorithmic
work it divides by (closed forms on the tiny workload), and the gating of
committed counter summaries by the kernel source hash."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_tiny_closed_form():
    wl = workloads.generate("tiny")
    nbytes, flops, pairs = bench.algorithmic_work(wl)
    N, q, H, H_kv, d, s = 144, 16, 4, 4, 64, 4
    # K and V of every key, Q and out of every row, the impact vector
    assert nbytes == N * 2 * H_kv * d * s + q * 2 * H * d * s + N * 4
    # query rows at the last q positions: each sees the 128 document keys and
    # the query keys up to its own position
    assert pairs == q * 128 + q * (q + 1) // 2 == 2184
    assert flops == 4 * pairs * H * d


def test_algorithmic_work_decode_has_no_impact_bytes():
    wl = workloads.generate("llama3_8b_decode_32l", problems=[0])
    nbytes, flops, pairs = bench.algorithmic_work(wl)
    N = 10000 + 228
    assert nbytes == N * 2 * 8 * 128 * 2 + 1 * 2 * 32 * 128 * 2
    assert pairs == N


def test_counter_summaries_follow_the_kernel_source(monkeypatch):
    t = bench.measured_traffic("llama3_8b_gqa_32l", "attn")
    m = bench.measured_mfma("llama3_8b_gqa_32l")
    if t is None or m is None:
        pytest.skip("committed summaries were taken on other kernel sources")
    assert t > 1.0e9 and m["executed_flops_per_launch"] > 5.0e11
    monkeypatch.setattr(bench, "kernel_source_sha", lambda kind="attn": "0000000000000000")
    assert bench.measured_traffic("llama3_8b_gqa_32l", "attn") is None
    assert bench.measured_mfma("llama3_8b_gqa_32l") is None
