"""Host-side parts of bench.py that need no GPU: the one-GPU refusal, the algorithmic byte
counts of the headline step, the median helper, and the rule that HBM traffic is reported
only for the kernel sources the counters were taken with."""

from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_multi_process_launch_is_refused():
    r = run_bench([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "single process" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_headline_step():
    # forward: the logits once + targets 8, logp 4, LSE 4, stats 8 per row;
    # backward: the logits once (valid rows) + dlogits once + targets 8, g 4, stats 8 per row
    fwd, bwd = bench.algorithmic_bytes(32768, 32768, 151936, 151936, False)
    assert fwd == 2 * 32768 * 151936 + 24 * 32768 == 9_958_064_128
    assert bwd == 4 * 32768 * 151936 + 20 * 32768 == 19_915_210_752
    # an active mask adds one byte per row to each; invalid rows are not read
    fwd_m, bwd_m = bench.algorithmic_bytes(10, 7, 100, 128, True, elem=4)
    assert fwd_m == 4 * 10 * 100 + 25 * 10
    assert bwd_m == 4 * 7 * 100 + 4 * 10 * 128 + 21 * 10


def test_median():
    assert bench.median([3.0, 1.0, 2.0]) == 2.0
    assert bench.median([4.0, 1.0, 2.0, 3.0]) == 2.5


def test_traffic_is_null_once_the_kernel_sources_differ(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("bwd") is None
    assert bench.measured_traffic("fwd") is None
