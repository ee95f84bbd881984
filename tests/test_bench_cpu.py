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


def test_oracle_leg_counts_against_known_outputs():
    """The bench's block-by-block comparison, fed the oracle's own outputs (logp and LSE
    rounded to float32, dlogits rounded to BF16): every element is correctly rounded and the
    largest error is the BF16 floor; one planted wrong element is counted."""
    import numpy as np
    import torch

    import oracle
    from workloads import random_case

    case = random_case(40, 5000, sigma=3.0, seed=4)
    case.meta["spike_row_index"] = [5, 7]
    y = case.targets.numpy()
    ref = oracle.forward(case.logits, y, 5000)
    d = oracle.backward(case.logits, y, case.grad.numpy(), 5000)
    logp = torch.from_numpy(ref["logp"].astype(np.float32))
    lse = torch.from_numpy(ref["lse"].astype(np.float32))
    bits = torch.from_numpy(d["bf16"].view(np.int16)).view(torch.bfloat16)
    leg = bench.oracle_leg(case, (logp, lse, None, bits), bwd_rows=16, threads=3, block=8)
    acc = leg["accuracy"]
    assert acc["rows_forward"] == 40 and acc["rows_backward"] == 16  # rows 5, 7 in the spread
    assert acc["dlogits"]["elements"] == 16 * 5000 and acc["dlogits"]["misrounded"] == 0
    assert acc["dlogits"]["max_err"] == acc["dlogits"]["floor"] > 0
    assert acc["logp_abs_err"]["max"] <= 2.0 ** -24 * 20 and acc["lse_abs_err"]["max"] < 1e-5
    # one element moved by one BF16 spacing on a sampled row
    wrong = bits.clone()
    w = wrong.view(torch.int16)
    w[0, 11] += 1
    leg2 = bench.oracle_leg(case, (logp, lse, None, wrong), bwd_rows=16, threads=2, block=5)
    assert leg2["accuracy"]["dlogits"]["misrounded"] == 1
    assert leg2["accuracy"]["dlogits"]["max_err"] >= acc["dlogits"]["max_err"]
    cpu = bench.cpu_baseline(leg, case, threads=3)
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] == 3


def test_ceiling_probes_validate_arguments_on_the_host():
    """The bench's ceiling probes refuse bad arguments before any launch (code 1), the
    matrix-core probe's flop count is its MFMA count times 2 x 32 x 32 x 16, and the LDS
    probe's byte counts are its accesses times their widths."""
    import ctypes
    import os

    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes")
    mfma = ctypes.CDLL(os.path.join(here, "libmfma_ceiling.so"))
    mfma.mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    mfma.mfma_bf16_flops.restype = ctypes.c_double
    mfma.mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                               ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    per = 2.0 * 32 * 32 * 16
    assert mfma.mfma_bf16_flops(4, 1024, 5000) == 1024 * 4 * 5000 * 16 * per
    assert mfma.mfma_bf16_flops(8, 256, 10) == 256 * 8 * 10 * 8 * per
    for bad in ((2, 1, 1), (4, 0, 1), (4, 1, 0), (8, 1 << 31, 1)):
        assert mfma.mfma_bf16_flops(*bad) == -1.0
        assert mfma.mfma_bf16(*bad, 1, 1, ctypes.c_void_p(0x1000), None) == 1
    assert mfma.mfma_bf16(4, 1, 1, 1, 1, None, None) == 1
    assert mfma.mfma_bf16(4, 1, 1, 1, 2, ctypes.c_void_p(0x1000), None) == 1  # toggle 0 or 1
    hbm = ctypes.CDLL(os.path.join(here, "libhbm_ceiling.so"))
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    hbm.hbm_read.argtypes = [P, I64, I32, I32, ctypes.c_uint32, P, P]
    hbm.hbm_copy.argtypes = [P, P, I64, I32, I32, P]
    a, b = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x8000000)
    assert hbm.hbm_read(a, 1 << 20, 7, 4, 0, b, None) == 1      # no such shape
    assert hbm.hbm_read(a, 1000, 8, 4, 0, b, None) == 1         # not whole chunks
    assert hbm.hbm_copy(a, ctypes.c_void_p(0x10010), 1 << 20, 8, 4, None) == 1  # overlap
    hbm.hbm_copy_nt.argtypes = [P, P, I64, P]
    hbm.hbm_write.argtypes = [P, I64, ctypes.c_uint32, P]
    assert hbm.hbm_copy_nt(a, ctypes.c_void_p(0x10010), 1 << 20, None) == 1      # overlap
    assert hbm.hbm_copy_nt(a, b, 1000, None) == 1                                # not whole chunks
    assert hbm.hbm_write(None, 1 << 20, 0, None) == 1
    assert hbm.hbm_write(ctypes.c_void_p(0x10008), 1 << 20, 0, None) == 1      # misaligned
    assert hbm.hbm_write(a, (16 << 10) + 16, 0, None) == 1                      # not whole chunks
    lds = ctypes.CDLL(os.path.join(here, "liblds_ceiling.so"))
    lds.lds_read.argtypes = [I32, I64, I32, I32, P, P, P]
    lds.lds_dma.argtypes = [I32, I64, I32, P, I64, P, P, P]
    lds.lds_read_bytes.argtypes = [I32, I32, I32]
    lds.lds_read_bytes.restype = ctypes.c_double
    lds.lds_dma_bytes.argtypes = [I32, I32]
    lds.lds_dma_bytes.restype = ctypes.c_double
    assert lds.lds_read_bytes(8, 10, 16) == 8 * 10 * 16 * 64 * 16
    assert lds.lds_dma_bytes(4, 10) == 4 * 10 * 8 * 1024
    assert lds.lds_read_bytes(8, 10, 12) == -1.0 and lds.lds_dma_bytes(16, 10) == -1.0
    assert lds.lds_read(8, 1, 1, 12, b, b, None) == 1                # no such width
    assert lds.lds_read(6, 1, 1, 16, b, b, None) == 1                # no such wave count
    assert lds.lds_read(8, 1, 1, 16, None, b, None) == 1
    assert lds.lds_dma(8, 1, 1, a, 4096, b, b, None) == 1            # source under 8 KiB
    assert lds.lds_dma(8, 1, 1, a, 8192 + 512, b, b, None) == 1      # not whole KiB
    assert lds.lds_dma(16, 1, 1, a, 8192, b, b, None) == 1           # 16 waves do not fit
