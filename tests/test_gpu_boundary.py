"""Boundary behaviour on the GPU: device-pointer and extent checks, overlap rejection,
empty batches, the loud target check, and the long-sequence row count (131072 rows) with
a bounded workspace (peak memory = returned gradient + O(N))."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst
import oracle
from parity_checks import BackwardTally, bits_of, check_forward
from workloads import long_case, random_case
from workloads.synth import QWEN_VOCAB

pytestmark = pytest.mark.gpu
DEV = "cuda"
DEVICE_ERR, RANGE_ERR, OVERLAP_ERR = 4, 5, 6


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def raw_forward(logits_ptr, ld, n, v, targets_ptr, logp_ptr, lse_ptr=None, stats_ptr=None):
    return dst.library().logp_forward(logits_ptr, ld, n, v, v, targets_ptr, None, -100,
                                      logp_ptr, lse_ptr, stats_ptr, None)


def test_host_pointers_are_rejected():
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros(4, dtype=torch.int64, device=DEV)
    out = torch.empty(4, dtype=torch.float32, device=DEV)
    host_x = torch.zeros((4, 64), dtype=torch.bfloat16)
    host_out = torch.empty(4, dtype=torch.float32)
    say("host pointers")
    assert raw_forward(host_x.data_ptr(), 64, 4, 64, y.data_ptr(), out.data_ptr()) == DEVICE_ERR
    assert raw_forward(x.data_ptr(), 64, 4, 64, y.data_ptr(), host_out.data_ptr()) == DEVICE_ERR
    # the call left no error behind for the caller's next HIP operation
    torch.cuda.synchronize()
    assert torch.all(x == 0)


def test_extent_past_the_allocation_is_rejected():
    torch.cuda.empty_cache()
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros(1 << 20, dtype=torch.int64, device=DEV)
    out = torch.empty(1 << 20, dtype=torch.float32, device=DEV)
    say("extent check")
    # claim 2^20 rows of 2^20 columns: ~2 TiB of logits that the allocation cannot hold
    rc = dst.library().logp_forward(x.data_ptr(), 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                    y.data_ptr(), None, -100, out.data_ptr(), None, None, None)
    assert rc == RANGE_ERR


def test_overlapping_outputs_are_rejected():
    x = torch.randn((4, 64), device=DEV).to(torch.bfloat16)
    y = torch.zeros(8, dtype=torch.int64, device=DEV)
    say("overlap check")
    # logp written over the targets
    assert raw_forward(x.data_ptr(), 64, 4, 64, y.data_ptr(), y.data_ptr()) == OVERLAP_ERR
    # logp and lse on the same buffer
    out = torch.empty(8, dtype=torch.float32, device=DEV)
    assert raw_forward(x.data_ptr(), 64, 4, 64, y.data_ptr(), out.data_ptr(),
                       out.data_ptr() + 4) == OVERLAP_ERR
    # dlogits partially overlapping the logits (not an exact alias) is rejected
    _, _, stats = dst.logp_forward(x, y[:4])
    g = torch.ones(4, device=DEV)
    with pytest.raises(dst.LogpError, match="OVERLAP"):
        dst.logp_backward(x[:, :32], y[:4], g, stats, dlogits=x[:, 16:48])


def test_empty_batch():
    x = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    y = torch.empty(0, dtype=torch.int64, device=DEV)
    say("empty batch")
    logp, lse, stats = dst.logp_forward(x, y)
    d = dst.logp_backward(x, y, torch.empty(0, device=DEV), stats)
    assert logp.numel() == 0 and d.shape == (0, 128)
    bad = dst.logp_check_targets(y, 128, bad_count=torch.full((1,), 7, device=DEV))
    assert int(bad) == 0


def test_check_targets_counts_bad_active_targets():
    case = random_case(5000, 1000, 1024, seed=5, device=DEV, inactive_frac=0.2,
                       ignore_frac=0.1, bad_target_frac=0.1)
    say("check_targets")
    got = dst.logp_check_targets(case.targets, case.vocab_real, active=case.active)
    want = oracle.count_bad_targets(case.targets.cpu(), case.vocab_real,
                                    active=case.active.cpu())
    assert int(got) == want > 0
    assert int(dst.logp_check_targets(case.targets, case.vocab_real)) == \
        oracle.count_bad_targets(case.targets.cpu(), case.vocab_real)


def test_long_sequence_131072_rows_bounded_workspace():
    n, v = 131072, QWEN_VOCAB
    say(f"long sequence: n={n} V={v} ({2 * n * v / 2**30:.1f} GiB logits)")
    case = long_case(device=DEV, n=n)
    logits, y, g = case.logits, case.targets, case.grad
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    logp, lse, stats = dst.logp_forward(logits, y)
    d = dst.logp_backward(logits, y, g, stats)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    grad_bytes = d.numel() * d.element_size()
    say(f"long sequence: peak - base = {peak / 2**30:.3f} GiB, grad {grad_bytes / 2**30:.3f} GiB")
    assert grad_bytes <= peak <= grad_bytes + 64 * n + (2 << 20)
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(1).choice(n, 30)]))
    rt = torch.from_numpy(rows).to(DEV)
    host = logits[rt].cpu()
    check_forward(host, y[rt].cpu().numpy(), v, None, -100, logp[rt].cpu().numpy(),
                  lse[rt].cpu().numpy(), stats[rt].cpu().numpy(), "long sequence")
    t = BackwardTally()
    t.add_block(host, y[rt].cpu().numpy(), g[rt].cpu().numpy(), v, v, None, -100,
                bits_of(d[rt]), "long sequence")
    say(f"long sequence: {t.finish('long sequence')}")
