"""linear_logp_backward_noalloc (the entry point for callers that cannot allocate) against
linear_logp_backward_ex with a caller workspace: the same chunked products, so the same bits.

Two calls in a row on one stream, the second with a smaller input: the static scratch array
keeps the first call's contents, and the second call must not depend on them.  After a first
call on the device, a call must not change the device's free memory (it allocates nothing).
"""

from __future__ import annotations

import pytest
import torch

import deterministic_selected_token_amd as dst
from deterministic_selected_token_amd import linear

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def make(n, H, V, seed):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn((n, H), generator=g).to(torch.bfloat16)
    W = (torch.randn((V, H), generator=g) * (3.0 / H ** 0.5)).to(torch.bfloat16)
    y = torch.randint(0, V, (n,), generator=g)
    y[torch.rand(n, generator=g) < 0.1] = -100
    active = (torch.rand(n, generator=g) >= 0.1).to(torch.uint8)
    grad = torch.randn(n, generator=g) * 0.1
    return h.to(DEV), W.to(DEV), y.to(DEV), active.to(DEV), grad.to(DEV)


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return a.shape == b.shape and torch.equal(a.view(torch.int32), b.view(torch.int32))


# n, H, V, inv_temperature, chunk_cols: the second call is the smaller one
CASES = [(300, 1024, 10000, 1.0 / 0.7, 4096), (97, 256, 5000, 1.0, 4096)]


def run_pair(n, H, V, inv_t, chunk, seed):
    say(f"noalloc backward: n={n} H={H} V={V} inv_t={inv_t:.4f} chunk={chunk}")
    h, W, y, active, g = make(n, H, V, seed)
    _, _, stats = linear.linear_logp_forward(h, W, y, V, V, active=active,
                                             inv_temperature=inv_t)
    ref_dh, ref_dw = linear.linear_logp_backward(h, W, y, g, stats, V, V, active=active,
                                                 inv_temperature=inv_t, chunk_cols=chunk)
    dh = torch.full((n, H), float("nan"), device=DEV)
    dw = torch.full((V, H), float("nan"), device=DEV)
    linear.linear_logp_backward(h, W, y, g, stats, V, V, active=active, inv_temperature=inv_t,
                                chunk_cols=chunk, dhidden=dh, dweight=dw, noalloc=True)
    torch.cuda.synchronize()
    assert same_bits(dh, ref_dh) and same_bits(dw, ref_dw)
    assert torch.count_nonzero(dh) > 0 and torch.count_nonzero(dw) > 0
    return h, W, y, active, g, stats, dh, dw


def test_noalloc_matches_the_workspace_entry_point_on_two_calls_in_a_row():
    for seed, case in enumerate(CASES):
        run_pair(*case, seed=seed)


def test_noalloc_allocates_nothing():
    n, H, V, inv_t, chunk = CASES[1]
    h, W, y, active, g, stats, dh, dw = run_pair(n, H, V, inv_t, chunk, seed=7)
    out_dh, out_dw = torch.empty_like(dh), torch.empty_like(dw)
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info()[0]  # device-wide free bytes (hipMemGetInfo)
    allocated = torch.cuda.memory_allocated()
    linear.linear_logp_backward(h, W, y, g, stats, V, V, active=active, inv_temperature=inv_t,
                                chunk_cols=chunk, dhidden=out_dh, dweight=out_dw, noalloc=True)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free_before
    assert torch.cuda.memory_allocated() == allocated
    assert same_bits(out_dh, dh) and same_bits(out_dw, dw)


def test_noalloc_refuses_work_beyond_its_scratch_array():
    n, H, V = 4097, 4096, 4096
    assert linear.linear_logp_backward_workspace(n, H, 4096) > linear.NOALLOC_SCRATCH_BYTES
    say(f"noalloc backward beyond the scratch array: n={n} H={H} V={V}")
    h, W, y, active, g = make(n, H, V, seed=3)
    stats = torch.zeros((n, 2), device=DEV)
    with pytest.raises(dst.LogpError) as err:
        linear.linear_logp_backward(h, W, y, g, stats, V, V, chunk_cols=4096, noalloc=True)
    assert err.value.status == 9  # LOGP_ERR_SCRATCH, nothing launched
