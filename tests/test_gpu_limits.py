"""Widest rows: the fused forward at its limit of 4096 tiles (16,777,216 columns) with a
ragged real vocabulary, one tile more (the fused forward refuses it; partials + merge take
it), and one row of 2^30 + 776 columns through partials + merge and the backward, checked
against the oracle on the forward and on sampled gradient elements."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst
import oracle
from parity_checks import BackwardTally, check_forward, host_values, spacing

pytestmark = pytest.mark.gpu
DEV = "cuda"
T = dst.TILE_COLS


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def gaussian_bf16(n, width, seed, sigma=3.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    out = torch.empty((n, width), dtype=torch.bfloat16, device=DEV)
    step = 1 << 24  # bounded float32 staging
    for c0 in range(0, width, step):
        c1 = min(width, c0 + step)
        out[:, c0:c1] = (torch.randn((n, c1 - c0), generator=g, device=DEV) * sigma)
    return out


def test_fused_forward_at_the_tile_limit_and_one_tile_more():
    n, P = 3, T * dst.FWD_MAX_TILES          # 16,777,216 columns
    V = P - 5
    say(f"fused forward + backward at {P} columns")
    x = gaussian_bf16(n, P, seed=5)
    y = torch.tensor([0, V - 1, 12_345_678], device=DEV)
    g = torch.tensor([1.0, -0.5, 0.25], device=DEV)
    logp, lse, stats = dst.logp_forward(x, y, V, P)
    d = dst.logp_backward(x, y, g, stats, V, P)
    torch.cuda.synchronize()
    host = x.cpu()
    yh, gh = y.cpu().numpy(), g.cpu().numpy()
    fwd = check_forward(host, yh, V, None, -100, logp.cpu().numpy(), lse.cpu().numpy(),
                        stats.cpu().numpy(), "tile limit")
    t = BackwardTally()
    t.add_block(host, yh, gh, V, P, None, -100, host_values(d), "tile limit")
    bwd = t.finish("tile limit")
    say(f"tile limit: {fwd} {bwd}")
    del d

    # one tile more: the fused forward has no LDS slot for it; partials + merge do
    P2 = P + T
    x2 = torch.zeros((n, P2), dtype=torch.bfloat16, device=DEV)
    x2[:, :P] = x
    x2[:, P:] = gaussian_bf16(n, T, seed=6)
    with pytest.raises(dst.LogpError, match="SHAPE"):
        dst.logp_forward(x2, y, P2 - 3, P2)
    L = dst.logp_num_tiles(P2)
    partials = torch.empty((n, L, 3), device=DEV)
    dst.logp_partials(x2, y, P2 - 3, P2, 0, P2, partials)
    lp2, ls2, st2 = dst.logp_merge(partials, y, P2 - 3)
    torch.cuda.synchronize()
    check_forward(x2.cpu(), yh, P2 - 3, None, -100, lp2.cpu().numpy(), ls2.cpu().numpy(),
                  st2.cpu().numpy(), "one tile more")


def test_row_of_two_to_the_thirty_columns():
    """One row of 2^30 + 776 columns (2 GiB of BF16): 64-bit offsets, 31-bit column arithmetic,
    262145 tiles merged by logp_merge, and the flat backward over 2^27 + 97 vectors."""
    P = (1 << 30) + 776
    V = P - 100
    say(f"one row of {P} columns")
    x = gaussian_bf16(1, P, seed=7)
    y = torch.tensor([V - 1], device=DEV)
    g = torch.tensor([0.5], device=DEV)
    L = dst.logp_num_tiles(P)
    partials = torch.empty((1, L, 3), device=DEV)
    dst.logp_partials(x, y, V, P, 0, P, partials)
    logp, lse, stats = dst.logp_merge(partials, y, V)
    d = dst.logp_backward(x, y, g, stats, V, P)
    torch.cuda.synchronize()
    host = x.cpu()
    yh, gh = y.cpu().numpy(), g.cpu().numpy()
    ref = oracle.forward(host, yh, V)
    fwd = {"logp_err": abs(float(logp[0]) - ref["logp"][0]),
           "lse_err": abs(float(lse[0]) - ref["lse"][0])}
    assert fwd["logp_err"] <= 1e-4 and fwd["lse_err"] <= 1e-4, fwd
    assert float(stats[0, 0]) == ref["max"][0]
    assert abs(float(stats[0, 1]) - ref["sumexp"][0]) <= 2e-5 * ref["sumexp"][0]
    gen = np.random.default_rng(0)
    cols = np.unique(np.concatenate([gen.integers(0, P, 200_000), [0, V - 2, V - 1, V, P - 1],
                                     np.arange(V - 64, P)]))
    want = oracle.backward_elements(host[0], cols, int(yh[0]), float(gh[0]), ref["lse"][0], V)
    got_bits = d[0, torch.from_numpy(cols).to(DEV)].cpu().view(torch.int16).numpy()
    got = oracle.bf16_bits_to_f64(got_bits.view(np.uint16))
    rounded = oracle.bf16_bits_to_f64(oracle.rne_bf16(want))
    err = np.abs(got - want)
    allow = spacing(want, "bf16")
    allow[cols == yh[0]] += 2.0 ** -20 * abs(float(gh[0]))
    assert np.all(err <= allow), (np.argwhere(err > allow)[:5], err[err > allow][:5])
    assert np.all(got[cols >= V] == 0)
    frac = float(np.mean(got == rounded))
    assert frac >= 0.9999, frac
    say(f"2^30 row: {fwd}, sampled dlogits correctly rounded {frac:.6f} over {cols.size}")
