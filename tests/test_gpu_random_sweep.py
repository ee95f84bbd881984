"""Seeded random sweep over the shapes, dtypes and options of both GPU paths, each case against
the FP64 oracle and the bitwise contract.

Every case draws its configuration from its own seed (numpy PCG64): for the logp path the
logits dtype (BF16, FP16, FP32), rows, real and padded vocabulary (with a share of tile-edge
widths), the row stride, the temperature, the logit scale and the shares of ignored, bad and
inactive targets; for linear_logp the rows, hidden size, real and padded vocabulary,
temperature, logit scale and share of inactive rows.  Checks, with the tolerances of the dedicated tests (test_gpu_dtypes.py,
test_gpu_linear.py):
  - logp forward and backward against the oracle on every row (the correctly-rounded share
    of dlogits counted over the non-target entries: at V = 7 and scores of spread 20 a
    dominant target's g' (1 - p) cancels in FP32 in a sizeable share of the rows, and the
    per-element bound, with its 2^-20 |g'| term at the target, holds it instead);
  - a random tile-aligned shard layout of the partials merged back bitwise to the forward,
    and the backward of a random column range bitwise equal to that range of the full one;
  - linear_logp's forward against the oracle on every row, the balanced launch bitwise equal
    to the one-kernel launch, a random shard layout merged back bitwise, the backward's dh and
    dW against the oracle, and the kept-logits forward and backward bitwise equal to those;
  - the GRPO loss (random sequences, lengths, row strides, reductions, clip bounds, KL weight,
    ratio spread, masks with empty sequences, global normalizers) against its oracle.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst
from deterministic_selected_token_amd import linear
from deterministic_selected_token_amd import grpo
from test_gpu_dtypes import case_in, check_ex, same_bits
from test_gpu_grpo import check_against_oracle, make_batch
from test_gpu_linear import bwd_reference, bwd_run, check, check_bwd, make

pytestmark = pytest.mark.gpu
DEV = "cuda"
T = dst.TILE_COLS
EDGE_WIDTHS = [1, 7, T - 1, T, T + 1, 2 * T, 3 * T - 8, 5 * T + 3]
SMALL_SAMPLE = 20000  # dlogits entries below which 2 misrounded ones are allowed


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def random_layout(rng, tiles: int) -> list[int]:
    """Tiles per shard, summing to `tiles`, 1 to 4 shards."""
    k = int(rng.integers(1, min(4, tiles) + 1))
    cuts = sorted(rng.choice(np.arange(1, tiles), size=k - 1, replace=False).tolist()) \
        if k > 1 else []
    edges = [0] + cuts + [tiles]
    return [b - a for a, b in zip(edges, edges[1:])]


def logp_config(seed: int) -> dict:
    rng = np.random.default_rng(1000 + seed)
    dtype = ["bf16", "f16", "f32"][seed % 3]
    vr = int(rng.choice(EDGE_WIDTHS)) if rng.random() < 0.4 else int(rng.integers(1, 20000))
    vp = vr + (0 if rng.random() < 0.5 else int(rng.integers(1, 2 * T)))
    ld = vp + (0 if rng.random() < 0.5 else int(rng.integers(1, 64)))
    return dict(rng=rng, dtype=dtype, n=int(rng.integers(1, 97)), vr=vr, vp=vp, ld=ld,
                inv_t=float(rng.choice([1.0, 1 / 0.7, 2.0, 0.5])),
                sigma=float(rng.choice([1.0, 3.0, 10.0])),
                ignore=float(rng.choice([0.0, 0.1])), bad=float(rng.choice([0.0, 0.1])),
                inactive=float(rng.choice([0.0, 0.2])))


@pytest.mark.parametrize("seed", range(24))
def test_logp_random_case(seed):
    c = logp_config(seed)
    rng, dtype, n, vr, vp, ld, inv_t = (c[k] for k in ("rng", "dtype", "n", "vr", "vp", "ld",
                                                       "inv_t"))
    say(f"logp sweep seed={seed}: {dtype} n={n} V={vr}/{vp} ld={ld} inv_t={inv_t:.4g} "
        f"sigma={c['sigma']}")
    case = case_in(dtype, n, vr, vp, ld=ld, sigma=c["sigma"], seed=seed,
                   ignore_frac=c["ignore"], bad_target_frac=c["bad"],
                   inactive_frac=c["inactive"])
    ulps, min_cr = (16.0, 0.0) if dtype == "f32" else (1.0, None)
    if dtype != "f32" and n * vr < SMALL_SAMPLE:
        # the correctly-rounded bar is a population share: a sample this small may hold a
        # rare misrounded entry (per entry at most 2^-13 for BF16, 2^-10 for FP16, from the
        # ~4 FP32 units of the value rounded), so up to 2 are allowed; every entry is still
        # held to one spacing of its dtype
        bar = {"bf16": 0.9999, "f16": 1.0 - 2.0 ** -10}[dtype]
        min_cr = min(bar, 1.0 - 2.0 / (n * vr))
    (logp, lse, stats, d), fwd, bwd = check_ex(case, inv_t=inv_t, ulps=ulps, min_cr=min_cr,
                                               cr_skip_targets=True)
    say(f"seed={seed}: {fwd} {bwd}")

    # a random tile-aligned shard layout merges back to the forward's bits
    x = case.logits[:, :vp]
    L = dst.logp_num_tiles(vp)
    layout = random_layout(rng, L) if L > 1 else [1]
    partials = torch.full((n, L, 3), float("nan"), dtype=torch.float32, device=DEV)
    c0 = 0
    for tiles in layout:
        c1 = min(vp, c0 + tiles * T)
        dst.logp_partials_ex(x[:, c0:c1], case.targets, vr, vp, c0, c1, partials,
                             active=case.active, inv_temperature=inv_t)
        c0 = c1
    got = dst.logp_merge(partials, case.targets, vr, active=case.active)
    assert all(same_bits(u, w) for u, w in zip((logp, lse, stats), got)), layout

    # the backward of a random column range is that range of the full backward
    b0 = int(rng.integers(0, vp))
    b1 = int(rng.integers(b0 + 1, vp + 1))
    part = dst.logp_backward_ex(x[:, b0:b1], case.targets, case.grad, stats, vr, vp,
                                col_begin=b0, col_end=b1, active=case.active,
                                inv_temperature=inv_t)
    torch.cuda.synchronize()
    assert same_bits(part, d[:, b0:b1]), (b0, b1)


def linear_config(seed: int) -> dict:
    rng = np.random.default_rng(2000 + seed)
    V = int(rng.choice(EDGE_WIDTHS[1:])) if rng.random() < 0.3 else int(rng.integers(1, 12000))
    Vp = V + (0 if rng.random() < 0.5 else int(rng.integers(1, 2 * T)))
    return dict(rng=rng, n=int(rng.integers(1, 300)),
                H=int(8 * rng.integers(1, 80)), V=V, Vp=Vp,
                inv_t=float(rng.choice([1.0, 1 / 0.7, 2.0])),
                scale=float(rng.choice([0.5, 2.0, 10.0, 40.0])),
                inactive=float(rng.choice([0.0, 0.0, 0.3])))


@pytest.mark.parametrize("seed", range(16))
def test_linear_random_case(seed):
    c = linear_config(seed)
    rng, n, H, V, Vp, inv_t = (c[k] for k in ("rng", "n", "H", "V", "Vp", "inv_t"))
    say(f"linear sweep seed={seed}: n={n} H={H} V={V}/{Vp} inv_t={inv_t:.4g} "
        f"scale={c['scale']} inactive={c['inactive']}")
    h, W, y = make(n, H, V, Vp, seed=3000 + seed, scale=c["scale"], pad_value=float("nan"))
    active = None
    if c["inactive"] > 0:
        active = torch.from_numpy((rng.random(n) >= c["inactive"]).astype(np.uint8)).to(DEV)
    res, got = check(h, W, y, V, Vp, active=active, inv_t=inv_t)
    ref = linear.linear_logp_forward(h, W, y, V, Vp, active=active, inv_temperature=inv_t,
                                     balance=False)
    torch.cuda.synchronize()
    assert all(same_bits(u, w) for u, w in zip(got, ref))

    L = dst.logp_num_tiles(Vp)
    layout = random_layout(rng, L) if L > 1 else [1]
    partials = torch.full((n, L, 3), float("nan"), dtype=torch.float32, device=DEV)
    c0 = 0
    for tiles in layout:
        c1 = min(Vp, c0 + tiles * T)
        linear.linear_logp_partials(h, W[c0:c1], y, V, Vp, c0, c1, partials, active=active,
                                    inv_temperature=inv_t)
        c0 = c1
    merged = dst.logp_merge(partials, y, V, active=active)
    assert all(same_bits(u, w) for u, w in zip(got, merged)), layout

    g, stats, dh, dW, ws = bwd_run(h, W, y, V, Vp, active=active, inv_t=inv_t, chunk=T,
                                   seed=seed)
    bref = bwd_reference(h, W, y, g, V, active=active, inv_t=inv_t)
    bres = check_bwd(h, W, y, g, dh, dW, V, bref)
    if active is not None:
        assert torch.all(dh[active == 0] == 0)

    # kept logits: the same partials, and the backward from them the same bits
    # rows of the kept logits: a stride that is a multiple of 4 floats (16-byte aligned rows)
    z = torch.empty((n, (Vp + 3) // 4 * 4), dtype=torch.float32, device=DEV)[:, :Vp]
    Pz = torch.full((n, L, 3), float("nan"), dtype=torch.float32, device=DEV)
    linear.linear_logp_partials(h, W, y, V, Vp, 0, Vp, Pz, active=active, inv_temperature=inv_t,
                                logits=z)
    assert all(same_bits(u, w) for u, w in zip(got, dst.logp_merge(Pz, y, V, active=active)))
    dh2, dW2 = linear.linear_logp_backward(h, W, y, g, stats, V, Vp, active=active,
                                           inv_temperature=inv_t, chunk_cols=T, workspace=ws,
                                           logits=z)
    torch.cuda.synchronize()
    assert same_bits(dh, dh2) and same_bits(dW, dW2)
    say(f"seed={seed}: {res} {bres}")


def grpo_config(seed: int) -> dict:
    rng = np.random.default_rng(4000 + seed)
    n = int(rng.integers(1, 65))
    T_ = int(rng.choice([1, 255, 256, 257, 4096])) if rng.random() < 0.3 \
        else int(rng.integers(1, 5000))
    return dict(n=n, T=T_, ld=T_ + (0 if rng.random() < 0.5 else int(rng.integers(1, 40))),
                mode=list(grpo.MODES)[seed % 3], beta=float(rng.choice([0.0, 0.04, 0.3])),
                use_ref=bool(rng.random() < 0.7), use_mask=bool(rng.random() < 0.7),
                eps_low=float(rng.choice([0.1, 0.2])), eps_high=float(rng.choice([0.2, 0.28])),
                spread=float(rng.choice([0.05, 0.3, 2.0])),
                empty=tuple(int(r) for r in rng.choice(n, size=min(n, 2), replace=False))
                if rng.random() < 0.4 else (),
                norm_tokens=int(rng.choice([0, 0, 10000])), norm_seqs=int(rng.choice([0, 0, 96])))


@pytest.mark.parametrize("seed", range(18))
def test_grpo_random_case(seed):
    c = grpo_config(seed)
    say(f"grpo sweep seed={seed}: {c}")
    b = make_batch(c["n"], c["T"], seed=5000 + seed, spread=c["spread"], ld=c["ld"],
                   empty_rows=c["empty"] if c["use_mask"] else ())
    L, o = check_against_oracle(b, c["T"], c["mode"], c["beta"], eps_low=c["eps_low"],
                                eps_high=c["eps_high"], use_ref=c["use_ref"],
                                use_mask=c["use_mask"], norm_tokens=c["norm_tokens"],
                                norm_seqs=c["norm_seqs"])
    say(f"seed={seed}: loss {L['loss']:.6g} vs {o['loss']:.6g}")
