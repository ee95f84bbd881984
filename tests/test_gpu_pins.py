"""GPU-side pins that follow from the definition itself rather than from a stored value.

* Replication: one row copied V times with targets 0..V-1 gives every logp_y of that row;
  sum_y exp(logp_y) = 1 (issue #241 "[WS2] TP-aware deterministic logprob ...",
  Background: the logprob is the log-softmax taken at the target), and since nothing in the
  reduction depends on the row's position, every copy's LSE and (M, S) are the same bits.
* The BF16 gradient rows: the exact rows sum to 0 (softmax sums to 1), and rounding an
  element to nearest BF16 moves it by at most half a spacing, at most 2^-8 of its magnitude,
  so a rounded row sums to at most 2^-8 * sum |d| (PR #495 "zero-workspace backward for
  generic CUDA fused logp", Summary item 2: the gradient is written in the logits' dtype).
  With g = 1/3891 the target element alone, g (1 - p_y) at the bottom of its binade, can
  carry half of that bound.
* A valid row whose target logit is -inf while other logits are finite (PR #495 Tests:
  -inf masked vocab tails): logp = -inf, LSE finite, and p_y = 0 makes d_y = g exactly.
* Tensor parallelism at degree 8 over the 38 tiles of the Qwen vocabulary: tile-aligned
  shards of 5,5,5,5,5,5,4,4 tiles (PR #314 "[WS2][Logp] Deterministic config option",
  Tensor Parallel doc, steps 1-6) merge to the fused forward's bits, and each rank's
  backward slice from the merged stats is the whole-row backward's slice.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst
import oracle
from parity_checks import BackwardTally, bits_of, check_forward
from workloads import mid_case, random_case

pytestmark = pytest.mark.gpu
DEV = "cuda"
T = dst.TILE_COLS


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("v", [10007, 151936])
def test_replicated_row_softmax_sums_to_one(v):
    rng = np.random.default_rng(v)
    row = torch.from_numpy(rng.normal(0.0, 3.0, size=(1, v)).astype(np.float32))
    row = row.to(torch.bfloat16).to(DEV)
    say(f"replicated row: V={v}, {v} copies ({v * v * 2 / 2**30:.1f} GiB)")
    x = row.expand(v, v).contiguous()
    y = torch.arange(v, device=DEV)
    logp, lse, stats = dst.logp_forward(x, y)
    torch.cuda.synchronize()
    # every copy has the same LSE and (M, S) bits
    assert torch.equal(lse.view(torch.int32), lse[:1].expand(v).view(torch.int32))
    assert torch.equal(stats.view(torch.int64), stats[:1].expand(v, 2).contiguous()
                       .view(torch.int64))
    lp = logp.cpu().numpy().astype(np.float64)
    total = math.fsum(np.exp(lp))
    say(f"V={v}: sum exp(logp) - 1 = {total - 1.0:.3e}")
    assert abs(total - 1.0) <= 1e-5
    # the copies are rows of the oracle too: a sample of targets against it
    pick = np.unique(np.concatenate([rng.choice(v, 62, replace=False), [0, v - 1]]))
    host = row.cpu().expand(pick.size, v).contiguous()
    check_forward(host, pick, v, None, -100, lp[pick].astype(np.float32),
                  lse.cpu().numpy()[pick], stats.cpu().numpy()[pick], f"replicated V={v}")
    del x, logp, lse, stats
    torch.cuda.empty_cache()


def test_bf16_gradient_rows_sum_within_rounding():
    case = mid_case(device=DEV)
    say(f"mid config row sums: n={case.n} V={case.vocab_real} P={case.vocab_padded}")
    logp, lse, stats = dst.logp_forward(case.logits, case.targets, case.vocab_real,
                                        case.vocab_padded, active=case.active)
    d = dst.logp_backward(case.logits, case.targets, case.grad, stats, case.vocab_real,
                          case.vocab_padded, active=case.active)
    torch.cuda.synchronize()
    sums = torch.empty(case.n, dtype=torch.float64, device=DEV)
    abs_sums = torch.empty_like(sums)
    for r0 in range(0, case.n, 512):
        blk = d[r0:r0 + 512].double()
        sums[r0:r0 + 512] = blk.sum(1)
        abs_sums[r0:r0 + 512] = blk.abs().sum(1)
    valid = torch.from_numpy(
        np.asarray(case.active.cpu().numpy() != 0)).to(DEV)  # every target is in range
    ratio = (sums.abs() / abs_sums.clamp_min(1e-300))[valid]
    say(f"largest |row sum| / sum |d| = {float(ratio.max()):.3e} (bound 2^-8 = {2**-8:.3e})")
    assert torch.all(sums.abs()[valid] <= 2.0 ** -8 * abs_sums[valid])
    assert torch.all(abs_sums[~valid] == 0)


@pytest.mark.parametrize("width", [9001, 9008], ids=["tile_items", "flat"])
@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_valid_target_at_minus_inf(width, dt):
    """Rows with the target inside a -inf tail or a -inf run: logp -inf, LSE finite,
    d_y = g bit for bit, everything else against the oracle.  Width 9001 is not a multiple
    of 8, so the backward takes its (row, tile) kernel; 9008 takes the flat one."""
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
    n, v = 6, width
    gen = torch.Generator().manual_seed(width)
    x = torch.randn((n, v), generator=gen) * 3
    x[0, 5000:] = float("-inf")        # target inside the -inf tail
    x[1, 100:200] = float("-inf")      # target inside a -inf run, finite both sides
    x[2, :] = float("-inf")
    x[2, 4100] = 2.0                   # a single finite logit, not the target
    x[3, 8000:] = float("-inf")        # a -inf tail, target finite (control row)
    x[4, 4095] = float("-inf")         # an isolated -inf target at a tile's last column
    x[5, 7] = 30.0                     # dominant logit elsewhere, target a -inf column
    x[5, 4096:4100] = float("-inf")
    y = torch.tensor([5001, 150, 3, 17, 4095, 4097])
    g = torch.tensor([0.5, -2.0, 1.0, 0.25, -0.75, 3.0])  # exact in every output dtype
    logits = x.to(tdt).to(DEV)
    yd, gd = y.to(DEV), g.to(DEV)
    say(f"valid targets at -inf: n={n} V={v} {dt}")
    logp, lse, stats = dst.logp_forward_ex(logits, yd)
    d = dst.logp_backward_ex(logits, yd, gd, stats)
    torch.cuda.synchronize()
    inf_rows = [0, 1, 2, 4, 5]
    assert torch.all(torch.isneginf(logp[inf_rows]))
    assert torch.all(torch.isfinite(lse)) and torch.isfinite(logp[3])
    dh = d.cpu()
    assert torch.all(torch.isfinite(dh.float()))
    for r in inf_rows:
        assert dh[r, y[r]].item() == g[r].item(), (r, dh[r, y[r]].item(), g[r].item())
    host = logits.cpu()
    check_forward(host, y.numpy(), v, None, -100, logp.cpu().numpy(), lse.cpu().numpy(),
                  stats.cpu().numpy(), f"targets at -inf, {dt}")
    tally = BackwardTally()
    gpu_vals = bits_of(d) if dt == "bf16" else d.cpu().numpy()
    tally.add_block(host, y.numpy(), g.numpy(), v, v, None, -100, gpu_vals,
                    f"targets at -inf, {dt}", ulps=16.0 if dt == "f32" else 1.0)
    tally.finish(f"targets at -inf, {dt}")


def tp_bounds(num_tiles: int, ranks: int, vocab_padded: int) -> list[tuple[int, int]]:
    """Tile-aligned shard bounds: the first num_tiles % ranks ranks take one tile more."""
    base, extra = divmod(num_tiles, ranks)
    out, t0 = [], 0
    for r in range(ranks):
        t1 = t0 + base + (1 if r < extra else 0)
        out.append((t0 * T, min(t1 * T, vocab_padded)))
        t0 = t1
    return out


@pytest.mark.parametrize("padded", [151936, 152064])
def test_tensor_parallel_degree_8_layout(padded):
    n, v = 2048, 151936
    case = random_case(n, v, padded, sigma=3.0, seed=8, inactive_frac=0.05,
                       ignore_frac=0.05, device=DEV)
    L = dst.logp_num_tiles(padded)
    bounds = tp_bounds(L, 8, padded)
    assert L == 38 and [(c1 - c0 + T - 1) // T for c0, c1 in bounds] == [5] * 6 + [4] * 2
    say(f"TP=8 layout over {L} tiles: n={n} P={padded}")
    x = case.logits
    ref = dst.logp_forward(x, case.targets, v, padded, active=case.active)
    partials = torch.empty((n, L, 3), dtype=torch.float32, device=DEV)
    for c0, c1 in bounds:
        dst.logp_partials(x[:, c0:c1], case.targets, v, padded, c0, c1, partials,
                          active=case.active)
    got = dst.logp_merge(partials, case.targets, v, active=case.active)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    # each rank's backward slice from the merged (replicated) stats
    whole = dst.logp_backward(x, case.targets, case.grad, got[2], v, padded,
                              active=case.active)
    for c0, c1 in bounds:
        part = dst.logp_backward(x[:, c0:c1], case.targets, case.grad, got[2], v, padded,
                                 col_begin=c0, col_end=c1, active=case.active)
        torch.cuda.synchronize()
        assert torch.equal(part.view(torch.int16), whole[:, c0:c1].view(torch.int16)), (c0, c1)
    # and the fused forward against the oracle on these rows
    check_forward(x.cpu(), case.targets.cpu().numpy(), v, case.active.cpu().numpy(), -100,
                  ref[0].cpu().numpy(), ref[1].cpu().numpy(), ref[2].cpu().numpy(), "TP=8")
