"""Bitwise determinism contract on the GPU (GPU against GPU, through the C ABI).

  * run to run; a row alone vs inside batches of every sweep size at front/middle/back
    (the 2232-comparison protocol of the fused-backward pull request, "Prior art &
    reuse decision" section);
  * permutation, chunking and active-row compaction of the batch (the provider
    experiment of the same pull request's author reply);
  * 1, 2 and 4 emulated vocab shards through partials + merge vs the fused forward, and
    padded vs unpadded vocabularies (issue #241 "PR 3"; PR #314 Tensor Parallel doc);
  * 16-byte vs 2-byte load paths; in-place backward; a non-default stream.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst
import oracle
from workloads import (SWEEP_SIZES, mid_case, random_case, shard_case, sweep_filler_rows,
                       sweep_positions, sweep_probe_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"
T = dst.TILE_COLS


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def fwd_bwd(x, y, g, vocab_real=None, vocab_padded=None, active=None):
    logp, lse, stats = dst.logp_forward(x, y, vocab_real, vocab_padded, active=active)
    d = dst.logp_backward(x, y, g, stats, vocab_real, vocab_padded, active=active)
    return logp, lse, stats, d


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    view = torch.int32 if a.element_size() == 4 else torch.int16
    return a.shape == b.shape and torch.equal(a.contiguous().view(view),
                                              b.contiguous().view(view))


def test_run_to_run():
    case = mid_case(device=DEV)
    say("run to run, mid config x3")
    a = fwd_bwd(case.logits, case.targets, case.grad, case.vocab_real, case.vocab_padded,
                case.active)
    for _ in range(2):
        b = fwd_bwd(case.logits, case.targets, case.grad, case.vocab_real, case.vocab_padded,
                    case.active)
        assert all(same_bits(u, w) for u, w in zip(a, b))


def test_vector_and_scalar_load_paths_agree():
    case = random_case(24, 10000, sigma=3.0, seed=17, device=DEV, ignore_frac=0.1)
    say("16-byte vs 2-byte paths")
    ref = fwd_bwd(case.logits, case.targets, case.grad)
    for ld, off in ((10003, 0), (10008, 1), (10016, 3)):
        buf = torch.zeros((24, ld), dtype=torch.bfloat16, device=DEV)
        buf[:, off:off + 10000] = case.logits
        x = buf[:, off:off + 10000]
        out_buf = torch.zeros((24, ld), dtype=torch.bfloat16, device=DEV)
        logp, lse, stats = dst.logp_forward(x, case.targets)
        d = dst.logp_backward(x, case.targets, case.grad, stats,
                              dlogits=out_buf[:, off:off + 10000])
        assert same_bits(logp, ref[0]) and same_bits(lse, ref[1]) and same_bits(stats, ref[2])
        assert same_bits(d, ref[3]), (ld, off)


def test_permutation_chunking_and_compaction():
    case = random_case(300, 20000, sigma=3.0, seed=23, device=DEV, inactive_frac=0.3)
    say("permutation / chunking / compaction")
    ref = fwd_bwd(case.logits, case.targets, case.grad, active=case.active)
    perm = torch.randperm(300, generator=torch.Generator().manual_seed(1)).to(DEV)
    p = fwd_bwd(case.logits[perm].contiguous(), case.targets[perm].contiguous(),
                case.grad[perm].contiguous(), active=case.active[perm].contiguous())
    for u, w in zip(ref, p):
        assert same_bits(u[perm], w)
    for chunk in (1, 7, 64):
        for r0 in range(0, 300, chunk):
            s = slice(r0, min(300, r0 + chunk))
            c = fwd_bwd(case.logits[s], case.targets[s], case.grad[s], active=case.active[s])
            for u, w in zip(ref, c):
                assert same_bits(u[s], w), chunk
    keep = torch.nonzero(case.active).flatten()
    c = fwd_bwd(case.logits[keep].contiguous(), case.targets[keep].contiguous(),
                case.grad[keep].contiguous())
    for u, w in zip(ref, c):
        assert same_bits(u[keep], w)


def test_in_place_backward_and_side_stream():
    case = random_case(10, 9000, sigma=3.0, seed=29, device=DEV)
    say("in-place backward, side stream")
    ref = fwd_bwd(case.logits, case.targets, case.grad)
    x = case.logits.clone()
    d = dst.logp_backward(x, case.targets, case.grad, ref[2], dlogits=x)
    assert d.data_ptr() == x.data_ptr() and same_bits(d, ref[3])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = fwd_bwd(case.logits, case.targets, case.grad)
    s.synchronize()
    assert all(same_bits(u, w) for u, w in zip(ref, out))


# ------------------------------------------------------------------ emulated vocab shards

SHARD_LAYOUTS = {1: [39], 2: [20, 19], 4: [13, 13, 12, 1]}  # tiles per shard, in order


def shard_merge(case, layout):
    n, P = case.n, case.vocab_padded
    L = dst.logp_num_tiles(P)
    partials = torch.full((n, L, 3), float("nan"), dtype=torch.float32, device=DEV)
    c0 = 0
    for tiles in layout:
        c1 = min(P, c0 + tiles * T)
        dst.logp_partials(case.logits[:, c0:c1], case.targets, case.vocab_real, P, c0, c1,
                          partials, active=case.active)
        c0 = c1
    assert c0 == P
    return partials, dst.logp_merge(partials, case.targets, case.vocab_real,
                                    active=case.active)


def test_shards_are_bitwise_equal_to_the_fused_forward():
    case = shard_case(device=DEV)
    say("shard config: fused forward")
    ref = dst.logp_forward(case.logits, case.targets, case.vocab_real, case.vocab_padded)
    for k, layout in SHARD_LAYOUTS.items():
        say(f"shard config: {k} shard(s) {layout}")
        partials, got = shard_merge(case, layout)
        assert all(same_bits(u, w) for u, w in zip(ref, got)), k
        if k == 4:  # the last shard is one all-padding tile: exactly (-inf, 0, 0)
            last = partials[:, 38].cpu()
            assert torch.all(last[:, 0] == float("-inf")) and torch.all(last[:, 1:] == 0)
    # padding invariance: the same real logits with vocab_padded = vocab_real
    unpadded = case.logits[:, :case.vocab_real].contiguous()
    say("shard config: unpadded buffer")
    got = dst.logp_forward(unpadded, case.targets, case.vocab_real, case.vocab_real)
    assert all(same_bits(u, w) for u, w in zip(ref, got))
    # the backward over each shard's slice reproduces the whole-row backward
    stats = ref[2]
    whole = dst.logp_backward(case.logits, case.targets, case.grad, stats, case.vocab_real,
                              case.vocab_padded)
    for c0, c1 in ((0, 20 * T), (20 * T, case.vocab_padded), (13 * T, 26 * T)):
        part = dst.logp_backward(case.logits[:, c0:c1], case.targets, case.grad, stats,
                                 case.vocab_real, case.vocab_padded, col_begin=c0, col_end=c1)
        assert same_bits(part, whole[:, c0:c1].contiguous()), (c0, c1)


def test_partials_against_oracle_tiles():
    case = random_case(12, 20000, 24576, sigma=3.0, seed=31, device=DEV, pad_fill=100.0,
                       ignore_frac=0.2, inactive_frac=0.2)
    say("partials vs oracle per-tile stats")
    L = dst.logp_num_tiles(case.vocab_padded)
    partials = torch.zeros((case.n, L, 3), dtype=torch.float32, device=DEV)
    dst.logp_partials(case.logits, case.targets, case.vocab_real, case.vocab_padded, 0,
                      case.vocab_padded, partials, active=case.active)
    got = partials.cpu().numpy().astype(np.float64)
    ref = oracle.tile_partials(case.logits.cpu(), case.targets.cpu(), case.vocab_real,
                               case.vocab_padded, active=case.active.cpu())
    assert np.array_equal(got[:, :, 0], ref["max"])         # max: exact
    assert np.array_equal(got[:, :, 2], ref["sel"])         # selected logit: exact copy
    fin = np.isfinite(ref["max"])
    rel = np.abs(got[:, :, 1][fin] - ref["sumexp"][fin]) / ref["sumexp"][fin]
    assert rel.max() <= 2e-6, rel.max()
    assert np.all(got[:, :, 1][~fin] == 0.0)


# ------------------------------------------------------------------ batch invariance sweep

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_batch_invariance_sweep(seed):
    probes = sweep_probe_rows(device=DEV, seed=seed)
    filler = sweep_filler_rows(device=DEV, seed=seed)
    say(f"sweep seed {seed}: 8 probes x {len(SWEEP_SIZES)} batch sizes")
    alone = [fwd_bwd(probes.logits[i:i + 1], probes.targets[i:i + 1], probes.grad[i:i + 1])
             for i in range(8)]
    comparisons = differing_logp = differing_dlogits = 0
    for B in SWEEP_SIZES:
        x = filler.logits[:B].clone()
        y = filler.targets[:B].clone()
        g = filler.grad[:B].clone()
        for pos in sweep_positions(B):
            for i in range(8):
                x[pos] = probes.logits[i]
                y[pos] = probes.targets[i]
                g[pos] = probes.grad[i]
                logp, lse, stats, d = fwd_bwd(x, y, g)
                a = alone[i]
                comparisons += 1
                differing_logp += not (same_bits(logp[pos:pos + 1], a[0])
                                       and same_bits(lse[pos:pos + 1], a[1])
                                       and same_bits(stats[pos:pos + 1], a[2]))
                differing_dlogits += not same_bits(d[pos:pos + 1], a[3])
            x[pos] = filler.logits[pos]
            y[pos] = filler.targets[pos]
            g[pos] = filler.grad[pos]
    say(f"sweep seed {seed}: {comparisons} comparisons, differing logp {differing_logp}, "
        f"dlogits {differing_dlogits}")
    assert comparisons == 744
    assert differing_logp == 0 and differing_dlogits == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("inv_t", [1.0, 1 / 0.7])
@pytest.mark.parametrize("V", [20480, 3001])  # the flat backward grid, the (row, tile) one
def test_backward_run_to_run_every_dtype_and_path(dtype, inv_t, V):
    """The backward twice into fresh (uninitialised) buffers, and once in place: the same bits
    for every logits dtype, with and without temperature, on both backward kernels -- the
    check that catches a store whose data registers are overwritten before it reads them."""
    n = 64
    g = torch.Generator(device=DEV).manual_seed(31)
    x = (torch.randn((n, V), generator=g, device=DEV) * 3).to(dtype)
    y = torch.randint(0, V, (n,), generator=g, device=DEV)
    y[::9] = -100
    gr = torch.randn(n, generator=g, device=DEV)
    say(f"backward run to run {dtype} inv_t={inv_t:.3g} V={V}")
    _, _, st = dst.logp_forward_ex(x, y, inv_temperature=inv_t)
    outs = [dst.logp_backward_ex(x, y, gr, st, inv_temperature=inv_t) for _ in range(2)]
    xi = x.clone()
    dst.logp_backward_ex(xi, y, gr, st, inv_temperature=inv_t, dlogits=xi)
    torch.cuda.synchronize()
    assert same_bits(outs[0], outs[1]) and same_bits(outs[0], xi)
