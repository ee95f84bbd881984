"""The merge's fixed summation order, bitwise.

With every tile maximum at 0 the merge weights are the tile sums themselves
(s_l * exp(0 - 0) = s_l * 1 exactly), so the merged S must carry the exact bits of the order
the numerical contract fixes (issue #241 "PR 3" and PR #314's Tensor Parallel doc, step 4: a
fixed global order): lane i adds w_i, w_{i+64}, w_{i+128}, ... in float32 from +0, then the
64 lane sums combine pairwise, partners at lane xor 1, 2, 4, 8, 16, 32.  Identity tiles
(max -inf) add +0.  The expected bits come from a float32 emulation of that order on the CPU;
the inputs span several binades, so a different order (a plain left-to-right sum, or a tree
over other partners) gives different bits on most rows, which the test also checks.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst

DEV = "cuda"


def canonical_sum(w: np.ndarray) -> np.float32:
    """float32 emulation of the contract's order for one row of weights."""
    lanes = np.zeros(64, dtype=np.float32)
    for l, x in enumerate(w.astype(np.float32)):
        lanes[l % 64] = np.float32(lanes[l % 64] + x)
    o = 1
    while o < 64:
        lanes = (lanes + lanes[np.arange(64) ^ o]).astype(np.float32)
        o <<= 1
    assert np.all(lanes == lanes[0])
    return lanes[0]


def sequential_sum(w: np.ndarray) -> np.float32:
    acc = np.float32(0.0)
    for x in w.astype(np.float32):
        acc = np.float32(acc + x)
    return acc


def test_emulation_is_the_exact_sum_when_order_cannot_matter():
    # small integers: every partial sum is exact, so any order gives the plain sum
    w = np.arange(1, 301, dtype=np.float32)
    assert canonical_sum(w) == np.float32(w.sum())
    assert canonical_sum(np.zeros(5, np.float32)) == 0.0


@pytest.mark.gpu
@pytest.mark.parametrize("L", [1, 63, 64, 65, 200, 1000])
def test_merge_sum_follows_the_fixed_order(L):
    n = 32
    rng = np.random.default_rng(L)
    s = np.exp(rng.normal(0.0, 4.0, size=(n, L))).astype(np.float32)  # several binades
    m = np.zeros((n, L), dtype=np.float32)
    ident = rng.random((n, L)) < 0.1  # identity tiles: (-inf, 0)
    ident[:, 0] = False               # keep M = 0 on every row
    m[ident] = -np.inf
    s[ident] = 0.0
    part = np.stack([m, s, np.zeros_like(s)], axis=2)
    print(f"[gpu] merge order: n={n} L={L}", flush=True)
    partials = torch.from_numpy(part).to(DEV)
    y = torch.full((n,), -100, dtype=torch.int64, device=DEV)
    _, _, stats = dst.logp_merge(partials, y, vocab_real=L * 4096)
    torch.cuda.synchronize()
    got = stats[:, 1].cpu().numpy()
    assert np.all(stats[:, 0].cpu().numpy() == 0.0)
    want = np.array([canonical_sum(np.where(ident[r], 0.0, s[r])) for r in range(n)],
                    dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        np.argwhere(got != want)[:5]
    if L >= 64:
        # the order is visible: a left-to-right sum differs on most rows
        seq = np.array([sequential_sum(np.where(ident[r], 0.0, s[r])) for r in range(n)],
                       dtype=np.float32)
        assert np.mean(seq != want) > 0.5
