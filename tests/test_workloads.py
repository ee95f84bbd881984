"""Input generators: determinism and the shape of each recipe (CPU only)."""

import os

import numpy as np
import torch

from workloads import SWEEP_SIZES, case_digest, random_case, sweep_positions, tiny_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_tiny_case_digest_is_pinned():
    want = open(os.path.join(GOLDEN, "tiny_case.sha256")).read().split()[0]
    assert case_digest(tiny_case()) == want
    assert case_digest(tiny_case()) == case_digest(tiny_case())


def test_tiny_case_structure():
    c = tiny_case()
    assert c.logits.shape == (64, 1024) and c.logits.dtype == torch.bfloat16
    y = c.targets.numpy()
    assert (y == -100).sum() == 8 and np.all((y == -100) | ((y >= 0) & (y < 1024)))
    r_eq, r_sp = c.meta["equal_row"], c.meta["spike_row"]
    assert y[r_eq] >= 0 and y[r_sp] >= 0
    assert torch.all(c.logits[r_eq] == c.logits[r_eq, 0])
    x = c.logits[r_sp].float()
    assert int(torch.argmax(x)) == c.meta["spike_col"] and float(x.max()) > 25.0
    assert c.grad.dtype == torch.float32


def test_sweep_protocol_reproduces_2232_comparisons():
    spec = dict(line.split() for line in open(os.path.join(GOLDEN, "sweep_counts.txt"))
                if line.strip() and not line.startswith("#"))
    assert len(SWEEP_SIZES) == int(spec["sizes"]) and max(SWEEP_SIZES) == 2048
    per = sum(len(sweep_positions(b)) for b in SWEEP_SIZES)
    assert per == int(spec["comparisons_per_probe_and_seed"])
    assert per * int(spec["probes"]) * int(spec["seeds"]) == int(spec["comparisons"])
    assert sweep_positions(1) == [0] and sweep_positions(2) == [0, 1]
    assert sweep_positions(5) == [0, 2, 4]


def test_random_case_targets_and_padding():
    c = random_case(40, 300, 320, ld=330, seed=4, pad_fill=100.0, inactive_frac=0.25,
                    ignore_frac=0.1, bad_target_frac=0.2)
    assert c.logits.shape == (40, 330) and c.ld == 330
    assert torch.all(c.logits[:, 300:].float() == 100.0)
    y = c.targets
    assert ((y == -100).sum() > 0) and ((y >= 300).sum() > 0)
    assert c.active is not None and c.active.dtype == torch.uint8
    again = random_case(40, 300, 320, ld=330, seed=4, pad_fill=100.0, inactive_frac=0.25,
                        ignore_frac=0.1, bad_target_frac=0.2)
    assert case_digest(c) == case_digest(again)
