"""Pins for the FP64 oracle, independent of the oracle's own code.

Each test checks the oracle against something the pages or the mathematics fix:
closed forms, invariants, a 50-digit ``decimal`` brute force, special cases that
reduce to a library routine (torch float64 log_softmax and autograd, torch's
float32->bfloat16 rounding), and exact bit patterns.  Together they are chosen so
that a plausible slip in the oracle (a dropped term, a wrong sign, an off-by-one
index, a transposed operand, summing padded columns, double rounding) fails at
least one of them; ``test_planted_mistakes_are_caught`` checks exactly that by
compiling altered copies of the oracle.

What the pages fix (cited by title and section):
  * logp_t = x[t, y_t] - logsumexp_v x[t, v]  (issue #241, Background)
  * dlogits = g (onehot - softmax)  (PR #495, Summary item 2; its Benchmark script)
  * targets outside [0, V), e.g. -100, V, V+5, give logp 0 and an exactly zero
    gradient row  (PR #495, Behavior changes and Tests)
  * padded columns are masked before the local (max, sumexp)  (PR #314 commit notes)
  * tile partials merge as M = max m_l, S = sum s_l exp(m_l - M), LSE = M + log S,
    the target logit copied from its owner, inactive rows 0  (issue #241 PR 3;
    PR #314 Tensor Parallel doc steps 1-6); (-inf, 0) is the identity partial
    (PR #314 commit notes)
"""

from __future__ import annotations

import itertools
import math
import os
import shutil
import subprocess
import tempfile
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
from oracle import bf16_bits_to_f64
from workloads import random_case

NEG_INF = float("-inf")


def bf16_bits(values) -> np.ndarray:
    """BF16 bit patterns of values that are exactly representable in BF16."""
    t = torch.tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)
    back = t.float().numpy()
    assert np.array_equal(back, np.asarray(values, dtype=np.float32)) or \
        np.all(np.isnan(back) == np.isnan(np.asarray(values, dtype=np.float32)))
    return t.view(torch.int16).numpy().view(np.uint16)


def rows_bits(rows) -> np.ndarray:
    return np.stack([bf16_bits(r) for r in rows])


# ------------------------------------------------------------------ BF16 rounding

def test_rne_bf16_exact_bit_patterns():
    # a list, not a dict: 0.0 and -0.0 compare equal as keys
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3F80), (-2.0, 0xC000), (0.5, 0x3F00),
        (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
        # halfway between 1 and 1+2^-7: ties to the even significand (1)
        (1.0 + 2.0 ** -8, 0x3F80),
        # halfway between 1+2^-7 (odd) and 1+2^-6: ties up to even
        (1.0 + 3 * 2.0 ** -8, 0x3F82),
        # just above the halfway point: rounds up; a float32 step first would tie to even
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),
        # just below halfway: rounds down
        (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),
        # largest finite BF16 and the overflow threshold (ties to even -> inf)
        ((2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),
        ((2.0 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),
        ((2.0 - 2.0 ** -8 - 2.0 ** -20) * 2.0 ** 127, 0x7F7F),
        # subnormals: spacing 2^-133
        (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (1.5 * 2.0 ** -134, 0x0001),
        (3 * 2.0 ** -134, 0x0002), (2.0 ** -126, 0x0080), (-(2.0 ** -127), 0x8040),
        # 2^-126 - 2^-134 is halfway between the largest subnormal (odd) and 2^-126
        (2.0 ** -126 - 2.0 ** -134, 0x0080),
    ]
    got = oracle.rne_bf16([v for v, _ in cases])
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))
    assert (int(oracle.rne_bf16([float("nan")])[0]) & 0x7FFF) > 0x7F80


def test_rne_bf16_matches_torch_on_float32_values():
    # Every float32 is exactly a double, and torch rounds float32 -> bfloat16 to nearest
    # even, so on these inputs both must give identical bits (normals, subnormals, huge).
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    extra = np.array([1e-45, -1e-45, 1.1754942e-38, 3.389e38, 3.3895314e38, 3.4e38],
                     dtype=np.float32)
    f = np.concatenate([f, extra])
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.rne_bf16(f.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(f[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


# ------------------------------------------------------------------ forward: closed forms

@pytest.mark.parametrize("vocab", [1, 2, 3, 1024, 4097, 151936])
def test_uniform_row_gives_minus_log_v_exactly(vocab):
    c = -1.25
    x = np.full((3, vocab), bf16_bits([c])[0], dtype=np.uint16)
    y = np.array([0, vocab - 1, vocab // 2])
    out = oracle.forward(x, y, vocab)
    assert np.all(out["logp"] == -math.log(vocab))
    assert np.all(out["lse"] == c + math.log(vocab))
    assert np.all(out["max"] == c) and np.all(out["sumexp"] == vocab)


def test_single_column_vocab():
    x = rows_bits([[3.5], [-7.0]])
    y = np.array([0, 0])
    out = oracle.forward(x, y, 1)
    assert np.all(out["logp"] == 0.0)
    d = oracle.backward(x, y, np.array([2.0, -1.5], np.float32), 1)
    # g * (1 - 1) is a signed zero; values are compared, so -0 and +0 are equal
    assert np.all(d["d64"] == 0.0) and np.all((d["bf16"] & 0x7FFF) == 0)


def test_two_column_vocab_log1p_form():
    vals = [-3.5, -1.0, 0.0, 0.5, 2.0, 7.0]
    pairs = [(a, b) for a in vals for b in vals]
    x = rows_bits(pairs)
    for y in (0, 1):
        out = oracle.forward(x, np.full(len(pairs), y), 2)
        for i, (a, b) in enumerate(pairs):
            xy, xo = (a, b) if y == 0 else (b, a)
            want = -math.log1p(math.exp(xo - xy))
            # log(S) with S = 1 + e^(xo - xy) carries up to ~1 ulp of 1 in absolute terms
            assert out["logp"][i] == pytest.approx(want, rel=1e-15, abs=5e-16)


@pytest.mark.parametrize("vocab,spike", [(1024, 40.0), (151936, 30.0), (7, 3.0)])
def test_spike_row_closed_form(vocab, spike):
    row = np.zeros(vocab, dtype=np.float32)
    s_col = vocab // 3
    row[s_col] = spike
    x = rows_bits([row, row])
    other = (s_col + 1) % vocab
    out = oracle.forward(x, np.array([s_col, other]), vocab)
    tail = math.log1p((vocab - 1) * math.exp(-spike))
    # The oracle sums in column order in FP64; after the spike every addend is far below
    # one ulp of the running sum, so its error is bounded by vocab * 2^-53 (absolute).
    tol = vocab * 2.0 ** -52
    assert out["lse"][0] == pytest.approx(spike + tail, rel=0, abs=tol + 1e-14)
    assert out["logp"][0] == pytest.approx(-tail, rel=0, abs=tol)
    assert out["logp"][1] == pytest.approx(-spike - tail, rel=0, abs=tol + 1e-14)


def test_softmax_of_all_targets_sums_to_one():
    case = random_case(1, 1000, sigma=3.0, seed=11)
    v = case.vocab_real
    x = np.repeat(oracle._bits(case.logits), v, axis=0)
    out = oracle.forward(x, np.arange(v), v)
    assert abs(math.fsum(np.exp(out["logp"])) - 1.0) <= 1e-12
    assert np.all(out["lse"] == out["lse"][0])


def _dec(x: float) -> Decimal:
    return Decimal(x)


def _brute_row(vals, y, g):
    """50-digit brute force of logp, LSE and dlogits for one tiny row."""
    getcontext().prec = 50
    finite = [_dec(v) for v in vals if v != NEG_INF]
    if not finite:
        return None
    Z = sum((v.exp() for v in finite), Decimal(0))
    lse = Z.ln()
    logp = None if vals[y] == NEG_INF else _dec(vals[y]) - lse
    d = []
    for c, v in enumerate(vals):
        p = Decimal(0) if v == NEG_INF else (_dec(v) - lse).exp()
        d.append(_dec(g) * ((Decimal(1) if c == y else Decimal(0)) - p))
    return lse, logp, d


def test_decimal_brute_force_tiny_rows():
    alphabet = [NEG_INF, -3.5, -1.0, 0.0, 0.5, 2.0, 40.0]
    rows = []
    for vocab in (1, 2, 3):
        rows += [list(r) for r in itertools.product(alphabet, repeat=vocab)]
    rng = np.random.default_rng(3)
    rows += [list(rng.choice(alphabet, 4)) for _ in range(60)]
    g = np.float32(-0.8125)
    checked = 0
    for vals in rows:
        vocab = len(vals)
        x = rows_bits([vals])
        for y in range(vocab):
            ref = _brute_row(vals, y, float(g))
            out = oracle.forward(x, np.array([y]), vocab)
            d = oracle.backward(x, np.array([y]), np.array([g]), vocab)["d64"][0]
            if ref is None:  # every logit is -inf
                assert out["lse"][0] == NEG_INF and out["logp"][0] == NEG_INF
                assert np.all(d == 0.0)
                continue
            lse, logp, dref = ref
            assert out["lse"][0] == pytest.approx(float(lse), rel=1e-15, abs=1e-15)
            if logp is None:
                assert out["logp"][0] == NEG_INF
            else:
                assert out["logp"][0] == pytest.approx(float(logp), rel=1e-14, abs=1e-15)
            for c in range(vocab):
                assert d[c] == pytest.approx(float(dref[c]), rel=1e-14, abs=1e-15), (vals, y, c)
            checked += 1
    assert checked > 1000


def test_matches_torch_float64_log_softmax_and_autograd():
    for seed, (n, v, pad) in enumerate([(16, 1031, 0), (9, 255, 9), (5, 4097, 3000)]):
        case = random_case(n, v, v + pad, sigma=3.0, seed=seed, pad_fill=100.0)
        x64 = case.logits[:, :v].double().requires_grad_(True)
        lsm = torch.log_softmax(x64, dim=1)
        want_logp = lsm.gather(1, case.targets.view(-1, 1)).flatten()
        (want_logp * case.grad.double()).sum().backward()
        out = oracle.forward(case.logits, case.targets, v)
        assert np.allclose(out["logp"], want_logp.detach().numpy(), rtol=1e-13, atol=1e-13)
        assert np.allclose(out["lse"], torch.logsumexp(x64, 1).detach().numpy(), rtol=1e-14)
        d = oracle.backward(case.logits, case.targets, case.grad, v, v + pad)
        assert np.allclose(d["d64"][:, :v], x64.grad.numpy(), rtol=1e-12, atol=1e-15)
        assert np.all(d["d64"][:, v:] == 0.0)
        assert np.array_equal(d["bf16"], oracle.rne_bf16(d["d64"]))


# ------------------------------------------------------------------ invalid rows, masking

def test_invalid_rows_are_zero_and_others_unchanged():
    case = random_case(12, 300, 320, sigma=3.0, seed=5, pad_fill=100.0)
    v, p = case.vocab_real, case.vocab_padded
    base_y = case.targets.clone()
    base = oracle.forward(case.logits, base_y, v)
    base_d = oracle.backward(case.logits, base_y, case.grad, v, p)["d64"]
    y = base_y.clone()
    bad = {1: -100, 3: v, 4: v + 5, 6: -7, 8: p - 1}  # ignore index, out of range, padded
    for r, t in bad.items():
        y[r] = t
    active = np.ones(12, np.uint8)
    active[10] = 0
    out = oracle.forward(case.logits, y, v, active=active)
    d = oracle.backward(case.logits, y, case.grad, v, p, active=active)["d64"]
    invalid = sorted(list(bad) + [10])
    for r in range(12):
        if r in invalid:
            assert out["logp"][r] == 0.0 and np.all(d[r] == 0.0)
            assert out["lse"][r] == base["lse"][r]  # the LSE depends only on the logits
        else:
            assert out["logp"][r] == base["logp"][r]
            assert np.array_equal(d[r], base_d[r])
    # a non-negative ignore index also marks a row invalid
    out2 = oracle.forward(case.logits, base_y, v, ignore_index=int(base_y[0]))
    assert out2["logp"][0] == 0.0


def test_padding_columns_are_masked_by_index():
    case = random_case(6, 500, 640, sigma=3.0, seed=9, pad_fill=100.0)
    trimmed = case.logits[:, :500].contiguous()
    a = oracle.forward(case.logits, case.targets, 500)
    b = oracle.forward(trimmed, case.targets, 500)
    for k in ("logp", "lse", "max", "sumexp"):
        assert np.array_equal(a[k], b[k])
    da = oracle.backward(case.logits, case.targets, case.grad, 500, 640)
    db = oracle.backward(trimmed, case.targets, case.grad, 500, 500)
    assert np.array_equal(da["d64"][:, :500], db["d64"]) and np.all(da["d64"][:, 500:] == 0)


def test_all_minus_inf_rows():
    x = rows_bits([[NEG_INF] * 5, [NEG_INF] * 5])
    y = np.array([2, -100])
    out = oracle.forward(x, y, 5)
    assert out["lse"][0] == NEG_INF and out["logp"][0] == NEG_INF and out["logp"][1] == 0.0
    assert out["sumexp"][0] == 0.0
    d = oracle.backward(x, y, np.array([1.0, 1.0], np.float32), 5)
    assert np.all(d["d64"] == 0.0)


def test_minus_inf_masked_tail_gives_finite_zero_gradient():
    row = [0.5, -1.0, 2.0, NEG_INF, NEG_INF, NEG_INF]
    x = rows_bits([row])
    d = oracle.backward(x, np.array([1]), np.array([3.0], np.float32), 6)["d64"][0]
    assert np.all(np.isfinite(d)) and np.all(d[3:] == 0.0)


# ------------------------------------------------------------------ gradient invariants

def test_gradient_rows_sum_to_zero_and_uniform_closed_form():
    case = random_case(20, 3000, sigma=3.0, seed=21, grad_std=5.0)
    d = oracle.backward(case.logits, case.targets, case.grad, 3000)["d64"]
    g = case.grad.numpy().astype(np.float64)
    for r in range(20):
        assert abs(math.fsum(d[r])) <= 1e-12 * abs(g[r])
    v = 257
    x = np.full((2, v), bf16_bits([0.75])[0], dtype=np.uint16)
    gg = np.array([1.5, -0.25], np.float32)
    d = oracle.backward(x, np.array([3, 200]), gg, v)["d64"]
    for r, y in enumerate((3, 200)):
        want = np.full(v, -float(gg[r]) / v)
        want[y] = float(gg[r]) * (1.0 - 1.0 / v)
        assert np.allclose(d[r], want, rtol=2e-16, atol=0)


def test_gradient_entries_match_exp_of_logp():
    # d[c] for c != y equals -g * exp(logp_c) where logp_c is the forward for target c.
    case = random_case(1, 700, sigma=3.0, seed=31)
    x = oracle._bits(case.logits)
    y = int(case.targets[0])
    g = np.float32(0.375)
    d = oracle.backward(x, np.array([y]), np.array([g]), 700)["d64"][0]
    all_logp = oracle.forward(np.repeat(x, 700, axis=0), np.arange(700), 700)["logp"]
    want = -float(g) * np.exp(all_logp)
    want[y] += float(g)
    assert np.allclose(d, want, rtol=1e-13, atol=1e-18)


# ------------------------------------------------------------------ partials and merge

@pytest.mark.parametrize("tile", [4096, 64, 7])
def test_merge_of_tile_partials_equals_direct_lse(tile):
    case = random_case(10, 10000, 10000 + 3 * tile, sigma=3.0, seed=41, pad_fill=100.0,
                       inactive_frac=0.2, ignore_frac=0.1)
    v, p = case.vocab_real, case.vocab_padded
    part = oracle.tile_partials(case.logits, case.targets, v, p, active=case.active, tile=tile)
    L = oracle.num_tiles(p, tile)
    assert part["max"].shape == (10, L)
    merged = oracle.merge(part["max"], part["sumexp"], part["sel"], case.targets, v,
                          active=case.active, tile=tile)
    direct = oracle.forward(case.logits, case.targets, v, active=case.active)
    assert np.allclose(merged["lse"], direct["lse"], rtol=1e-13, atol=0)
    assert np.allclose(merged["logp"], direct["logp"], rtol=0, atol=1e-13)
    assert np.array_equal(merged["logp"] == 0.0, direct["logp"] == 0.0)
    xs = bf16_bits_to_f64(oracle._bits(case.logits))
    for r in range(10):
        for l in range(L):
            lo, hi = l * tile, min((l + 1) * tile, v)
            if lo >= v:  # all-padding tile: the (-inf, 0) identity
                assert part["max"][r, l] == NEG_INF and part["sumexp"][r, l] == 0.0
            else:
                assert part["max"][r, l] == xs[r, lo:hi].max()
                assert part["sumexp"][r, l] == pytest.approx(
                    np.exp(xs[r, lo:hi] - xs[r, lo:hi].max()).sum(), rel=1e-13)


def test_merge_identity_partials_change_nothing():
    case = random_case(8, 9000, sigma=3.0, seed=43)
    part = oracle.tile_partials(case.logits, case.targets, 9000)
    m, s, sel = part["max"], part["sumexp"], part["sel"]
    a = oracle.merge(m, s, sel, case.targets, 9000)
    pad = lambda a_, v_: np.concatenate([a_, np.full((8, 2), v_)], axis=1)  # noqa: E731
    b = oracle.merge(pad(m, NEG_INF), pad(s, 0.0), pad(sel, 0.0), case.targets, 9000)
    assert np.array_equal(a["logp"], b["logp"]) and np.array_equal(a["lse"], b["lse"])
    # all-identity rows give (LSE, logp) = (-inf, -inf) for a valid target
    ident = oracle.merge(np.full((1, 3), NEG_INF), np.zeros((1, 3)), np.zeros((1, 3)),
                         np.array([5]), 9000)
    assert ident["lse"][0] == NEG_INF and ident["logp"][0] == NEG_INF


def test_selected_logit_is_copied_from_its_owner_tile():
    case = random_case(30, 9000, sigma=3.0, seed=45, ignore_frac=0.2)
    part = oracle.tile_partials(case.logits, case.targets, 9000)
    xs = bf16_bits_to_f64(oracle._bits(case.logits))
    for r in range(30):
        y = int(case.targets[r])
        for l in range(part["sel"].shape[1]):
            want = xs[r, y] if (0 <= y < 9000 and y // 4096 == l) else 0.0
            assert part["sel"][r, l] == want


def test_count_bad_targets():
    y = np.array([0, 5, -100, -1, 10, 11, 3, 10**9])
    act = np.array([1, 1, 1, 1, 1, 0, 1, 1], np.uint8)
    assert oracle.count_bad_targets(y, 10, active=act) == 3      # -1, 10, 1e9
    assert oracle.count_bad_targets(y, 10) == 4                  # + row 5 (11)
    assert oracle.count_bad_targets(y, 10, ignore_index=-1) == 4  # -100 now bad, -1 not


# ------------------------------------------------------------------ FP16 / FP32 logits

def test_rne_f16_exact_bit_patterns():
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF),
        (65519.99, 0x7BFF), (65520.0, 0x7C00), (1e6, 0x7C00), (float("inf"), 0x7C00),
        (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (1.5 * 2.0 ** -25, 0x0001),
        (2.0 ** -14, 0x0400), (2.0 ** -14 - 2.0 ** -25, 0x0400),
        (1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02),
        # above the tie by far less than a float32 ulp: a float32 step would tie to even
        (1.0 + 2.0 ** -11 + 2.0 ** -40, 0x3C01),
    ]
    got = oracle.rne_f16([v for v, _ in cases])
    for (v, want), g in zip(cases, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))


def test_rne_f16_matches_numpy():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100_000) * 10.0 ** rng.integers(-9, 5, 100_000),
                        rng.uniform(-70000, 70000, 2000)])
    with np.errstate(over="ignore"):  # values past 65520 round to inf on purpose
        want = x.astype(np.float16).view(np.uint16)  # numpy rounds double -> half directly
    got = oracle.rne_f16(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(x[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_f16_decode_is_exact_for_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    vals = bits.view(np.float16)
    keep = np.isfinite(vals)
    x = vals[keep].reshape(-1, 1)  # one value per row: the single-column tile max is x
    part = oracle.tile_partials(x, np.zeros(x.shape[0], np.int64), 1, tile=1)
    assert np.array_equal(part["max"][:, 0], x[:, 0].astype(np.float64))


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_f16_f32_logits_match_torch_float64(dtype):
    tdt = {"f16": torch.float16, "f32": torch.float32}[dtype]
    for seed, (n, v) in enumerate([(6, 1), (7, 255), (5, 1031), (2, 151936)]):
        gen = torch.Generator().manual_seed(seed)
        x = (torch.randn((n, v), generator=gen) * 3).to(tdt)
        y = torch.randint(0, v, (n,), generator=gen)
        g = torch.randn((n,), generator=gen)
        x64 = x.double().requires_grad_(True)
        lsm = torch.log_softmax(x64, 1)
        want = lsm.gather(1, y.view(-1, 1)).flatten()
        (want * g.double()).sum().backward()
        out = oracle.forward(x, y, v)
        assert np.allclose(out["logp"], want.detach().numpy(), rtol=1e-13, atol=1e-12)
        d = oracle.backward(x, y, g, v)
        assert np.allclose(d["d64"], x64.grad.numpy(), rtol=1e-12, atol=1e-15)
        npdt = np.float16 if dtype == "f16" else np.float32
        assert d["rounded"].dtype == npdt
        assert np.array_equal(d["rounded"], d["d64"].astype(npdt))  # numpy rounds to nearest


# ------------------------------------------------------------------ temperature

@pytest.mark.parametrize("inv_t", [1.0 / 0.7, 0.5, 3.0])
def test_temperature_scores_fl32_products(inv_t):
    it32 = np.float32(inv_t)
    vals = [-3.5, -1.0, 0.0, 0.5, 2.0, 7.0, 0.1015625, -2.71875]
    pairs = [(a, b) for a in vals for b in vals]
    x = rows_bits(pairs)
    z = bf16_bits_to_f64(x).astype(np.float32) * it32  # numpy float32 product: IEEE single
    out = oracle.forward(x, np.zeros(len(pairs), np.int64), 2, inv_temperature=inv_t)
    for i in range(len(pairs)):
        want = -math.log1p(math.exp(float(z[i, 1]) - float(z[i, 0])))
        assert out["logp"][i] == pytest.approx(want, rel=1e-15, abs=5e-16)
    # a uniform row stays exactly -log V at any temperature
    u = np.full((1, 300), bf16_bits([1.75])[0], dtype=np.uint16)
    assert oracle.forward(u, np.array([7]), 300, inv_temperature=inv_t)["logp"][0] == \
        -math.log(300)


def test_temperature_gradient_is_chain_rule_of_scored_logits():
    inv_t = np.float32(1.0 / 0.7)
    case = random_case(6, 777, sigma=3.0, seed=51, grad_std=2.0)
    z = (case.logits.float() * torch.tensor(inv_t)).double()  # fl32(x * inv_t), promoted
    zz = z.clone().requires_grad_(True)
    lsm = torch.log_softmax(zz, 1)
    sel = lsm.gather(1, case.targets.view(-1, 1)).flatten()
    (sel * case.grad.double()).sum().backward()
    out = oracle.forward(case.logits, case.targets, 777, inv_temperature=float(inv_t))
    assert np.allclose(out["logp"], sel.detach().numpy(), rtol=1e-13, atol=1e-12)
    d = oracle.backward(case.logits, case.targets, case.grad, 777, inv_temperature=float(inv_t))
    assert np.allclose(d["d64"], zz.grad.numpy() * float(inv_t), rtol=1e-12, atol=1e-15)
    # tile partials of the scored logits merge to the direct LSE
    part = oracle.tile_partials(case.logits, case.targets, 777, tile=100,
                                inv_temperature=float(inv_t))
    mg = oracle.merge(part["max"], part["sumexp"], part["sel"], case.targets, 777, tile=100)
    assert np.allclose(mg["lse"], out["lse"], rtol=1e-13)


# ------------------------------------------------------------------ planted mistakes

MUTATIONS = {
    "gradient sign": ("v = g * (onehot - softmax);", "v = g * (softmax - onehot);"),
    "dropped log S": ("- M) - log_s : 0.0;\n    }\n    if (c->logp)",
                      "- M) : 0.0;\n    }\n    if (c->logp)"),
    "padded columns summed": ("row_max_sumexp(&row, c->vocab_real, &M, &S);\n    int valid",
                              "row_max_sumexp(&row, c->ld, &M, &S);\n    int valid"),
    "target off by one": ("onehot = (col == y) ? 1.0 : 0.0;",
                          "onehot = (col == y + 1) ? 1.0 : 0.0;"),
    "no max shift in gradient": ("exp(row_x(&row, col) - M) / S;",
                                 "exp(row_x(&row, col)) / S;"),
    "f16 exponent bias": ("v = ldexp(1024.0 + m, e - 25);", "v = ldexp(1024.0 + m, e - 24);"),
    "temperature missing in gradient": ("double g = (double)c->grad[t] * (double)c->inv_t;",
                                        "double g = (double)c->grad[t];"),
    "f16 rounded through float32": ("double v = ldexp(nearbyint(ldexp(a, -q_exp)), q_exp);",
                                    "double v = ldexp(nearbyint(ldexp((double)(float)a, -q_exp)), q_exp);"),
    "temperature product in double": ("float z = x * inv_temperature;",
                                      "double z = (double)x * inv_temperature;"),
    "f16 subnormal scale": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "ignore index accepted": ("if (y == ignore_index) return 0;", ""),
    "round through float32": ("double q = ldexp(a, -q_exp);",
                              "double q = ldexp((double)(float)a, -q_exp);"),
    "merge without rescale": ("S += st[l] * exp(mt[l] - M);", "S += st[l];"),
    "selected tile transposed": ("sel[t * num_tiles + targets[t] / tile]",
                                 "sel[(targets[t] / tile) * n + t]"),
    "tile max over padding": ("if (hi > c->vocab_real) hi = c->vocab_real;", ""),
}


def _pins(lib) -> list[str]:
    """Run a compact subset of the pins above against an oracle build; return failures."""
    failed = []
    try:
        case = random_case(6, 600, 700, sigma=3.0, seed=1, pad_fill=100.0, ignore_frac=0.3)
        v, p = 600, 700
        x64 = case.logits[:, :v].double().requires_grad_(True)
        want = torch.log_softmax(x64, 1)
        y_ok = torch.where(case.targets >= 0, case.targets, 0)
        sel = want.gather(1, y_ok.view(-1, 1)).flatten()
        (sel * case.grad.double() * (case.targets >= 0)).sum().backward()
        out = oracle.forward(case.logits, case.targets, v, lib=lib)
        ok_rows = (case.targets >= 0).numpy()
        if not np.allclose(out["logp"][ok_rows], sel.detach().numpy()[ok_rows], atol=1e-12):
            failed.append("torch logp")
        if not np.all(out["logp"][~ok_rows] == 0):
            failed.append("invalid logp")
        d = oracle.backward(case.logits, case.targets, case.grad, v, p, lib=lib)
        if not np.allclose(d["d64"][:, :v], x64.grad.numpy(), atol=1e-14):
            failed.append("torch grad")
        if not np.all(d["d64"][:, v:] == 0):
            failed.append("padded grad")
        if np.any(oracle.rne_bf16([1.0 + 2.0 ** -8 + 2.0 ** -30], lib=lib) != 0x3F81):
            failed.append("rne")
        part = oracle.tile_partials(case.logits, case.targets, v, p, tile=64, lib=lib)
        mg = oracle.merge(part["max"], part["sumexp"], part["sel"], case.targets, v, tile=64,
                          lib=lib)
        if not (np.allclose(mg["lse"], out["lse"], rtol=1e-13)
                and np.allclose(mg["logp"], out["logp"], atol=1e-12)):
            failed.append("merge")
        x = np.full((1, 9), bf16_bits([0.75])[0], dtype=np.uint16)
        if oracle.forward(x, np.array([2]), 9, lib=lib)["logp"][0] != -math.log(9):
            failed.append("uniform")
        if oracle.forward(x, np.array([1]), 9, ignore_index=1, lib=lib)["logp"][0] != 0.0:
            failed.append("ignore index")
        # FP16: decode of every finite pattern and direct rounding
        h = np.arange(65536, dtype=np.uint16).view(np.float16)
        h = h[np.isfinite(h)].reshape(-1, 1)
        pm = oracle.tile_partials(h, np.zeros(h.shape[0], np.int64), 1, tile=1, lib=lib)["max"]
        if not np.array_equal(pm[:, 0], h[:, 0].astype(np.float64)):
            failed.append("f16 decode")
        if np.any(oracle.rne_f16([1.0 + 2.0 ** -11 + 2.0 ** -40, 2.0 ** -24, 65520.0],
                                 lib=lib) != [0x3C01, 0x0001, 0x7C00]):
            failed.append("f16 rne")
        # temperature: scored logits fl32(x * inv_t) and the chain-rule factor
        inv_t = np.float32(1.0 / 0.7)
        xt = case.logits[:, :v].float()
        z = (xt * torch.tensor(inv_t)).double().requires_grad_(True)
        lz = torch.log_softmax(z, 1).gather(1, y_ok.view(-1, 1)).flatten()
        (lz * case.grad.double() * (case.targets >= 0)).sum().backward()
        ot = oracle.forward(case.logits, case.targets, v, lib=lib, inv_temperature=float(inv_t))
        if not np.allclose(ot["logp"][ok_rows], lz.detach().numpy()[ok_rows], rtol=0,
                           atol=1e-13):
            failed.append("temperature logp")
        dt = oracle.backward(case.logits, case.targets, case.grad, v, p, lib=lib,
                             inv_temperature=float(inv_t))
        if not np.allclose(dt["d64"][:, :v], z.grad.numpy() * float(inv_t), atol=1e-14):
            failed.append("temperature grad")
    except Exception as e:  # a mutant may also crash; that counts as caught
        failed.append(f"exception {type(e).__name__}")
    return failed


def test_pins_pass_on_the_oracle():
    assert _pins(oracle._load()) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name):
    old, new = MUTATIONS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name!r} not unique"
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        path_c = os.path.join(tmp, "mutant.c")
        path_so = os.path.join(tmp, "libmutant.so")
        open(path_c, "w").write(src.replace(old, new))
        subprocess.run(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
                        "-pthread", "-ffp-contract=off", "-o", path_so, path_c, "-lm"],
                       check=True)
        lib = oracle.load_library(path_so)
        assert _pins(lib) != [], f"planted mistake {name!r} passed every pin"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_backward_elements_match_whole_row_backward():
    """The sampled-column form used for rows too wide to expand gives the same values as the
    whole-row backward (both evaluate g (onehot - softmax) in float64)."""
    g = torch.Generator().manual_seed(41)
    x = (torch.randn((3, 5000), generator=g) * 3).to(torch.bfloat16)
    y = np.array([17, 4999, -100])
    grad = np.array([0.75, -1.5, 2.0], dtype=np.float32)
    vr = 4990  # target 4999 lies in padding: invalid
    f = oracle.forward(x, y, vr)
    b = oracle.backward(x, y, grad, vr, 5000)
    cols = np.array([0, 17, 100, 4989, 4990, 4999])
    for r in range(3):
        valid = 0 <= y[r] < vr
        e = oracle.backward_elements(x[r], cols, int(y[r]), float(grad[r]), f["lse"][r], vr,
                                     valid=valid)
        np.testing.assert_allclose(e, b["d64"][r, cols], rtol=1e-13, atol=1e-300)
