"""Pins of the FP64 GRPO-loss oracle (CPU only).

Each pin checks the oracle against something other than itself: hand-worked values of the
clipped objective, the KL=0 identity that issue #241's PR5 states as its acceptance test,
invariants of the reductions, a central finite difference of the loss, torch float64
autograd of an independently written loss, and torch's unbiased std.  Planted mistakes
(altered copies of the oracle source) must each fail at least one pin.
"""

from __future__ import annotations

import math
import os
import types

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "grpo_oracle.py")


def load_oracle(src: str = None):
    if src is None:
        src = open(ORACLE_SRC).read()
    mod = types.ModuleType("grpo_oracle_copy")
    exec(compile(src, ORACLE_SRC, "exec"), mod.__dict__)
    return mod


def f32(x):
    return np.asarray(x, dtype=np.float32)


def random_batch(rng, n_seqs=6, seq_len=50, spread=0.3, mask_frac=0.2):
    lp = f32(rng.normal(-2.0, 1.0, (n_seqs, seq_len)))
    old = f32(lp + rng.normal(0.0, spread, lp.shape))
    ref = f32(lp + rng.normal(0.0, spread, lp.shape))
    adv = f32(rng.normal(0.0, 1.0, n_seqs))
    mask = (rng.random(lp.shape) >= mask_frac).astype(np.uint8)
    return lp, old, ref, adv, mask


# ------------------------------------------------------------------ pins (take the oracle)

def pin_hand_worked_tokens(o):
    """Single tokens with ratio 1.5, 0.5 and 1.1, eps 0.2, A = +-2 (values worked by hand;
    the ratio is exp of the float32 rounding of log r, so within 1e-7 of r)."""
    cases = [  # ratio, A, pg, d pg / d logp, clipped
        (1.5, 2.0, -2.4, 0.0, 1),    # A > 0, r > 1 + eps: clipped at 1.2, no gradient
        (1.5, -2.0, 3.0, 3.0, 0),    # A < 0, r > 1 + eps: unclipped
        (0.5, 2.0, -1.0, -1.0, 0),   # A > 0, r < 1 - eps: unclipped
        (0.5, -2.0, 1.6, 0.0, 1),    # A < 0, r < 1 - eps: clipped at 0.8
        (1.1, 2.0, -2.2, -2.2, 0),   # inside the interval
    ]
    for r, A, pg, dpg, clipped in cases:
        lp = f32([[math.log(r)]])
        res = o.loss(lp, f32([[0.0]]), None, f32([A]), mode="token_mean", eps_low=0.2,
                     eps_high=0.2)
        assert abs(res["pg_loss"] - pg) < 2e-6, (r, A)
        assert abs(res["loss"] - pg) < 2e-6, (r, A)
        assert abs(res["dlogp"][0, 0] - dpg) < 2e-6, (r, A)
        assert res["clipped"] == clipped and res["tokens"] == 1


def pin_kl_zero_identity(o):
    """logp == old_logp == ref_logp: ratio exactly 1, per-token pg exactly -A, kl exactly 0,
    and d loss / d logp exactly the gradient of -A logp under the same normalizer."""
    rng = np.random.default_rng(1)
    lp, _, _, adv, mask = random_batch(rng)
    for mode in o.MODES:
        res = o.loss(lp, lp, lp, adv, mask, mode=mode, beta=0.04)
        t = res["terms"]
        act = mask != 0
        assert np.all(t["ratio"][act] == 1.0)
        assert np.all(t["pg"][act] == -np.broadcast_to(adv[:, None], lp.shape)[act])
        assert np.all(t["kl"] == 0.0) and np.all(t["dkl"] == 0.0)
        n_i = act.sum(1)
        if mode == "token_mean":
            w = np.broadcast_to(1.0 / n_i.sum(), lp.shape)
            want_loss = -(adv.astype(np.float64) * n_i).sum() / n_i.sum()
        elif mode == "seq_mean":
            w = np.broadcast_to((1.0 / (n_i * (n_i > 0).sum()))[:, None], lp.shape)
            want_loss = -adv.astype(np.float64)[n_i > 0].mean()
        else:
            w = np.broadcast_to((1.0 / n_i)[:, None], lp.shape)
            want_loss = -adv.astype(np.float64)[n_i > 0].sum()
        want = np.where(act, -adv.astype(np.float64)[:, None] * w, 0.0)
        assert np.array_equal(res["dlogp"], want)
        assert abs(res["loss"] - want_loss) <= 1e-12 * (1 + abs(want_loss))
        assert res["kl_loss"] == 0.0 and res["clipped"] == 0


def pin_reduction_invariants(o):
    rng = np.random.default_rng(2)
    lp, old, ref, adv, _ = random_batch(rng, n_seqs=5, seq_len=40)
    # equal lengths: seq_mean == token_mean; seq_sum == n_seqs * seq_mean
    tm = o.loss(lp, old, ref, adv, None, mode="token_mean", beta=0.1)
    sm = o.loss(lp, old, ref, adv, None, mode="seq_mean", beta=0.1)
    ss = o.loss(lp, old, ref, adv, None, mode="seq_sum_token_mean", beta=0.1)
    assert abs(tm["loss"] - sm["loss"]) < 1e-12
    assert abs(ss["loss"] - 5 * sm["loss"]) < 1e-11
    np.testing.assert_allclose(ss["dlogp"], 5 * sm["dlogp"], rtol=1e-12, atol=0)
    # a global normalizer twice the local one halves loss and gradient
    tm2 = o.loss(lp, old, ref, adv, None, mode="token_mean", beta=0.1, norm_tokens=400)
    assert abs(tm2["loss"] - tm["loss"] / 2) < 1e-12
    np.testing.assert_allclose(tm2["dlogp"], tm["dlogp"] / 2, rtol=1e-12, atol=0)
    sm2 = o.loss(lp, old, ref, adv, None, mode="seq_mean", beta=0.1, norm_seqs=10)
    assert abs(sm2["loss"] - sm["loss"] / 2) < 1e-12
    # masking a token is removing it: token_mean over the masked batch equals token_mean
    # over the kept tokens laid out as one-token sequences
    _, _, _, _, mask = random_batch(rng, n_seqs=5, seq_len=40)
    mk = o.loss(lp, old, ref, adv, mask, mode="token_mean", beta=0.1)
    keep = mask != 0
    A = np.broadcast_to(adv[:, None], lp.shape)
    flat = o.loss(lp[keep][:, None], old[keep][:, None], ref[keep][:, None], A[keep], None,
                  mode="token_mean", beta=0.1)
    assert abs(mk["loss"] - flat["loss"]) < 1e-12 and flat["tokens"] == keep.sum()
    assert mk["clipped"] == flat["clipped"]
    np.testing.assert_allclose(mk["dlogp"][keep], flat["dlogp"][:, 0], rtol=1e-12, atol=0)
    t = o.token_terms(lp, old, ref, adv, mask, 0.2, 0.2)
    # sequence permutation and token permutation inside a sequence leave the loss unchanged
    perm = rng.permutation(5)
    pm = o.loss(lp[perm], old[perm], ref[perm], adv[perm], mask[perm], mode="seq_mean",
                beta=0.1)
    base = o.loss(lp, old, ref, adv, mask, mode="seq_mean", beta=0.1)
    assert abs(pm["loss"] - base["loss"]) < 1e-12
    cols = rng.permutation(40)
    pc = o.loss(lp[:, cols], old[:, cols], ref[:, cols], adv, mask[:, cols], mode="seq_mean",
                beta=0.1)
    assert abs(pc["loss"] - base["loss"]) < 1e-12
    # KL estimator is non-negative and zero only where ref == logp
    assert np.all(t["kl"] >= 0) and np.all((t["kl"] == 0) == ((ref == lp) | ~keep))
    # with nothing clipped the policy term is linear in A
    wide = o.loss(lp, old, None, adv, mask, mode="token_mean", eps_low=0.99, eps_high=1e6)
    wide4 = o.loss(lp, old, None, 4 * adv, mask, mode="token_mean", eps_low=0.99,
                   eps_high=1e6)
    assert wide["clipped"] == 0
    assert abs(wide4["pg_loss"] - 4 * wide["pg_loss"]) < 1e-12
    # empty sequences contribute nothing and are not counted by seq_mean
    m0 = mask.copy()
    m0[2] = 0
    e = o.loss(lp, old, ref, adv, m0, mode="seq_mean", beta=0.1)
    keep_rows = [0, 1, 3, 4]
    e2 = o.loss(lp[keep_rows], old[keep_rows], ref[keep_rows], adv[keep_rows],
                mask[keep_rows], mode="seq_mean", beta=0.1)
    assert e["sequences"] == 4 and abs(e["loss"] - e2["loss"]) < 1e-12
    assert np.all(e["dlogp"][2] == 0)


def pin_finite_difference(o):
    """Central difference of the loss in float64 against d loss / d logp, on tokens away
    from the clip bounds (inputs on a 2^-12 grid so logp +- h stays exact in float32)."""
    rng = np.random.default_rng(3)
    n, T = 3, 12
    lp = f32(np.round(rng.normal(-2.0, 0.5, (n, T)) * 4096) / 4096)
    old = f32(np.round((lp + rng.normal(0, 0.3, lp.shape)) * 4096) / 4096)
    ref = f32(np.round((lp + rng.normal(0, 0.3, lp.shape)) * 4096) / 4096)
    adv = f32([1.5, -0.7, 0.9])
    mask = np.ones((n, T), np.uint8)
    mask[1, 3] = 0
    h = 2.0 ** -12
    for mode in o.MODES:
        base = o.loss(lp, old, ref, adv, mask, mode=mode, beta=0.25)
        t = base["terms"]
        for i in range(n):
            for j in range(T):
                r = t["ratio"][i, j]
                if min(abs(r - 0.8), abs(r - 1.2)) < 0.01:
                    continue
                up, dn = lp.copy(), lp.copy()
                up[i, j] += h
                dn[i, j] -= h
                fd = (o.loss(up, old, ref, adv, mask, mode=mode, beta=0.25)["loss"] -
                      o.loss(dn, old, ref, adv, mask, mode=mode, beta=0.25)["loss"]) / (2 * h)
                assert abs(fd - base["dlogp"][i, j]) < 1e-6, (mode, i, j)


def pin_torch_autograd(o):
    """d loss / d logp against torch float64 autograd of the loss written with torch's
    maximum / clamp / exp (not the oracle's branch form or expm1)."""
    rng = np.random.default_rng(4)
    lp, old, ref, adv, mask = random_batch(rng, n_seqs=7, seq_len=33, spread=0.4)
    mask[3] = 0
    for mode in o.MODES:
        for beta in (0.0, 0.3):
            x = torch.tensor(lp.astype(np.float64), requires_grad=True)
            od = torch.tensor(old.astype(np.float64))
            rf = torch.tensor(ref.astype(np.float64))
            A = torch.tensor(adv.astype(np.float64))[:, None]
            m = torch.tensor(mask.astype(np.float64))
            lo = float(np.float32(1) - np.float32(0.2))
            hi = float(np.float32(1) + np.float32(0.28))
            b32 = float(np.float32(beta))  # beta is a float32 parameter
            ratio = torch.exp(x - od)
            pg = torch.maximum(-A * ratio, -A * torch.clamp(ratio, lo, hi))
            kl = torch.exp(rf - x) - (rf - x) - 1
            per = (pg + b32 * kl) * m
            n_i = m.sum(1)
            if mode == "token_mean":
                L = per.sum() / m.sum()
            else:
                seqm = torch.where(n_i > 0, per.sum(1) / n_i.clamp(min=1), torch.zeros_like(n_i))
                L = seqm.sum() / ((n_i > 0).sum() if mode == "seq_mean" else 1)
            L.backward()
            res = o.loss(lp, old, ref, adv, mask, mode=mode, eps_low=0.2, eps_high=0.28,
                         beta=beta)
            ok = ~res["ambiguous"]
            np.testing.assert_allclose(res["dlogp"][ok], x.grad.numpy()[ok], rtol=1e-12,
                                       atol=1e-15)
            assert abs(res["loss"] - L.item()) < 1e-12 * (1 + abs(L.item()))


def pin_advantages(o):
    rng = np.random.default_rng(5)
    r = rng.normal(0, 2, 64)
    for G in (2, 4, 8, 16):
        a = o.advantages(r, G, eps=1e-6)
        g = torch.tensor(r).reshape(-1, G)
        want = (g - g.mean(1, keepdim=True)) / (g.std(1, keepdim=True) + float(np.float32(1e-6)))
        np.testing.assert_allclose(a, want.reshape(-1).numpy(), rtol=1e-13, atol=1e-14)
        assert np.all(np.abs(a.reshape(-1, G).sum(1)) < 1e-12)
    a2 = o.advantages([0.0, 1.0], 2, eps=0.0)
    assert np.allclose(a2, [-1 / math.sqrt(2), 1 / math.sqrt(2)], rtol=1e-15, atol=0)
    assert np.all(o.advantages([3.0, 5.0, 7.0], 1) == 0.0)
    np.testing.assert_allclose(o.advantages([1.0, 2.0, 6.0, 7.0], 2, scale_by_std=False),
                               [-0.5, 0.5, -0.5, 0.5], rtol=0, atol=0)
    assert np.all(o.advantages([4.0, 4.0, 4.0, 4.0], 4) == 0.0)


PINS = [pin_hand_worked_tokens, pin_kl_zero_identity, pin_reduction_invariants,
        pin_finite_difference, pin_torch_autograd, pin_advantages]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_grpo_oracle_pin(pin):
    pin(load_oracle())


# ------------------------------------------------------------------ planted mistakes

MUTATIONS = [
    ("policy term sign", "pg = np.where(A == 0, 0.0, -A * np.where(clipped, rc, ratio))",
     "pg = np.where(A == 0, 0.0, A * np.where(clipped, rc, ratio))"),
    ("clip bounds swapped", "clipped = ((A > 0) & (r32 > hi)) | ((A < 0) & (r32 < lo))",
     "clipped = ((A > 0) & (r32 < lo)) | ((A < 0) & (r32 > hi))"),
    ("gradient through the clipped branch", "dpg = np.where(clipped, 0.0, -A * ratio)",
     "dpg = -A * ratio"),
    ("KL sign of the linear part", "kl = np.expm1(e) - e", "kl = np.expm1(e) + e"),
    ("KL gradient sign", "dkl = -np.expm1(e)", "dkl = np.expm1(e)"),
    ("biased std", "/ (group_size - 1))", "/ group_size)"),
    ("seq_mean counts empty sequences",
     "D = float(norm_seqs if norm_seqs > 0 else nonempty)",
     "D = float(norm_seqs if norm_seqs > 0 else len(n_i))"),
    ("token_mean ignores the global normalizer",
     "D = float(norm_tokens if norm_tokens > 0 else tokens)", "D = float(tokens)"),
    ("masked tokens kept", "for a in (pg, dpg, kl, dkl):", "for a in ():"),
    ("ratio inverted", "ratio = np.exp(lp - old32.astype(np.float64))",
     "ratio = np.exp(old32.astype(np.float64) - lp)"),
    ("per-sequence scale without the sequence count",
     "scale = np.where(n_i > 0, 1.0 / (safe_n * D), 0.0)",
     "scale = np.where(n_i > 0, 1.0 / D, 0.0)"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    src = open(ORACLE_SRC).read()
    assert old in src, name
    bad = load_oracle(src.replace(old, new))
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bad)
        except Exception:
            failed += 1
    assert failed >= 1, f"no pin catches: {name}"
