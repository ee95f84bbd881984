"""Pins of the FP64 linear_logp oracle (CPU only).

Each pin checks it against something other than itself: one-hot hidden states, which turn
h W^T into columns of W and so reduce linear_logp to the (separately pinned) logp oracle on
BF16 logits; an exactness case that a float32 accumulation would get wrong; torch float64
log_softmax of h W^T; uniform rows; padded vocabulary rows that must not count; and
linearity in h.  The backward is pinned by torch float64 autograd, central finite differences
of the pinned forward, one-hot hidden rows (which reduce dz to the logp oracle's own dlogits)
and the zero row sums of dz.  Planted mistakes (altered copies of the oracle source) must each
fail one.
"""

from __future__ import annotations

import math
import os
import types

import numpy as np
import pytest
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "linear_oracle.py")


def load(src: str = None):
    src = open(SRC).read() if src is None else src
    mod = types.ModuleType("oracle.linear_oracle_copy")
    mod.__package__ = "oracle"
    exec(compile(src, SRC, "exec"), mod.__dict__)
    return mod


def bf16(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def rand_bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


def pin_one_hot_rows(o):
    """h[t] = c_t e_{k_t}: logits[t, v] = c_t W[v, k_t] exactly, so linear_logp equals the
    logp oracle on the BF16 logits c_t W[:, k_t] (c_t powers of two keep them BF16)."""
    n, H, V = 6, 40, 300
    W = rand_bf16((V, H), 1, 2.0)
    ks = [0, 7, 39, 12, 12, 25]
    cs = [1.0, 2.0, 0.5, -1.0, 4.0, 1.0]
    h = torch.zeros((n, H), dtype=torch.bfloat16)
    for t, (k, c) in enumerate(zip(ks, cs)):
        h[t, k] = c
    y = np.array([3, 0, 299, 150, 7, 42])
    got = o.forward(h, W, y, V)
    z = torch.stack([W[:, k].float() * c for k, c in zip(ks, cs)]).to(torch.bfloat16)
    want = oracle.forward(z, y, V)
    assert np.array_equal(got["logits"], z.double().numpy())
    for key in ("logp", "lse", "max", "sumexp"):
        assert np.array_equal(got[key], want[key]), key


def pin_exact_accumulation(o):
    """2^10 * 1 + 1 * 2^-20 + (-2^10) * 1 = 2^-20 exactly; a float32 running sum loses the
    small term (2^10 + 2^-20 needs 31 significand bits)."""
    h = bf16([[1024.0, 1.0, -1024.0]])
    W = bf16([[1.0, 2.0 ** -20, 1.0], [0.0, 0.0, 0.0]])
    z = o.logits(h, W)
    assert z[0, 0] == 2.0 ** -20 and z[0, 1] == 0.0
    assert np.all(o.logit_abs(h, W)[0] == [2048.0 + 2.0 ** -20, 0.0])


def pin_torch_log_softmax(o):
    n, H, V = 9, 64, 517
    h = rand_bf16((n, H), 2)
    W = rand_bf16((V, H), 3, 0.3)
    y = np.array([0, 5, 516, 100, 200, 300, 400, 1, 2])
    got = o.forward(h, W, y, V)
    z = h.double() @ W.double().T
    ls = torch.log_softmax(z, dim=1)
    np.testing.assert_allclose(got["logp"], ls[np.arange(n), y].numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["lse"], torch.logsumexp(z, 1).numpy(), rtol=0, atol=1e-12)


def pin_uniform_and_padding(o):
    """Equal rows of W give -log V; rows at or beyond vocab_real never count, even huge ones."""
    V, Vp, H = 1000, 1024, 16
    W = torch.zeros((Vp, H), dtype=torch.bfloat16)
    W[:V] = bf16(np.full((V, H), 0.25))
    W[V:] = 100.0
    h = rand_bf16((3, H), 4)
    got = o.forward(h, W, np.array([0, 999, 500]), V)
    assert np.allclose(got["logp"], -math.log(V), rtol=0, atol=1e-13)
    p = o.tile_partials(h, W, np.array([0, 999, 500]), V, Vp, tile=256)
    assert np.all(np.isfinite(p["max"][:, :3])) and p["max"].shape == (3, 4)
    assert np.all(p["max"][:, 3] == got["max"])  # the last tile holds 232 real columns


def pin_linearity_and_orientation(o):
    """z(h1 + h2) = z(h1) + z(h2) (exact here: small integers), and z[t, v] pairs hidden row t
    with vocabulary row v on a non-square shape."""
    h1 = bf16(np.arange(12).reshape(3, 4) % 5 - 2)
    h2 = bf16(np.arange(12).reshape(3, 4) % 3)
    W = bf16(np.arange(20).reshape(5, 4) % 7 - 3)
    z = o.logits(h1, W)
    assert z.shape == (3, 5)
    assert np.array_equal(o.logits(bf16(h1.float() + h2.float()), W), z + o.logits(h2, W))
    assert z[2, 4] == sum(float(h1[2, k]) * float(W[4, k]) for k in range(4))


def pin_temperature(o):
    """Scoring at inv_temperature = 1/2 equals halving W (exact in BF16 and in float64), on the
    forward and the tile partials; at 1/0.7 it is torch's float64 log_softmax of z times the
    float32 value of 1/0.7."""
    n, H, V = 7, 48, 700
    h = rand_bf16((n, H), 5)
    W = rand_bf16((V, H), 6, 0.5)
    y = np.array([0, 1, 699, 350, 2, 698, 10])
    half = (W.float() * 0.5).to(torch.bfloat16)
    got = o.forward(h, W, y, V, inv_temperature=0.5)
    want = o.forward(h, half, y, V)
    for key in ("logp", "lse", "max", "sumexp"):
        assert np.array_equal(got[key], want[key]), key
    pg = o.tile_partials(h, W, y, V, 768, tile=256, inv_temperature=0.5)
    pw = o.tile_partials(h, half, y, V, 768, tile=256)
    for key in ("max", "sumexp", "sel"):
        assert np.array_equal(pg[key], pw[key]), key
    inv_t = float(np.float32(1 / 0.7))
    got = o.forward(h, W, y, V, inv_temperature=1 / 0.7)
    z = (h.double() @ W.double().T) * inv_t
    ls = torch.log_softmax(z, dim=1)
    np.testing.assert_allclose(got["logp"], ls[np.arange(n), y].numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["max"], z.max(1).values.numpy(), rtol=0, atol=0)


def _bwd_case(seed=8, n=6, H=12, V=40):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn((n, H), generator=g, dtype=torch.float64)
    W = torch.randn((V, H), generator=g, dtype=torch.float64) * 0.7
    y = np.array([0, V - 1, 5, 17, -100, 3])[:n]
    grad = np.array([1.0, -0.5, 2.0, 0.25, 1.0, -1.5], dtype=np.float32)[:n]
    active = np.array([1, 1, 1, 0, 1, 1], dtype=np.uint8)[:n]
    return h, W, y, grad, active


def pin_backward_autograd(o):
    """torch float64 autograd of sum over valid rows of g_t log_softmax(h W^T inv_t)[t, y_t]
    (row 3 inactive, row 4 ignored)."""
    h, W, y, grad, active = _bwd_case()
    inv_t = 1 / 0.7
    got = o.backward(h.numpy(), W.numpy(), y, grad, W.shape[0], active=active,
                     inv_temperature=inv_t)
    hh, WW = h.clone().requires_grad_(), W.clone().requires_grad_()
    ls = torch.log_softmax((hh @ WW.T) * float(np.float32(inv_t)), dim=1)
    loss = sum(float(grad[t]) * ls[t, y[t]] for t in range(len(y))
               if active[t] and 0 <= y[t] < W.shape[0])
    loss.backward()
    np.testing.assert_allclose(got["dh"], hh.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["dW"], WW.grad.numpy(), rtol=0, atol=1e-12)
    assert np.all(got["dz"][3] == 0) and np.all(got["dz"][4] == 0)
    assert np.all(got["dh"][3] == 0) and np.all(got["dh"][4] == 0)


def pin_backward_finite_difference(o):
    """Central differences of L(h, W) = sum_t g_t logp_t, with logp from the (separately
    pinned) forward, on a few coordinates of h and of W."""
    h, W, y, grad, active = _bwd_case(seed=9, n=4, H=6, V=11)
    y = np.array([0, 10, 4, 7])
    inv_t = 0.5
    got = o.backward(h.numpy(), W.numpy(), y, grad, 11, inv_temperature=inv_t)

    def loss(hv, wv):
        f = o.forward(hv, wv, y, 11, inv_temperature=inv_t)
        return float(np.sum(grad.astype(np.float64) * f["logp"]))

    eps = 1e-6
    for (t, k) in ((0, 0), (2, 5), (3, 3)):
        hp, hm = h.numpy().copy(), h.numpy().copy()
        hp[t, k] += eps
        hm[t, k] -= eps
        fd = (loss(hp, W.numpy()) - loss(hm, W.numpy())) / (2 * eps)
        assert abs(fd - got["dh"][t, k]) <= 1e-6 * (1 + abs(fd)), (t, k, fd, got["dh"][t, k])
    for (v, k) in ((0, 1), (10, 5), (4, 0)):
        wp, wm = W.numpy().copy(), W.numpy().copy()
        wp[v, k] += eps
        wm[v, k] -= eps
        fd = (loss(h.numpy(), wp) - loss(h.numpy(), wm)) / (2 * eps)
        assert abs(fd - got["dW"][v, k]) <= 1e-6 * (1 + abs(fd)), (v, k, fd, got["dW"][v, k])


def pin_backward_one_hot_rows(o):
    """h[t] = c_t e_{k_t} makes the logits BF16 columns of W, so dz is the logp oracle's own
    dlogits on them, and dW[:, k] collects c_t dz[t, :] over the rows with k_t = k."""
    n, H, V = 5, 9, 50
    W = rand_bf16((V, H), 10, 2.0)
    ks, cs = [0, 4, 8, 4, 2], [1.0, 2.0, -0.5, 1.0, 4.0]
    h = torch.zeros((n, H), dtype=torch.bfloat16)
    for t, (k, c) in enumerate(zip(ks, cs)):
        h[t, k] = c
    y = np.array([1, 0, 49, 20, 33])
    grad = np.array([1.0, -2.0, 0.5, 1.5, -1.0], dtype=np.float32)
    got = o.backward(h, W, y, grad, V)
    z = torch.stack([W[:, k].float() * c for k, c in zip(ks, cs)]).to(torch.bfloat16)
    want = oracle.backward(z, y, grad, V, want_bf16=False)["d64"]
    np.testing.assert_allclose(got["dz"], want, rtol=0, atol=1e-14)
    wf = W.double().numpy()
    for k in range(H):
        col = sum(cs[t] * want[t] for t in range(n) if ks[t] == k)
        np.testing.assert_allclose(got["dW"][:, k], col if np.ndim(col) else np.zeros(V),
                                   rtol=0, atol=1e-13)
    np.testing.assert_allclose(got["dh"], want @ wf, rtol=0, atol=1e-13)


def pin_backward_rows_sum_to_zero(o):
    """Each valid dz row sums to 0 (softmax sums to 1), so identical rows of W give dh = 0;
    the rows of an all-zero h give dW = 0."""
    h, W, y, grad, active = _bwd_case(seed=11)
    Weq = np.tile(W.numpy()[:1], (W.shape[0], 1))
    got = o.backward(h.numpy(), Weq, y, grad, W.shape[0], active=active)
    assert np.all(np.abs(got["dz"].sum(axis=1)) <= 1e-14)
    assert np.all(np.abs(got["dh"]) <= 1e-13 * (1 + got["dh_abs"]))
    zero = o.backward(np.zeros_like(h.numpy()), W.numpy(), y, grad, W.shape[0])
    assert np.all(zero["dW"] == 0)


PINS = [pin_one_hot_rows, pin_exact_accumulation, pin_torch_log_softmax,
        pin_uniform_and_padding, pin_linearity_and_orientation, pin_temperature,
        pin_backward_autograd, pin_backward_finite_difference, pin_backward_one_hot_rows,
        pin_backward_rows_sum_to_zero]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_linear_oracle_pin(pin):
    pin(load())


MUTATIONS = [
    ("float32 accumulation", "    return h @ w[:v].T\n",
     "    return (h.astype(np.float32) @ w[:v].T.astype(np.float32)).astype(np.float64)\n"),
    ("weight used untransposed", "    return h @ w[:v].T\n", "    return h @ w[:v, :v]\n"),
    ("vocabulary order reversed", "    return h @ w[:v].T\n", "    return h @ w[:v][::-1].T\n"),
    ("temperature dropped from the forward",
     "lib=lib,\n                   inv_temperature=inv_temperature)", "lib=lib)"),
    ("temperature dropped from the tile partials",
     "lib=lib,\n                          inv_temperature=inv_temperature)", "lib=lib)"),
    ("backward without the temperature factor",
     "dz[rows] = (g[rows] * it)[:, None] * d", "dz[rows] = g[rows][:, None] * d"),
    ("backward with the softmax sign flipped", "        d = -p\n", "        d = p\n"),
    ("backward keeps inactive rows", "        ok &= np.asarray(active).astype(bool)\n",
     "        pass\n"),
    ("dh with the vocabulary order reversed", '"dh": dz @ w,', '"dh": dz @ w[::-1],'),
    ("dW with the rows of h reversed", '"dW": dz.T @ h,', '"dW": dz.T @ h[::-1],'),
    ("bf16 decoded with the wrong shift",
     "(a.astype(np.uint32) << 16).view(np.float32)",
     "(a.astype(np.uint32) << 15).view(np.float32)"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    src = open(SRC).read()
    assert old in src, name
    bad = load(src.replace(old, new, 1))
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bad)
        except Exception:
            failed += 1
    assert failed >= 1, f"no pin catches: {name}"
