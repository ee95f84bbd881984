"""linear_logp with kept logits: linear_logp_partials_save writes the scored logits it forms, and
linear_logp_backward_saved reads them instead of forming h W^T again.  Checks: the partials are
bitwise those of the plain launch; the kept logits are the scored logits (against the FP64
oracle's h W^T within the FP32 accumulation bound, and consistent bit for bit with the
partials' tile maxima and target logits); only the view's real columns are written; and the
backward from them is bitwise the recomputing backward, for FP32 and BF16 gradients, at
temperature, with inactive rows, on column ranges, and at the 8192 x 4096 x 151936 shape."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst
from deterministic_selected_token_amd import linear
from test_gpu_linear import make

pytestmark = pytest.mark.gpu
DEV = "cuda"
T = dst.TILE_COLS


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view({4: torch.int32, 2: torch.int16}[t.element_size()])


def partials_of(h, W, y, V, Vp, inv_t, active=None, logits=None, balance=True):
    n = h.shape[0]
    P = torch.full((n, dst.logp_num_tiles(Vp), 3), float("nan"), device=DEV)
    ws = None
    if balance:
        need = linear.linear_logp_partials_workspace(n, V, 0, Vp)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    linear.linear_logp_partials(h, W, y, V, Vp, 0, Vp, P, active=active, inv_temperature=inv_t,
                                workspace=ws, logits=logits)
    torch.cuda.synchronize()
    return P


@pytest.mark.parametrize("n,H,V,Vp,inv_t,balance", [
    (300, 200, 9000, 9100, 1.0, True), (300, 200, 9000, 9100, 1 / 0.7, False),
    (257, 64, 4096, 4096, 2.0, True), (33, 8, 5003, 8192, 1.0, False),
    (600, 512, 40000, 40000, 1 / 0.7, True)], ids=lambda v: str(v))
def test_saved_forward_keeps_the_scored_logits(n, H, V, Vp, inv_t, balance):
    from oracle import linear_oracle as LO
    say(f"saved forward n={n} H={H} V={V}/{Vp} inv_t={inv_t:.3g} balance={balance}")
    h, W, y = make(n, H, V, Vp, seed=n + H)
    ld = (Vp + 3) // 4 * 4 + 8  # a row stride beyond the width: the margin must stay untouched
    zbuf = torch.full((n, ld), float("nan"), device=DEV)
    z = zbuf[:, :Vp]
    P0 = partials_of(h, W, y, V, Vp, inv_t, balance=balance)
    P1 = partials_of(h, W, y, V, Vp, inv_t, logits=z, balance=balance)
    assert torch.equal(bits(P0), bits(P1)), "keeping the logits changed the partials"
    zc = zbuf.cpu().double().numpy()
    assert np.all(np.isfinite(zc[:, :V])), "a real column was not written"
    assert np.all(np.isnan(zc[:, V:])), "a column past the real vocabulary was written"
    # the scored logits: FP32 accumulation of h W^T, times fl32(inv_t) once
    it = float(np.float32(inv_t))
    exact = LO.logits(h.cpu(), W.cpu()[:V], V) * it
    mag = LO.logit_abs(h.cpu(), W.cpu()[:V], V) * it
    bound = H * 2.0 ** -24 * mag + np.abs(exact) * 2.0 ** -23 + 1e-30
    err = np.abs(zc[:, :V] - exact)
    assert np.all(err <= bound), float((err / bound).max())
    # bit for bit the values the partials came from: each tile's max and the target's logit
    Pc = P1.cpu().numpy()
    zt = zbuf[:, :V].cpu().numpy()
    yc = y.cpu().numpy()
    for l in range(dst.logp_num_tiles(V)):
        c0, c1 = l * T, min(V, (l + 1) * T)
        assert np.array_equal(Pc[:, l, 0], zt[:, c0:c1].max(axis=1)), l
        rows = np.nonzero((yc >= c0) & (yc < c1))[0]
        assert np.array_equal(Pc[rows, l, 2], zt[rows, yc[rows]]), l
    say(f"max |z - z64| / bound {float((err / bound).max()):.3g}")


def backward_pair(h, W, y, V, Vp, inv_t, out_dtype, chunk, active=None, c0=0, c1=None):
    """(recomputing, saved) backward outputs on the same inputs and view [c0, c1)."""
    n, H = h.shape
    c1 = Vp if c1 is None else c1
    g = (torch.randn(n, generator=torch.Generator().manual_seed(9)) * 0.5).to(DEV)
    z = torch.empty((n, Vp), device=DEV)
    P = torch.empty((n, dst.logp_num_tiles(Vp), 3), device=DEV)
    linear.linear_logp_partials(h, W, y, V, Vp, 0, Vp, P, active=active, inv_temperature=inv_t,
                                logits=z)
    _, _, stats = dst.logp_merge(P, y, V, active=active)
    ws = torch.empty(linear.linear_logp_backward_workspace(n, H, chunk, out_dtype),
                     dtype=torch.uint8, device=DEV)
    kw = dict(col_begin=c0, col_end=c1, active=active, inv_temperature=inv_t, chunk_cols=chunk,
              workspace=ws, out_dtype=out_dtype)
    a = linear.linear_logp_backward(h, W[c0:c1], y, g, stats, V, Vp, **kw)
    a = tuple(t.clone() for t in a)
    b = linear.linear_logp_backward(h, W[c0:c1], y, g, stats, V, Vp, logits=z[:, c0:c1], **kw)
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("n,H,V,Vp,inv_t,out,chunk,view", [
    (300, 200, 9000, 9100, 1.0, torch.float32, T, None),
    (300, 200, 9000, 9100, 1 / 0.7, torch.bfloat16, 2 * T, None),
    (257, 64, 20000, 20480, 2.0, torch.float32, T, (T, 4 * T)),
    (600, 512, 40000, 40000, 1 / 0.7, torch.float32, 4 * T, (2 * T, 40000)),
    (33, 8, 5003, 8192, 1.0, torch.bfloat16, T, None)], ids=lambda v: str(v))
def test_saved_backward_is_bitwise_the_recomputing_one(n, H, V, Vp, inv_t, out, chunk, view):
    say(f"saved backward n={n} H={H} V={V}/{Vp} inv_t={inv_t:.3g} {out} chunk={chunk} "
        f"view={view}")
    h, W, y = make(n, H, V, Vp, seed=2 * n + H)
    active = (torch.arange(n, device=DEV) % 7 != 3).to(torch.uint8)
    c0, c1 = view if view is not None else (0, Vp)
    (dh0, dW0), (dh1, dW1) = backward_pair(h, W, y, V, Vp, inv_t, out, chunk, active=active,
                                           c0=c0, c1=c1)
    assert torch.equal(bits(dh0), bits(dh1)) and torch.equal(bits(dW0), bits(dW1))
    assert torch.all(dh1[active == 0] == 0)


def test_saved_full_shape_bitwise():
    """8192 rows, hidden 4096, vocabulary 151936 (the Qwen3-8B LM head): the balanced forward
    keeping its 5.0 GB of logits gives the plain forward's partials, and the BF16-output
    backward from them is bitwise the recomputing one."""
    n, H, V = 8192, 4096, 151936
    say(f"saved logits at {n} x {H} x {V}")
    gen = torch.Generator(device=DEV).manual_seed(21)
    h = torch.randn((n, H), generator=gen, device=DEV).to(torch.bfloat16)
    W = (torch.randn((V, H), generator=gen, device=DEV) * (3.0 / H ** 0.5)).to(torch.bfloat16)
    y = torch.randint(0, V, (n,), generator=gen, device=DEV)
    y[::13] = -100
    z = torch.empty((n, V), device=DEV)
    P0 = partials_of(h, W, y, V, V, 1.0)
    P1 = partials_of(h, W, y, V, V, 1.0, logits=z)
    assert torch.equal(bits(P0), bits(P1))
    _, _, stats = dst.logp_merge(P1, y, V)
    g = torch.randn(n, generator=gen, device=DEV) * 0.1
    chunk = 4 * T
    ws = torch.empty(linear.linear_logp_backward_workspace(n, H, chunk, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)
    kw = dict(chunk_cols=chunk, workspace=ws, out_dtype=torch.bfloat16)
    dh0, dW0 = (t.clone() for t in linear.linear_logp_backward(h, W, y, g, stats, V, V, **kw))
    dh1, dW1 = linear.linear_logp_backward(h, W, y, g, stats, V, V, logits=z, **kw)
    torch.cuda.synchronize()
    assert torch.equal(bits(dh0), bits(dh1)) and torch.equal(bits(dW0), bits(dW1))


@pytest.mark.parametrize("V", [10000, 10007])
def test_autograd_keep_logits_is_bitwise(V):
    from deterministic_selected_token_amd.autograd import linear_logp
    n, H = 300, 128
    say("autograd linear_logp keep_logits")
    g = torch.Generator().manual_seed(8)
    h0 = torch.randn((n, H), generator=g).to(torch.bfloat16).to(DEV)
    W0 = (torch.randn((V, H), generator=g) * 0.2).to(torch.bfloat16).to(DEV)
    y = torch.randint(0, V, (n,), generator=g).to(DEV)
    w = torch.randn(n, generator=g).to(DEV)
    grads = []
    for keep in (False, True):
        h, W = h0.clone().requires_grad_(), W0.clone().requires_grad_()
        logp = linear_logp(h, W, y, inv_temperature=1 / 0.7, keep_logits=keep)
        (logp * w).sum().backward()
        torch.cuda.synchronize()
        grads.append((logp.detach(), h.grad, W.grad))
    for a, b in zip(*grads):
        assert torch.equal(bits(a), bits(b))


@pytest.mark.parametrize("inv_t", [1.0, 1 / 0.7])
def test_saved_forward_on_vocab_shards(inv_t):
    """Each tile-aligned shard keeps the logits of its own columns, with column 0 of its
    buffer at the shard's first column: bitwise the full forward's columns, and the shard's
    partials bitwise those of the non-keeping call."""
    n, H, V, Vp = 200, 136, 21000, 21504
    say(f"saved forward on shards inv_t={inv_t:.3g}")
    h, W, y = make(n, H, V, Vp, seed=77)
    zfull = linear.kept_logits_buffer(n, Vp, DEV)
    P = torch.empty((n, dst.logp_num_tiles(Vp), 3), device=DEV)
    linear.linear_logp_partials(h, W, y, V, Vp, 0, Vp, P, inv_temperature=inv_t, logits=zfull)
    for c0, c1 in ((0, T), (T, 3 * T), (3 * T, Vp)):
        zs = linear.kept_logits_buffer(n, c1 - c0, DEV)
        zs.fill_(float("nan"))
        P0 = torch.full_like(P, float("nan"))
        P1 = torch.full_like(P, float("nan"))
        linear.linear_logp_partials(h, W[c0:c1], y, V, Vp, c0, c1, P0, inv_temperature=inv_t)
        linear.linear_logp_partials(h, W[c0:c1], y, V, Vp, c0, c1, P1, inv_temperature=inv_t,
                                    logits=zs)
        torch.cuda.synchronize()
        assert torch.equal(bits(P0), bits(P1)), (c0, c1)
        real = max(0, min(c1, V) - c0)
        assert torch.equal(bits(zs[:, :real]), bits(zfull[:, c0:c0 + real])), (c0, c1)
        assert torch.all(torch.isnan(zs[:, real:])), (c0, c1)
