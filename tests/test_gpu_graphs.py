"""The entry points under HIP graph capture (torch.cuda.CUDAGraph): no call allocates,
synchronizes or records a memory set, so each can be captured; every replay, with the
program's own eager work and synchronizations between replays and the outputs cleared
eagerly before each, reproduces the eager call's bits.  Outputs and workspaces are allocated
before capture."""

from __future__ import annotations

import pytest
import torch

import deterministic_selected_token_amd as dst
from deterministic_selected_token_amd import grpo, linear

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def bits(t: torch.Tensor) -> torch.Tensor:
    view = {8: torch.int64, 4: torch.int32, 2: torch.int16, 1: torch.uint8}[t.element_size()]
    return t.contiguous().view(view)


def check_capture(step, outputs, replays=3):
    """Eager run, capture, then `replays` replays checked bit for bit against the eager run."""
    step()
    torch.cuda.synchronize()
    ref = [bits(t).clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as capture expects
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    noise = torch.randn((2048, 2048), device=DEV)
    for r in range(replays):
        for t in outputs:
            t.zero_()
        noise = torch.tanh(noise @ noise.t() * 1e-3)  # the program's own eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, rr in zip(outputs, ref):
            assert torch.equal(bits(t), rr), (r, t.shape)
    return graph


def test_logp_forward_backward_capture():
    n, V = 96, 151936
    g = torch.Generator(device=DEV).manual_seed(3)
    x = (torch.randn((n, V), generator=g, device=DEV) * 3).to(torch.bfloat16)
    y = torch.randint(0, V, (n,), generator=g, device=DEV)
    y[::7] = -100
    gr = torch.randn(n, generator=g, device=DEV)
    logp, lse = torch.empty(n, device=DEV), torch.empty(n, device=DEV)
    st = torch.empty((n, 2), device=DEV)
    d = torch.empty_like(x)
    x16 = x.to(torch.float16)
    logp16, lse16 = torch.empty(n, device=DEV), torch.empty(n, device=DEV)
    st16 = torch.empty((n, 2), device=DEV)
    d16 = torch.empty_like(x16)
    say("logp forward + backward under capture (BF16, and FP16 at temperature 0.7)")

    def step():
        dst.logp_forward(x, y, logp=logp, lse=lse, stats=st)
        dst.logp_backward(x, y, gr, st, dlogits=d)
        dst.logp_forward_ex(x16, y, inv_temperature=1 / 0.7, logp=logp16, lse=lse16,
                            stats=st16)
        dst.logp_backward_ex(x16, y, gr, st16, inv_temperature=1 / 0.7, dlogits=d16)

    check_capture(step, [logp, lse, st, d, logp16, lse16, st16, d16])


def test_shard_partials_and_merge_capture():
    n, Vr, Vp = 40, 151936, 159744
    g = torch.Generator(device=DEV).manual_seed(4)
    x = (torch.randn((n, Vp), generator=g, device=DEV) * 3).to(torch.bfloat16)
    y = torch.randint(0, Vr, (n,), generator=g, device=DEV)
    L = dst.logp_num_tiles(Vp)
    partials = torch.empty((n, L, 3), device=DEV)
    logp, lse = torch.empty(n, device=DEV), torch.empty(n, device=DEV)
    st = torch.empty((n, 2), device=DEV)
    T = dst.TILE_COLS
    say("vocab-shard partials + merge under capture")

    def step():
        c0 = 0
        for tiles in (13, 13, 12, 1):
            c1 = min(Vp, c0 + tiles * T)
            dst.logp_partials(x[:, c0:c1], y, Vr, Vp, c0, c1, partials)
            c0 = c1
        dst.logp_merge(partials, y, Vr, logp=logp, lse=lse, stats=st)

    check_capture(step, [partials, logp, lse, st])


def test_linear_logp_capture():
    n, H, V = 600, 512, 40000
    g = torch.Generator(device=DEV).manual_seed(5)
    h = torch.randn((n, H), generator=g, device=DEV).to(torch.bfloat16)
    W = (torch.randn((V, H), generator=g, device=DEV) * (2.0 / H ** 0.5)).to(torch.bfloat16)
    y = torch.randint(0, V, (n,), generator=g, device=DEV)
    gr = torch.randn(n, generator=g, device=DEV)
    L = dst.logp_num_tiles(V)
    partials = torch.empty((n, L, 3), device=DEV)
    logp, lse = torch.empty(n, device=DEV), torch.empty(n, device=DEV)
    st = torch.empty((n, 2), device=DEV)
    ws_f = torch.empty(max(1, linear.linear_logp_partials_workspace(n, V, 0, V)),
                       dtype=torch.uint8, device=DEV)
    chunk = 2 * dst.TILE_COLS
    ws_b = torch.empty(linear.linear_logp_backward_workspace(n, H, chunk, torch.bfloat16),
                       dtype=torch.uint8, device=DEV)
    dh = torch.empty((n, H), dtype=torch.bfloat16, device=DEV)
    dW = torch.empty((V, H), dtype=torch.bfloat16, device=DEV)
    say("linear_logp forward (balanced) + BF16 backward under capture")

    def step():
        linear.linear_logp_forward(h, W, y, V, partials=partials, logp=logp, lse=lse, stats=st,
                                   workspace=ws_f, inv_temperature=1 / 0.7)
        linear.linear_logp_backward(h, W, y, gr, st, V, inv_temperature=1 / 0.7,
                                    chunk_cols=chunk, dhidden=dh, dweight=dW, workspace=ws_b,
                                    out_dtype=torch.bfloat16)

    check_capture(step, [partials, logp, lse, st, dh, dW])


def test_linear_logp_kept_logits_capture():
    n, H, V = 600, 512, 40000
    g = torch.Generator(device=DEV).manual_seed(7)
    h = torch.randn((n, H), generator=g, device=DEV).to(torch.bfloat16)
    W = (torch.randn((V, H), generator=g, device=DEV) * (2.0 / H ** 0.5)).to(torch.bfloat16)
    y = torch.randint(0, V, (n,), generator=g, device=DEV)
    gr = torch.randn(n, generator=g, device=DEV)
    L = dst.logp_num_tiles(V)
    partials = torch.empty((n, L, 3), device=DEV)
    z = torch.empty((n, V), device=DEV)
    logp, lse = torch.empty(n, device=DEV), torch.empty(n, device=DEV)
    st = torch.empty((n, 2), device=DEV)
    ws_f = torch.empty(max(1, linear.linear_logp_partials_workspace(n, V, 0, V)),
                       dtype=torch.uint8, device=DEV)
    chunk = 2 * dst.TILE_COLS
    ws_b = torch.empty(linear.linear_logp_backward_workspace(n, H, chunk, torch.bfloat16),
                       dtype=torch.uint8, device=DEV)
    dh = torch.empty((n, H), dtype=torch.bfloat16, device=DEV)
    dW = torch.empty((V, H), dtype=torch.bfloat16, device=DEV)
    say("linear_logp with kept logits (forward + BF16 backward) under capture")

    def step():
        linear.linear_logp_forward(h, W, y, V, partials=partials, logp=logp, lse=lse, stats=st,
                                   workspace=ws_f, logits=z)
        linear.linear_logp_backward(h, W, y, gr, st, V, chunk_cols=chunk, dhidden=dh,
                                    dweight=dW, workspace=ws_b, out_dtype=torch.bfloat16,
                                    logits=z)

    check_capture(step, [partials, logp, lse, st, dh, dW])


def test_grpo_loss_capture():
    n, T = 256, 3000
    g = torch.Generator(device=DEV).manual_seed(6)
    lp = torch.randn((n, T), generator=g, device=DEV) * 1.5 - 2.0
    old = lp + torch.randn((n, T), generator=g, device=DEV) * 0.3
    ref = lp + torch.randn((n, T), generator=g, device=DEV) * 0.3
    adv = torch.randn(n, generator=g, device=DEV)
    mask = (torch.rand((n, T), generator=g, device=DEV) > 0.1).to(torch.uint8)
    loss = torch.empty(6, dtype=torch.int64, device=DEV)
    sst = torch.empty((n, 4), dtype=torch.int32, device=DEV)
    dl = torch.empty((n, T), device=DEV)
    say("GRPO loss under capture")

    def step():
        grpo.grpo_loss(lp, old, adv, ref_logp=ref, mask=mask, mode="seq_mean", beta=0.04,
                       seq_stats=sst, loss=loss, dlogp=dl)

    check_capture(step, [loss, sst, dl])
