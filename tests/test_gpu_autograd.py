"""The torch.autograd binding: bitwise the library's own forward and backward, and against
torch float64 autograd of log_softmax + gather on the CPU."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst
from deterministic_selected_token_amd.autograd import selected_token_logp
from parity_checks import spacing

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dtype,inv_t", [(torch.bfloat16, 1.0), (torch.float16, 1 / 0.7),
                                         (torch.float32, 2.0)])
def test_autograd_matches_the_library_and_float64(dtype, inv_t):
    n, V = 37, 3000
    g = torch.Generator().manual_seed(3)
    x = (torch.randn((n, V), generator=g) * 2).to(dtype)
    y = torch.randint(0, V, (n,), generator=g)
    y[5] = -100
    w = torch.randn(n, generator=g)
    print(f"[gpu] autograd {dtype} inv_t={inv_t:.3g}", flush=True)
    xd = x.to(DEV).requires_grad_()
    logp = selected_token_logp(xd, y.to(DEV), inv_temperature=inv_t)
    (logp * w.to(DEV)).sum().backward()
    torch.cuda.synchronize()
    # bitwise the direct calls
    lp, _, stats = dst.logp_forward_ex(xd.detach(), y.to(DEV), inv_temperature=inv_t)
    d = dst.logp_backward_ex(xd.detach(), y.to(DEV), w.to(DEV), stats, inv_temperature=inv_t)
    torch.cuda.synchronize()
    assert torch.equal(logp.detach(), lp) and torch.equal(xd.grad, d)
    # float64 autograd of the scored logits on the CPU
    it = float(np.float32(inv_t))
    z = (x.float() * it).double().requires_grad_()  # the scored logits fl32(x * inv_t)
    ls = torch.log_softmax(z, dim=1)
    valid = y >= 0
    ref = torch.where(valid, ls[torch.arange(n), y.clamp(min=0)],
                      torch.zeros(n, dtype=torch.float64))
    (ref * w.double()).sum().backward()
    grad64 = (z.grad * it).numpy()  # d z / d x = inv_t
    got = xd.grad.float().cpu().double().numpy()
    assert np.abs(logp.detach().cpu().double().numpy() - ref.detach().numpy()).max() <= 1e-4
    tol = spacing(grad64, {torch.bfloat16: "bf16", torch.float16: "f16",
                           torch.float32: "f32"}[dtype]) + 1e-6 * np.abs(grad64).max()
    assert np.all(np.abs(got - grad64) <= tol), np.abs(got - grad64).max()
    assert torch.all(xd.grad[5] == 0)


def test_linear_logp_autograd_matches_the_library():
    from deterministic_selected_token_amd import linear
    from deterministic_selected_token_amd.autograd import linear_logp
    n, H, V = 40, 128, 5000
    g = torch.Generator().manual_seed(4)
    h = torch.randn((n, H), generator=g).to(torch.bfloat16).to(DEV).requires_grad_()
    W = (torch.randn((V, H), generator=g) * 0.2).to(torch.bfloat16).to(DEV).requires_grad_()
    y = torch.randint(0, V, (n,), generator=g).to(DEV)
    w = torch.randn(n, generator=g).to(DEV)
    print("[gpu] linear_logp autograd", flush=True)
    logp = linear_logp(h, W, y, inv_temperature=1 / 0.7, chunk_cols=4096)
    (logp * w).sum().backward()
    lp, _, stats = linear.linear_logp_forward(h.detach(), W.detach(), y, V, V,
                                              inv_temperature=1 / 0.7)
    dh, dW = linear.linear_logp_backward(h.detach(), W.detach(), y, w, stats, V, V,
                                         inv_temperature=1 / 0.7, chunk_cols=4096)
    dh16, dW16 = linear.linear_logp_backward(h.detach(), W.detach(), y, w, stats, V, V,
                                             inv_temperature=1 / 0.7, chunk_cols=4096,
                                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(logp.detach(), lp)
    assert h.grad.dtype == torch.bfloat16 and W.grad.dtype == torch.bfloat16
    # the gradients are the library's BF16 outputs: the FP32 ones rounded to nearest even
    assert torch.equal(h.grad.view(torch.int16), dh16.view(torch.int16))
    assert torch.equal(W.grad.view(torch.int16), dW16.view(torch.int16))
    assert torch.equal(h.grad, dh.to(torch.bfloat16)) and torch.equal(W.grad, dW.to(torch.bfloat16))
