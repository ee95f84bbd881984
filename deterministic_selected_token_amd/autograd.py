"""torch.autograd binding of the selected-token log-probability.

Marshalling only, like the rest of the package: the forward is ``logp_forward_ex`` and the
backward ``logp_backward_ex`` (dlogits straight to the logits' dtype); torch only carries the
tensors and the graph.  ``selected_token_logp(logits, targets)`` is the drop-in for
``log_softmax(logits).gather(targets)`` in a training loss, with this library's deterministic,
batch-invariant forward and backward.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import logp_backward_ex, logp_forward_ex


class SelectedTokenLogp(torch.autograd.Function):
    """logp [n] (float32) of ``targets`` under ``logits`` [n, V] (BF16 / FP16 / FP32, scored
    as fl32(x * inv_temperature)); gradient with respect to ``logits`` only."""

    @staticmethod
    def forward(ctx, logits, targets, vocab_real, vocab_padded, active, ignore_index,
                inv_temperature):
        logp, _, stats = logp_forward_ex(logits, targets, vocab_real, vocab_padded,
                                         active=active, ignore_index=ignore_index,
                                         inv_temperature=inv_temperature)
        ctx.save_for_backward(logits, targets, stats)
        ctx.active = active
        ctx.args = (vocab_real, vocab_padded, ignore_index, inv_temperature)
        return logp

    @staticmethod
    def backward(ctx, grad_logp):
        logits, targets, stats = ctx.saved_tensors
        vocab_real, vocab_padded, ignore_index, inv_temperature = ctx.args
        if grad_logp.dtype != torch.float32 or not grad_logp.is_contiguous():
            grad_logp = grad_logp.float().contiguous()
        dlogits = logp_backward_ex(logits, targets, grad_logp, stats, vocab_real, vocab_padded,
                                   active=ctx.active, ignore_index=ignore_index,
                                   inv_temperature=inv_temperature)
        return dlogits, None, None, None, None, None, None


def selected_token_logp(logits: torch.Tensor, targets: torch.Tensor,
                        vocab_real: Optional[int] = None, vocab_padded: Optional[int] = None,
                        active=None, ignore_index: int = -100,
                        inv_temperature: float = 1.0) -> torch.Tensor:
    """logp[t] = log softmax(fl32(logits[t] * inv_temperature))[targets[t]] (0 for rows that are
    masked, ignored or out of range), differentiable with respect to ``logits``."""
    return SelectedTokenLogp.apply(logits, targets, vocab_real, vocab_padded, active,
                                   ignore_index, inv_temperature)


class LinearLogp(torch.autograd.Function):
    """logp [n] (float32) of ``targets`` under the logits hidden W^T (BF16 hidden [n, H] and
    LM-head weight [V, H]), scored as fl32(acc * inv_temperature); gradients with respect to
    hidden and weight from linear_logp_backward_bf16: accumulated in FP32 and rounded once to
    BF16, the inputs' dtype, inside the library.  keep_logits: the forward keeps the scored
    logits (4 bytes each) and the backward reads them instead of forming them again (the same
    bits)."""

    @staticmethod
    def forward(ctx, hidden, weight, targets, vocab_real, active, ignore_index,
                inv_temperature, chunk_cols, keep_logits=False):
        from .linear import linear_logp_forward
        z = None
        if keep_logits:
            from .linear import kept_logits_buffer
            z = kept_logits_buffer(hidden.shape[0], weight.shape[0], hidden.device)
        logp, _, stats = linear_logp_forward(hidden, weight, targets, vocab_real,
                                             weight.shape[0], active=active,
                                             ignore_index=ignore_index,
                                             inv_temperature=inv_temperature, logits=z)
        ctx.save_for_backward(hidden, weight, targets, stats)
        ctx.active = active
        ctx.logits = z
        ctx.args = (vocab_real, ignore_index, inv_temperature, chunk_cols)
        return logp

    @staticmethod
    def backward(ctx, grad_logp):
        from .linear import linear_logp_backward
        hidden, weight, targets, stats = ctx.saved_tensors
        vocab_real, ignore_index, inv_temperature, chunk_cols = ctx.args
        if grad_logp.dtype != torch.float32 or not grad_logp.is_contiguous():
            grad_logp = grad_logp.float().contiguous()
        dh, dw = linear_logp_backward(hidden, weight, targets, grad_logp, stats, vocab_real,
                                      weight.shape[0], active=ctx.active,
                                      ignore_index=ignore_index,
                                      inv_temperature=inv_temperature, chunk_cols=chunk_cols,
                                      out_dtype=torch.bfloat16, logits=ctx.logits)
        ctx.logits = None
        return dh, dw, None, None, None, None, None, None, None


def linear_logp(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                vocab_real: Optional[int] = None, active=None, ignore_index: int = -100,
                inv_temperature: float = 1.0, chunk_cols: int = 4 * 4096,
                keep_logits: bool = False) -> torch.Tensor:
    """logp[t] = log softmax(hidden[t] W^T)[targets[t]] on the matrix cores, differentiable with
    respect to hidden and weight (rows of W at or past vocab_real are padding).  keep_logits
    trades 4 bytes per logit of memory for a backward that does not form the logits again."""
    vr = weight.shape[0] if vocab_real is None else int(vocab_real)
    return LinearLogp.apply(hidden, weight, targets, vr, active, ignore_index,
                            inv_temperature, chunk_cols, keep_logits)
