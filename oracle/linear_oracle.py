"""FP64 CPU oracle for the fused LM-head + selected-token log-probability (linear_logp).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the product path never imports it.

What it follows: PR #495 "zero-workspace backward for generic CUDA fused logp" names
``linear_logp`` (the fused LM-head plus logp op) next to the generic fused logp; the pages
give no more than its name.  The reading taken: hidden states h [n, H] (BF16) times the
LM-head weight W [V, H] (BF16, one row per vocabulary entry, as a linear layer stores it)
give the logits z = h W^T, and the op returns what the selected-token log-probability
path returns for those logits (issue #241: logp = z[y] - logsumexp z, LSE, and the
per-tile partials of the vocab-parallel merge), without materialising [n, V].

The oracle is the plain definition: z in float64 (each BF16 x BF16 product is exact in
double; numpy's float64 matmul adds them), rows of W at or beyond vocab_real left out,
then the float64 log-softmax of ``logp_oracle.c`` on those logits.  The kernels accumulate
z in float32, so parity is up to that rounding: ``logit_abs`` gives sum_k |h_k W_vk|, the
scale of the accumulation error of each logit.

Parity status (pins in tests/test_linear_oracle_pins.py): logits, forward, tile_partials:
pinned.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import _logits, forward as _forward, tile_partials as _tile_partials


def _f64(x) -> np.ndarray:
    """BF16 (torch tensor or raw uint16 bits), float16/32/64 -> float64 array."""
    a, dt = _logits(x)
    if dt == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def logits(hidden, weight, vocab_real: Optional[int] = None) -> np.ndarray:
    """z = h W^T in float64 for the first vocab_real rows of W: [n, vocab_real]."""
    h = _f64(hidden)
    w = _f64(weight)
    v = w.shape[0] if vocab_real is None else int(vocab_real)
    return h @ w[:v].T


def logit_abs(hidden, weight, vocab_real: Optional[int] = None) -> np.ndarray:
    """sum_k |h_k| |W_vk| per logit: [n, vocab_real]."""
    h = np.abs(_f64(hidden))
    w = np.abs(_f64(weight))
    v = w.shape[0] if vocab_real is None else int(vocab_real)
    return h @ w[:v].T


def forward(hidden, weight, targets, vocab_real: int, active=None, ignore_index: int = -100,
            lib=None, inv_temperature: float = 1.0) -> dict:
    """logp, LSE, M, S (float64) of the logits h W^T, as ``oracle.forward`` defines them;
    with inv_temperature the scored logits are z * inv_temperature (one float64 product with
    the float32 value of inv_temperature, PR #314's temperature-scaled scoring)."""
    z = np.ascontiguousarray(logits(hidden, weight, vocab_real))
    out = _forward(z, targets, vocab_real, active=active, ignore_index=ignore_index, lib=lib,
                   inv_temperature=inv_temperature)
    out["logits"] = z
    return out


def tile_partials(hidden, weight, targets, vocab_real: int, vocab_padded: int, tile: int = 4096,
                  active=None, ignore_index: int = -100, lib=None,
                  inv_temperature: float = 1.0) -> dict:
    """Per global tile (m_l, s_l, sel_l) of the logits h W^T scored by inv_temperature
    (columns >= vocab_real masked)."""
    z = logits(hidden, weight, vocab_real)
    zp = np.full((z.shape[0], vocab_padded), -np.inf)
    zp[:, :vocab_real] = z
    return _tile_partials(np.ascontiguousarray(zp), targets, vocab_real, vocab_padded,
                          tile=tile, active=active, ignore_index=ignore_index, lib=lib,
                          inv_temperature=inv_temperature)
