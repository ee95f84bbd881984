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

The backward (``backward``) is the gradient of sum_t g_t logp_t with respect to h and W for
the same scored logits: dz = g inv_t (onehot(y) - softmax(z inv_t)) per valid row (the
derivative the logp path's backward writes as dlogits, PR #495 Summary; the chain rule through
the scoring multiply, PR #314's temperature), then dh = dz W and dW = dz^T h, all in float64.

Parity status (pins in tests/test_linear_oracle_pins.py): logits, forward, tile_partials,
backward: pinned.
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


def _valid_rows(targets, vocab_real: int, active, ignore_index: int) -> np.ndarray:
    """A row is valid when it is active (or no mask is given), its target is not ignore_index
    and 0 <= target < vocab_real (issue #241's contract)."""
    y = np.asarray(targets, dtype=np.int64)
    ok = (y != ignore_index) & (y >= 0) & (y < vocab_real)
    if active is not None:
        ok &= np.asarray(active).astype(bool)
    return ok


def backward(hidden, weight, targets, grad, vocab_real: int, active=None,
             ignore_index: int = -100, inv_temperature: float = 1.0, lib=None) -> dict:
    """Gradients of sum_t g_t logp_t (float64) for logits z = (h W^T) inv_t over the first
    vocab_real rows of W:
      dz[t, v] = g_t inv_t (1[v == y_t] - exp(z[t, v] - LSE_t)) for valid rows, else 0,
      dh = dz W  [n, H],  dW = dz^T h  [vocab_real, H],
    plus dh_abs = |dz| |W| and dW_abs = |dz|^T |h| (the scales of rounding errors) and the
    float64 LSE.  g and inv_t enter as their float32 values."""
    h = _f64(hidden)
    w = _f64(weight)[:int(vocab_real)]
    it = float(np.float32(inv_temperature))
    z = np.ascontiguousarray((h @ w.T) * it)
    g = np.asarray(grad, dtype=np.float32).astype(np.float64)
    y = np.asarray(targets, dtype=np.int64)
    n = h.shape[0]
    lse = _forward(z, y, vocab_real, active=active, ignore_index=ignore_index, lib=lib)["lse"]
    valid = _valid_rows(y, vocab_real, active, ignore_index)
    dz = np.zeros((n, int(vocab_real)))
    rows = np.nonzero(valid)[0]
    if rows.size:
        p = np.exp(z[rows] - lse[rows, None])
        d = -p
        d[np.arange(rows.size), y[rows]] += 1.0
        dz[rows] = (g[rows] * it)[:, None] * d
    return {"dz": dz, "dh": dz @ w, "dW": dz.T @ h, "dh_abs": np.abs(dz) @ np.abs(w),
            "dW_abs": np.abs(dz).T @ np.abs(h), "lse": lse, "valid": valid}
