"""FP64 CPU oracle for the deterministic GRPO loss on selected-token log-probabilities.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg are the only users.  The product path never imports it, and it shares
no code with the HIP kernels.

What it follows: issue #241 "[WS2] TP-aware deterministic logprob …", planned PR5
("Deterministic GRPO loss on the TP-aware logprob path"): the GRPO objective (ratio, clip,
KL, advantage normalization) bound to a declared reduction (normalizers token_mean /
seq_mean / seq_sum_token_mean; n_non_ignore global or local), and the KL=0 identity as its
acceptance test.  The pages name these parts but print no formulas; the readings taken:

* ratio r = exp(logp - old_logp); clip bounds lo = fl32(1 - eps_low), hi = fl32(1 + eps_high);
  policy term pg = max(-A r, -A clip(r, lo, hi)), i.e. -A min(r, hi) for A > 0 and
  -A max(r, lo) for A < 0; the clipped branch is the active one exactly when A > 0 and r > hi,
  or A < 0 and r < lo, and then d pg / d logp = 0, else -A r.
* KL to the reference policy, the non-negative estimator of the GRPO formulation:
  kl = exp(ref - logp) - (ref - logp) - 1, d kl / d logp = 1 - exp(ref - logp).
* per-token loss l = pg + beta kl over active tokens (mask != 0); inactive tokens add
  nothing and get a zero gradient.
* normalizers: token_mean = sum over active tokens / D_tok (D_tok = the given global
  n_non_ignore, else the local active-token count); seq_mean = mean over non-empty
  sequences of each sequence's token mean (D_seq = the given global sequence count, else the
  local number of non-empty sequences); seq_sum_token_mean = sum over sequences of each
  sequence's token mean.  pg_loss and kl_loss are reduced separately and
  loss = pg_loss + beta kl_loss.
* advantage normalization per group of G consecutive responses:
  A = (r - mean) / (std + eps) with the unbiased std, or A = r - mean without std scaling;
  a group of one gets A = 0.

Precision: every value is computed in float64 from the float32 inputs, except the one
decision that picks the clip branch, which is taken on the float32 ratio
fl32(exp(fl32(logp - old_logp))) as the kernels take it; tokens whose float32 ratio lies
within two float32 spacings of a bound are flagged ``ambiguous`` (either branch is correct
for them, since a last-bit difference in exp moves them across).

Parity status (pins in tests/test_grpo_oracle_pins.py): advantages, token_terms, loss: pinned.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

MODES = ("token_mean", "seq_mean", "seq_sum_token_mean")


def advantages(rewards, group_size: int, eps: float = 1e-6, scale_by_std: bool = True):
    """Group-normalized advantages (issue #241, PR5: advantage normalization)."""
    r = np.asarray(rewards, dtype=np.float64)
    if r.size % group_size:
        raise ValueError("number of rewards must be a multiple of group_size")
    g = r.reshape(-1, group_size)
    if group_size == 1:
        return np.zeros_like(r)
    mean = g.mean(axis=1, keepdims=True)
    a = g - mean
    if scale_by_std:
        std = np.sqrt(((g - mean) ** 2).sum(axis=1, keepdims=True) / (group_size - 1))
        a = a / (std + float(np.float32(eps)))
    return a.reshape(-1)


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def token_terms(logp, old_logp, ref_logp, adv, mask, eps_low: float, eps_high: float):
    """Per-token GRPO terms for [n_seqs, seq_len] float32 inputs; adv is per sequence."""
    lp32, old32 = _f32(logp), _f32(old_logp)
    lp = lp32.astype(np.float64)
    A = _f32(adv).astype(np.float64)[:, None] * np.ones_like(lp)
    act = np.ones(lp.shape, dtype=bool) if mask is None else np.asarray(mask) != 0

    ratio = np.exp(lp - old32.astype(np.float64))
    # the clip decision, in the kernels' float32 arithmetic
    lo = np.float32(1.0) - np.float32(eps_low)
    hi = np.float32(1.0) + np.float32(eps_high)
    with np.errstate(over="ignore"):
        r32 = np.exp((lp32 - old32).astype(np.float64)).astype(np.float32)
    clipped = ((A > 0) & (r32 > hi)) | ((A < 0) & (r32 < lo))
    near = lambda b: np.abs(r32.astype(np.float64) - float(b)) <= 2.0 * float(np.spacing(b))
    ambiguous = act & (A != 0) & (near(hi) | near(lo))

    rc = np.where(A > 0, np.minimum(ratio, float(hi)), np.maximum(ratio, float(lo)))
    pg = np.where(A == 0, 0.0, -A * np.where(clipped, rc, ratio))
    dpg = np.where(clipped, 0.0, -A * ratio)
    if ref_logp is None:
        kl = np.zeros_like(lp)
        dkl = np.zeros_like(lp)
    else:
        e = _f32(ref_logp).astype(np.float64) - lp
        kl = np.expm1(e) - e
        dkl = -np.expm1(e)
    zero = ~act
    for a in (pg, dpg, kl, dkl):
        a[zero] = 0.0
    return {"ratio": ratio, "ratio32": r32, "clipped": clipped & act, "ambiguous": ambiguous,
            "pg": pg, "dpg": dpg, "kl": kl, "dkl": dkl, "active": act}


def loss(logp, old_logp, ref_logp, adv, mask=None, mode: str = "token_mean",
         eps_low: float = 0.2, eps_high: float = 0.2, beta: float = 0.0,
         norm_tokens: int = 0, norm_seqs: int = 0, seq_len: Optional[int] = None):
    """GRPO loss, its parts and d loss / d logp (float64) for [n_seqs, seq_len] inputs."""
    if mode not in MODES:
        raise ValueError(mode)
    t = token_terms(logp, old_logp, ref_logp, adv, mask, eps_low, eps_high)
    beta = float(np.float32(beta))
    if ref_logp is None:
        beta = 0.0
    act = t["active"]
    n_i = act.sum(axis=1).astype(np.int64)
    pg_i = t["pg"].sum(axis=1)
    kl_i = t["kl"].sum(axis=1)
    clip_i = t["clipped"].sum(axis=1).astype(np.int64)
    tokens = int(n_i.sum())
    nonempty = int((n_i > 0).sum())
    safe_n = np.where(n_i > 0, n_i, 1).astype(np.float64)

    if mode == "token_mean":
        D = float(norm_tokens if norm_tokens > 0 else tokens)
        pg_loss = pg_i.sum() / D if D > 0 else 0.0
        kl_loss = kl_i.sum() / D if D > 0 else 0.0
        scale = np.full(len(n_i), 1.0 / D if D > 0 else 0.0)
    else:
        pg_mean = np.where(n_i > 0, pg_i / safe_n, 0.0)
        kl_mean = np.where(n_i > 0, kl_i / safe_n, 0.0)
        if mode == "seq_mean":
            D = float(norm_seqs if norm_seqs > 0 else nonempty)
        else:
            D = 1.0
        pg_loss = pg_mean.sum() / D if D > 0 else 0.0
        kl_loss = kl_mean.sum() / D if D > 0 else 0.0
        scale = np.where(n_i > 0, 1.0 / (safe_n * D), 0.0) if D > 0 else np.zeros(len(n_i))
    dl = t["dpg"] + beta * t["dkl"]
    dlogp = np.where(act, dl * scale[:, None], 0.0)
    return {"loss": pg_loss + beta * kl_loss, "pg_loss": pg_loss, "kl_loss": kl_loss,
            "clip_frac": float(clip_i.sum()) / tokens if tokens else 0.0,
            "tokens": tokens, "sequences": nonempty, "clipped": int(clip_i.sum()),
            "seq_pg_sum": pg_i, "seq_kl_sum": kl_i, "seq_clipped": clip_i, "seq_tokens": n_i,
            "dlogp": dlogp, "ambiguous": t["ambiguous"], "terms": t,
            "per_token_abs": np.abs(t["pg"]) + beta * np.abs(t["kl"]),
            "grad_abs": np.abs(t["dpg"]) + beta * np.abs(t["dkl"])}
