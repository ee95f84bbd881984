"""Element-wise comparison of the GPU outputs with the FP64 oracle.

Tolerances (written here, used by every GPU parity test):
  * logp and LSE: |gpu - oracle| <= 1e-4 absolute, the bar the accuracy target sets for
    the selected-token logp.  Row max M is compared exactly (a max of BF16 values is
    exact in FP32); S to 2e-5 relative (FP32 sums of up to ~1.5e5 exp terms).
  * dlogits (BF16): at least 99.99% of all N x vocab_real elements equal the
    round-to-nearest-even of the FP64 value; the largest |gpu - d64| is at most
    max(1.5e-3 * max|d64|, 1.01 * E_floor), where E_floor = max|RNE(d64) - d64| is the
    error a perfectly rounded BF16 output already has (the pages show every correct
    implementation sharing that floor: the fused-backward pull request, author reply
    accuracy table); every non-target element lies within one BF16 spacing of d64 and
    the target element within one spacing plus 2^-20 |g| (1 - p is formed in FP32);
    padded columns and invalid rows are exactly +0.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import oracle

LOGP_TOL = 1e-4
SUMEXP_RTOL = 2e-5
CORRECTLY_ROUNDED_MIN = 0.9999
MAXERR_RATIO = 1.5e-3


def bits_of(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bits of a bf16 tensor (copied to the host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_spacing(v: np.ndarray) -> np.ndarray:
    """Spacing of BF16 numbers in the binade of |v| (2^-133 in the subnormal range)."""
    a = np.abs(v)
    _, e = np.frexp(a)  # a = f 2^e, f in [0.5, 1)
    sp = np.ldexp(np.ones_like(a), e - 8)
    return np.maximum(sp, 2.0 ** -133)


def valid_rows(targets, active, vocab_real: int, ignore_index: int) -> np.ndarray:
    y = np.asarray(targets)
    ok = (y != ignore_index) & (y >= 0) & (y < vocab_real)
    if active is not None:
        ok &= np.asarray(active) != 0
    return ok


def check_forward(logits_host, targets, vocab_real, active, ignore_index, logp, lse, stats,
                  what: str = "") -> dict:
    """Compare GPU forward outputs (numpy float32) with the oracle; returns stats."""
    ref = oracle.forward(logits_host, targets, vocab_real, active=active,
                         ignore_index=ignore_index)
    logp = np.asarray(logp, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    st = np.asarray(stats, dtype=np.float64)
    finite = np.isfinite(ref["lse"])
    d_logp = np.abs(logp - ref["logp"])
    d_logp[~np.isfinite(ref["logp"])] = 0.0
    assert np.array_equal(np.isneginf(logp), np.isneginf(ref["logp"])), what
    assert np.all(d_logp <= LOGP_TOL), (what, float(d_logp.max()), int(d_logp.argmax()))
    d_lse = np.abs(lse[finite] - ref["lse"][finite])
    assert np.all(np.isneginf(lse[~finite])), what
    assert d_lse.size == 0 or d_lse.max() <= LOGP_TOL, (what, float(d_lse.max()))
    assert np.array_equal(st[:, 0], ref["max"]), what
    s_rel = np.abs(st[finite, 1] - ref["sumexp"][finite]) / ref["sumexp"][finite]
    assert s_rel.size == 0 or s_rel.max() <= SUMEXP_RTOL, (what, float(s_rel.max()))
    v = valid_rows(targets, active, vocab_real, ignore_index)
    assert np.all(logp[~v] == 0.0), what
    return {"logp_max_abs_err": float(d_logp.max()) if d_logp.size else 0.0,
            "lse_max_abs_err": float(d_lse.max()) if d_lse.size else 0.0,
            "sumexp_max_rel_err": float(s_rel.max()) if s_rel.size else 0.0}


@dataclass
class BackwardTally:
    """Accumulates dlogits accuracy over row blocks."""
    elements: int = 0
    correctly_rounded: int = 0
    max_err: float = 0.0
    max_ref: float = 0.0
    floor: float = 0.0
    notes: list = field(default_factory=list)

    def add_block(self, logits_host, targets, grad, vocab_real, vocab_padded, active,
                  ignore_index, gpu_bits, what: str = ""):
        ref = oracle.backward(logits_host, targets, grad, vocab_real, vocab_padded,
                              active=active, ignore_index=ignore_index)
        d64, rb = ref["d64"], ref["bf16"]
        gpu_bits = np.asarray(gpu_bits, dtype=np.uint16)[:, :vocab_padded]
        gv = oracle.bf16_bits_to_f64(gpu_bits)
        assert np.all(np.isfinite(gv)), what
        # padded columns and invalid rows: exactly +0
        assert np.all(gpu_bits[:, vocab_real:] == 0), what
        v = valid_rows(targets, active, vocab_real, ignore_index)
        assert np.all(gpu_bits[~v] == 0), what
        real_g, real_r, real_d = gv[:, :vocab_real], rb[:, :vocab_real], d64[:, :vocab_real]
        same = real_g == oracle.bf16_bits_to_f64(real_r)  # by value: +0 equals -0
        self.elements += real_g.size
        self.correctly_rounded += int(same.sum())
        err = np.abs(real_g - real_d)
        if err.size:
            self.max_err = max(self.max_err, float(err.max()))
            self.max_ref = max(self.max_ref, float(np.abs(real_d).max()))
            self.floor = max(self.floor,
                             float(np.abs(oracle.bf16_bits_to_f64(real_r) - real_d).max()))
        # one BF16 spacing everywhere; the target element may add 2^-20 |g|
        allow = bf16_spacing(real_d)
        y = np.asarray(targets)
        g = np.abs(np.asarray(grad, dtype=np.float64))
        rows = np.nonzero(v)[0]
        allow[rows, y[rows]] += 2.0 ** -20 * g[rows]
        bad = err > allow
        assert not bad.any(), (what, np.argwhere(bad)[:5].tolist(),
                               err[bad][:5].tolist(), allow[bad][:5].tolist())

    def finish(self, what: str = "") -> dict:
        frac = self.correctly_rounded / max(1, self.elements)
        gate = max(MAXERR_RATIO * self.max_ref, 1.01 * self.floor)
        out = {"elements": self.elements, "correctly_rounded": frac,
               "max_err": self.max_err, "max_ref": self.max_ref, "floor": self.floor,
               "max_err_over_max": self.max_err / self.max_ref if self.max_ref else 0.0,
               "floor_over_max": self.floor / self.max_ref if self.max_ref else 0.0}
        assert frac >= CORRECTLY_ROUNDED_MIN, (what, out)
        assert self.max_err <= gate, (what, out)
        return out
