"""Element-wise comparison of the GPU outputs with the FP64 oracle.

Tolerances (written here, used by every GPU parity test):
  * logp and LSE: |gpu - oracle| <= 1e-4 absolute, the bar the accuracy target sets for
    the selected-token logp.  Row max M is compared exactly (a max of BF16 values is
    exact in FP32); S to 2e-5 relative (FP32 sums of up to ~1.5e5 exp terms).
  * dlogits (BF16, and FP16 outputs of FP16 logits): at least 99.99% of all
    N x vocab_real BF16 elements equal the round-to-nearest-even of the FP64 value; for FP16
    outputs at least 1 - 2^-10 of them.  The FP32 value the kernels round carries up to
    about 4 FP32 spacings of error (g/S, the exponential, the product), so an output lands
    on the wrong side of a rounding boundary with probability up to 2 * 2^-21 / 2^-10 =
    2^-10 for FP16's 11 significant bits, and 2^-13 for BF16's 8 (FP32 outputs: every
    element within 16 FP32 spacings instead, the FP32 row sum S carrying a few spacings of
    shared error).  The number of elements that are not correctly rounded is printed for
    every case; the largest |gpu - d64| is at most
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
CORRECTLY_ROUNDED_MIN = 0.9999            # BF16 outputs
CORRECTLY_ROUNDED_MIN_F16 = 1.0 - 2.0 ** -10  # FP16 outputs (see above)
MAXERR_RATIO = 1.5e-3


def bits_of(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bits of a bf16 tensor (copied to the host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_values(t: torch.Tensor) -> np.ndarray:
    """A dlogits tensor on the host in the oracle's layout for its dtype (BF16 as bits)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return bits_of(t)
    return t.cpu().numpy()


# significant bits and smallest subnormal spacing of each output dtype
PRECISION = {"bf16": (8, 2.0 ** -133), "f16": (11, 2.0 ** -24), "f32": (24, 2.0 ** -149)}


def spacing(v: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """Spacing of representable numbers of `dtype` in the binade of |v|."""
    bits, smallest = PRECISION[dtype]
    a = np.abs(v)
    _, e = np.frexp(a)  # a = f 2^e, f in [0.5, 1)
    sp = np.ldexp(np.ones_like(a), e - bits)
    return np.maximum(sp, smallest)


def bf16_spacing(v: np.ndarray) -> np.ndarray:
    """Spacing of BF16 numbers in the binade of |v| (2^-133 in the subnormal range)."""
    return spacing(v, "bf16")


def as_f64(values: np.ndarray, dtype: str) -> np.ndarray:
    return oracle.bf16_bits_to_f64(values) if dtype == "bf16" else values.astype(np.float64)


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
    dtype: str = ""
    notes: list = field(default_factory=list)
    # count the correctly-rounded share over the non-target elements only: the target entry
    # g' (1 - p) is formed in FP32, so when p is within a few FP32 units of 1 it cancels and
    # is held to the per-element bound below instead (rows of a handful of columns with a
    # dominant target make such entries a large share of a small sample)
    cr_skip_targets: bool = False

    def add_block(self, logits_host, targets, grad, vocab_real, vocab_padded, active,
                  ignore_index, gpu_vals, what: str = "", inv_temperature: float = 1.0,
                  ulps: float = 1.0):
        """gpu_vals: dlogits on the host in the oracle's layout (BF16 as uint16 bits)."""
        ref = oracle.backward(logits_host, targets, grad, vocab_real, vocab_padded,
                              active=active, ignore_index=ignore_index,
                              inv_temperature=inv_temperature)
        d64, rb = ref["d64"], ref["rounded"]
        dt = {np.uint16: "bf16", np.float16: "f16", np.float32: "f32"}[rb.dtype.type]
        self.dtype = dt
        gpu_vals = np.asarray(gpu_vals)[:, :vocab_padded]
        assert gpu_vals.dtype == rb.dtype, (what, gpu_vals.dtype, rb.dtype)
        gv = as_f64(gpu_vals, dt)
        assert np.all(np.isfinite(gv)), what
        # padded columns and invalid rows: exactly +0
        raw = gpu_vals.view(np.uint16 if dt != "f32" else np.uint32)
        assert np.all(raw[:, vocab_real:] == 0), what
        v = valid_rows(targets, active, vocab_real, ignore_index)
        assert np.all(raw[~v] == 0), what
        real_g, real_d = gv[:, :vocab_real], d64[:, :vocab_real]
        real_r = as_f64(rb[:, :vocab_real], dt)
        same = real_g == real_r  # by value: +0 equals -0
        counted = np.ones(same.shape, dtype=bool)
        if self.cr_skip_targets:
            vr = np.nonzero(v)[0]
            counted[vr, np.asarray(targets)[vr]] = False
        self.elements += int(counted.sum())
        self.correctly_rounded += int((same & counted).sum())
        err = np.abs(real_g - real_d)
        if err.size:
            self.max_err = max(self.max_err, float(err.max()))
            self.max_ref = max(self.max_ref, float(np.abs(real_d).max()))
            self.floor = max(self.floor, float(np.abs(real_r - real_d).max()))
        # `ulps` spacings of the output dtype everywhere; the target element may add
        # 2^-20 |g * inv_temperature| (1 - p is formed in FP32)
        allow = ulps * spacing(real_d, dt)
        y = np.asarray(targets)
        g = np.abs(np.asarray(grad, dtype=np.float64)) * float(np.float32(inv_temperature))
        rows = np.nonzero(v)[0]
        allow[rows, y[rows]] += 2.0 ** -20 * g[rows]
        bad = err > allow
        assert not bad.any(), (what, np.argwhere(bad)[:5].tolist(),
                               err[bad][:5].tolist(), allow[bad][:5].tolist())

    def finish(self, what: str = "", min_correctly_rounded: float | None = None) -> dict:
        """Check the accumulated counts; the correctly-rounded bar defaults to the output
        dtype's (BF16 99.99%, FP16 1 - 2^-10, FP32 none: its per-element bound applies)."""
        if min_correctly_rounded is None:
            min_correctly_rounded = {"bf16": CORRECTLY_ROUNDED_MIN,
                                     "f16": CORRECTLY_ROUNDED_MIN_F16}.get(self.dtype, 0.0)
        frac = self.correctly_rounded / max(1, self.elements)
        gate = max(MAXERR_RATIO * self.max_ref, 1.01 * self.floor)
        out = {"elements": self.elements, "correctly_rounded": frac,
               "max_err": self.max_err, "max_ref": self.max_ref, "floor": self.floor,
               "max_err_over_max": self.max_err / self.max_ref if self.max_ref else 0.0,
               "floor_over_max": self.floor / self.max_ref if self.max_ref else 0.0}
        misrounded = self.elements - self.correctly_rounded
        out["misrounded"] = misrounded
        print(f"[tally] {what}: {misrounded} of {self.elements} {self.dtype} elements not "
              f"correctly rounded; max err / max {out['max_err_over_max']:.3e} "
              f"(floor {out['floor_over_max']:.3e})", flush=True)
        assert misrounded <= (1.0 - min_correctly_rounded) * self.elements, (what, out)
        assert self.max_err <= gate, (what, out)
        return out
