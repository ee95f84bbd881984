"""Seeded synthetic workloads for the selected-token log-probability path.

Every workload is a batch of BF16 logits ``[n, ld]`` (row-major, ``ld >= vocab_padded``),
int64 targets ``[n]``, an optional uint8 active mask ``[n]`` and an FP32 upstream
gradient ``[n]`` (dL/dlogp per row).  Only input generation lives here: no max,
sum-exp, softmax or gradient arithmetic.

Recipes (all seeded).  FP32 samples are rounded to BF16 with round-to-nearest-even
(``torch.Tensor.to(torch.bfloat16)``).  Small cases are drawn on the CPU with numpy's
PCG64; the large cases are drawn on the requested device with a seeded
``torch.Generator`` in row chunks so the FP32 staging stays bounded.

* tiny      N=64, V=1024, logits ~ N(0, 2^2); targets uniform; 8 rows with target -100;
            one row of equal logits; one row with a +40 spike; g ~ N(0, 1).  Seed 0.
* mid       N=4096, V_real=151936 padded to 152064 (pad columns -inf, or +100 garbage
            to prove that masking is by index); logits ~ N(0, 3^2); targets uniform
            with row 0 -> 0 and row 1 -> V_real-1; 205 inactive rows; g = fl32(1/3891).
* headline  N=32768, V=151936, logits ~ N(0, 3^2); 328 rows (1%) with +30 added at one
            uniformly chosen column; targets 70% argmax (lowest index on ties) / 30%
            uniform; g ~ N(0, 0.01^2).  The ``pages_bench`` variant uses N(0, 1) logits,
            uniform targets and g = 1, the workload of the benchmark script printed with
            the fused-backward pull request (its "Benchmark script" section).
* shard     N=8192, V_real=151936, V_padded=ld=159744 (39 tiles of 4096, the last one
            all padding), pad columns -inf, logits ~ N(0, 3^2), uniform targets,
            g ~ N(0, 1).
* sweep     8 probe rows and a pool of 2048 filler rows at V=151936, logits ~ N(0, 3^2),
            uniform targets, g ~ N(0, 1); seeds 0, 1, 2.
* long      N=131072 rows at V=151936, logits ~ N(0, 3^2), uniform targets, g ~ N(0, 1).
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

IGNORE_INDEX = -100
QWEN_VOCAB = 151936

# Batch sizes of the batch-invariance sweep: 1..9, then 2^k-1, 2^k, 2^k+1 for
# k = 4..10, then 2047 and 2048 ("up to 2048").
SWEEP_SIZES = tuple(list(range(1, 10))
                    + [s for k in range(4, 11) for s in (2 ** k - 1, 2 ** k, 2 ** k + 1)]
                    + [2047, 2048])


def sweep_positions(batch: int) -> list[int]:
    """Front, middle and back slot of a batch, deduplicated, in that order."""
    out: list[int] = []
    for p in (0, batch // 2, batch - 1):
        if p not in out:
            out.append(p)
    return out


@dataclass
class Case:
    name: str
    logits: torch.Tensor            # [n, ld] bfloat16, row-major
    targets: torch.Tensor           # [n] int64
    active: Optional[torch.Tensor]  # [n] uint8 or None (= every row active)
    grad: torch.Tensor              # [n] float32, dL/dlogp
    vocab_real: int
    vocab_padded: int
    ignore_index: int = IGNORE_INDEX
    meta: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.logits.shape[0])

    @property
    def ld(self) -> int:
        return int(self.logits.stride(0))

    def to(self, device) -> "Case":
        return Case(self.name, self.logits.to(device), self.targets.to(device),
                    None if self.active is None else self.active.to(device),
                    self.grad.to(device), self.vocab_real, self.vocab_padded,
                    self.ignore_index, dict(self.meta))


def _bf16_from_f32(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def case_digest(case: Case) -> str:
    """sha256 over the raw bytes of every input array (determinism pin)."""
    h = hashlib.sha256()
    lg = case.logits.detach().cpu().contiguous()
    h.update(lg.view(torch.int16).numpy().tobytes())
    h.update(case.targets.detach().cpu().numpy().astype("<i8").tobytes())
    if case.active is not None:
        h.update(case.active.detach().cpu().numpy().astype("u1").tobytes())
    h.update(case.grad.detach().cpu().numpy().astype("<f4").tobytes())
    return h.hexdigest()


# --------------------------------------------------------------------------- tiny

def tiny_case(device="cpu", seed: int = 0) -> Case:
    rng = np.random.Generator(np.random.PCG64(seed))
    n, v = 64, 1024
    x = rng.normal(0.0, 2.0, size=(n, v)).astype(np.float32)
    targets = rng.integers(0, v, size=n, dtype=np.int64)
    ignored = np.sort(rng.choice(n, 8, replace=False))
    targets[ignored] = IGNORE_INDEX
    kept = np.setdiff1d(np.arange(n), ignored)
    r_equal, r_spike = (int(r) for r in rng.permutation(kept)[:2])
    x[r_equal, :] = np.float32(rng.normal(0.0, 2.0))
    spike_col = int(rng.integers(0, v))
    x[r_spike, spike_col] += np.float32(40.0)
    grad = rng.normal(0.0, 1.0, size=n).astype(np.float32)
    logits = _bf16_from_f32(torch.from_numpy(x))
    case = Case("tiny", logits, torch.from_numpy(targets), None,
                torch.from_numpy(grad), v, v,
                meta={"ignored_rows": ignored.tolist(), "equal_row": r_equal,
                      "spike_row": r_spike, "spike_col": spike_col, "seed": seed})
    return case.to(device) if str(device) != "cpu" else case


# ---------------------------------------------------------------- device helpers

def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal_bf16_rows(n: int, cols: int, ld: int, sigma: float, gen: torch.Generator,
                      device, chunk_bytes: int = 1 << 30) -> torch.Tensor:
    """[n, ld] bf16 buffer whose first ``cols`` columns hold bf16(N(0, sigma^2))."""
    out = torch.empty((n, ld), dtype=torch.bfloat16, device=device)
    rows = max(1, chunk_bytes // (4 * cols))
    for r0 in range(0, n, rows):
        r1 = min(n, r0 + rows)
        z = torch.randn((r1 - r0, cols), generator=gen, device=device, dtype=torch.float32)
        if sigma != 1.0:
            z.mul_(sigma)
        out[r0:r1, :cols] = _bf16_from_f32(z)
        del z
    return out


# ---------------------------------------------------------------------------- mid

def mid_case(device="cuda", seed: int = 1, pad_fill: float = float("-inf")) -> Case:
    n, v_real, v_pad = 4096, QWEN_VOCAB, 152064
    gen = _gen(device, seed)
    logits = _normal_bf16_rows(n, v_real, v_pad, 3.0, gen, device)
    logits[:, v_real:] = pad_fill
    targets = torch.randint(0, v_real, (n,), generator=gen, device=device, dtype=torch.int64)
    targets[0] = 0
    targets[1] = v_real - 1
    n_inactive = 205
    perm = torch.randperm(n - 2, generator=gen, device=device) + 2
    active = torch.ones(n, dtype=torch.uint8, device=device)
    active[perm[:n_inactive]] = 0
    n_active = n - n_inactive
    g = torch.full((n,), float(np.float32(1.0) / np.float32(n_active)), dtype=torch.float32,
                   device=device)
    return Case("mid", logits, targets, active, g, v_real, v_pad,
                meta={"seed": seed, "pad_fill": pad_fill, "n_active": n_active})


# ----------------------------------------------------------------------- headline

def headline_case(device="cuda", seed: int = 2, n: int = 32768, vocab: int = QWEN_VOCAB,
                  pages_bench: bool = False) -> Case:
    gen = _gen(device, seed)
    if pages_bench:
        logits = _normal_bf16_rows(n, vocab, vocab, 1.0, gen, device)
        targets = torch.randint(0, vocab, (n,), generator=gen, device=device, dtype=torch.int64)
        g = torch.ones(n, dtype=torch.float32, device=device)
        return Case("headline_pages_bench", logits, targets, None, g, vocab, vocab,
                    meta={"seed": seed, "sigma": 1.0})
    # logits ~ N(0, 9); 1% of rows get +30 at one column (added in FP32 before rounding)
    n_spike = max(1, round(0.01 * n))
    spike_rows = torch.randperm(n, generator=gen, device=device)[:n_spike]
    spike_cols = torch.randint(0, vocab, (n_spike,), generator=gen, device=device)
    logits = torch.empty((n, vocab), dtype=torch.bfloat16, device=device)
    rows_per_chunk = max(1, (1 << 30) // (4 * vocab))
    is_spike = torch.zeros(n, dtype=torch.bool, device=device)
    is_spike[spike_rows] = True
    spike_col_of = torch.full((n,), -1, dtype=torch.int64, device=device)
    spike_col_of[spike_rows] = spike_cols
    for r0 in range(0, n, rows_per_chunk):
        r1 = min(n, r0 + rows_per_chunk)
        z = torch.randn((r1 - r0, vocab), generator=gen, device=device, dtype=torch.float32)
        z.mul_(3.0)
        local = torch.nonzero(is_spike[r0:r1]).flatten()
        if local.numel():
            z[local, spike_col_of[r0 + local]] += 30.0
        logits[r0:r1] = _bf16_from_f32(z)
        del z
    # targets: 70% argmax (torch.argmax returns the lowest index among ties), 30% uniform
    take_argmax = torch.rand((n,), generator=gen, device=device) < 0.7
    uniform = torch.randint(0, vocab, (n,), generator=gen, device=device, dtype=torch.int64)
    amax = torch.empty(n, dtype=torch.int64, device=device)
    for r0 in range(0, n, rows_per_chunk):
        r1 = min(n, r0 + rows_per_chunk)
        amax[r0:r1] = torch.argmax(logits[r0:r1].float(), dim=1)
    targets = torch.where(take_argmax, amax, uniform)
    g = torch.randn((n,), generator=gen, device=device, dtype=torch.float32) * 0.01
    return Case("headline", logits, targets, None, g, vocab, vocab,
                meta={"seed": seed, "sigma": 3.0, "spike_rows": n_spike,
                      "spike_row_index": sorted(spike_rows.cpu().tolist())})


# -------------------------------------------------------------------------- shard

def shard_case(device="cuda", seed: int = 3, n: int = 8192) -> Case:
    v_real, v_pad = QWEN_VOCAB, 159744
    gen = _gen(device, seed)
    logits = _normal_bf16_rows(n, v_real, v_pad, 3.0, gen, device)
    logits[:, v_real:] = float("-inf")
    targets = torch.randint(0, v_real, (n,), generator=gen, device=device, dtype=torch.int64)
    g = torch.randn((n,), generator=gen, device=device, dtype=torch.float32)
    return Case("shard", logits, targets, None, g, v_real, v_pad, meta={"seed": seed})


# --------------------------------------------------------------------------- long

def long_case(device="cuda", seed: int = 77, n: int = 131072, vocab: int = QWEN_VOCAB) -> Case:
    """The extreme row count: n rows at the Qwen vocabulary, logits ~ N(0, 3^2), uniform
    targets, g ~ N(0, 1) (39.8 GB of BF16 logits at n = 131072)."""
    gen = _gen(device, seed)
    logits = _normal_bf16_rows(n, vocab, vocab, 3.0, gen, device)
    targets = torch.randint(0, vocab, (n,), generator=gen, device=device, dtype=torch.int64)
    g = torch.randn((n,), generator=gen, device=device, dtype=torch.float32)
    return Case("long", logits, targets, None, g, vocab, vocab, meta={"seed": seed})


# -------------------------------------------------------------------------- sweep

def sweep_probe_rows(device="cuda", seed: int = 0, probes: int = 8,
                     vocab: int = QWEN_VOCAB) -> Case:
    gen = _gen(device, 1000 + seed)
    logits = _normal_bf16_rows(probes, vocab, vocab, 3.0, gen, device)
    targets = torch.randint(0, vocab, (probes,), generator=gen, device=device, dtype=torch.int64)
    g = torch.randn((probes,), generator=gen, device=device, dtype=torch.float32)
    return Case(f"sweep_probes_s{seed}", logits, targets, None, g, vocab, vocab,
                meta={"seed": seed})


def sweep_filler_rows(device="cuda", seed: int = 0, rows: int = 2048,
                      vocab: int = QWEN_VOCAB) -> Case:
    gen = _gen(device, 2000 + seed)
    logits = _normal_bf16_rows(rows, vocab, vocab, 3.0, gen, device)
    targets = torch.randint(0, vocab, (rows,), generator=gen, device=device, dtype=torch.int64)
    g = torch.randn((rows,), generator=gen, device=device, dtype=torch.float32)
    return Case(f"sweep_filler_s{seed}", logits, targets, None, g, vocab, vocab,
                meta={"seed": seed})


# ------------------------------------------------------------------------- random

def random_case(n: int, vocab_real: int, vocab_padded: Optional[int] = None,
                ld: Optional[int] = None, sigma: float = 3.0, seed: int = 0, device="cpu",
                pad_fill: float = float("-inf"), inactive_frac: float = 0.0,
                ignore_frac: float = 0.0, bad_target_frac: float = 0.0,
                grad_std: float = 1.0) -> Case:
    """General small case for parity tests (drawn on the CPU, then moved).

    ``bad_target_frac`` replaces that share of targets by out-of-range or padded-column
    indices (vocab_real, vocab_real+5, vocab_padded-1 when padded, or -7).
    """
    vocab_padded = vocab_real if vocab_padded is None else vocab_padded
    ld = vocab_padded if ld is None else ld
    assert ld >= vocab_padded >= vocab_real >= 1
    gen = torch.Generator().manual_seed(seed)
    z = torch.randn((n, vocab_real), generator=gen, dtype=torch.float32) * sigma
    buf = torch.full((n, ld), pad_fill, dtype=torch.bfloat16)
    buf[:, :vocab_real] = _bf16_from_f32(z)
    targets = torch.randint(0, vocab_real, (n,), generator=gen, dtype=torch.int64)
    u = torch.rand((n,), generator=gen)
    if ignore_frac > 0:
        targets[u < ignore_frac] = IGNORE_INDEX
    if bad_target_frac > 0:
        bad = (u >= ignore_frac) & (u < ignore_frac + bad_target_frac)
        choices = [vocab_real, vocab_real + 5, -7]
        if vocab_padded > vocab_real:
            choices.append(vocab_padded - 1)
        idx = torch.nonzero(bad).flatten()
        for j, r in enumerate(idx.tolist()):
            targets[r] = choices[j % len(choices)]
    active = None
    if inactive_frac > 0:
        active = (torch.rand((n,), generator=gen) >= inactive_frac).to(torch.uint8)
    g = torch.randn((n,), generator=gen, dtype=torch.float32) * grad_std
    case = Case(f"random_n{n}_v{vocab_real}_p{vocab_padded}_ld{ld}_s{seed}", buf, targets,
                active, g, vocab_real, vocab_padded, meta={"seed": seed, "sigma": sigma})
    return case.to(device) if str(device) != "cpu" else case
