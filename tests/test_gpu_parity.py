"""GPU parity: the HIP path, called through the C ABI, against the FP64 oracle.

Every case prints its name before touching the GPU.  Sizes are small enough for the
oracle to finish in seconds while still spanning several 4096-column tiles and a ragged
tail; the full-size workloads are checked on sampled rows (all rows for the forward).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst
import oracle
from parity_checks import BackwardTally, bits_of, check_forward
from workloads import headline_case, mid_case, random_case, tiny_case

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def run(case, dlogits=None):
    """Forward then backward through the C ABI; returns GPU tensors."""
    x = case.logits[:, :case.vocab_padded]
    logp, lse, stats = dst.logp_forward(x, case.targets, case.vocab_real, case.vocab_padded,
                                        active=case.active, ignore_index=case.ignore_index)
    d = dst.logp_backward(x, case.targets, case.grad, stats, case.vocab_real,
                          case.vocab_padded, active=case.active,
                          ignore_index=case.ignore_index, dlogits=dlogits)
    torch.cuda.synchronize()
    return logp, lse, stats, d


def full_check(case, rows=None, block=512):
    """Forward on every row, backward element-wise on `rows` (default: all)."""
    say(f"{case.name}: n={case.n} V={case.vocab_real} P={case.vocab_padded} ld={case.ld}")
    logp, lse, stats, d = run(case)
    host = case.logits.cpu()
    y = case.targets.cpu().numpy()
    act = None if case.active is None else case.active.cpu().numpy()
    g = case.grad.cpu().numpy()
    fwd = check_forward(host, y, case.vocab_real, act, case.ignore_index, logp.cpu().numpy(),
                        lse.cpu().numpy(), stats.cpu().numpy(), case.name)
    rows = np.arange(case.n) if rows is None else np.asarray(rows)
    tally = BackwardTally()
    for r0 in range(0, rows.size, block):
        r = rows[r0:r0 + block]
        rt = torch.from_numpy(r)
        tally.add_block(host[rt], y[r], g[r], case.vocab_real, case.vocab_padded,
                        None if act is None else act[r], case.ignore_index,
                        bits_of(d[rt.to(DEV)]), case.name)
    bwd = tally.finish(case.name)
    say(f"{case.name}: fwd {fwd} bwd {bwd}")
    return logp, lse, stats, d, fwd, bwd


# ------------------------------------------------------------------ small and tiny

def test_tiny_config():
    case = tiny_case(device=DEV)
    logp, lse, stats, d, _, _ = full_check(case)
    r_eq = case.meta["equal_row"]
    V = case.vocab_real
    # a row of equal logits gives -log V (within a few FP32 ulps of it)
    assert abs(float(logp[r_eq]) + np.log(V)) <= 2e-6
    assert float(stats[r_eq, 1]) == V
    ign = case.meta["ignored_rows"]
    assert torch.all(logp[ign] == 0) and torch.all(d[ign].view(torch.int16) == 0)


SMALL = [
    # n, vocab_real, vocab_padded, ld, sigma, pad_fill, inactive, ignore, bad targets
    (33, 10000, 10000, 10000, 3.0, float("-inf"), 0.0, 0.0, 0.0),      # ragged last tile
    (37, 10007, 10007, 10007, 3.0, float("-inf"), 0.1, 0.1, 0.1),      # odd ld: 2-byte path
    (16, 4096, 4096, 4096, 2.0, float("-inf"), 0.0, 0.0, 0.0),         # exactly one tile
    (9, 1, 1, 1, 1.0, float("-inf"), 0.0, 0.0, 0.0),                   # V = 1
    (12, 255, 255, 255, 3.0, float("-inf"), 0.0, 0.2, 0.0),
    (12, 1031, 1031, 1031, 3.0, float("-inf"), 0.0, 0.0, 0.2),
    (20, 8200, 8704, 8704, 3.0, 100.0, 0.2, 0.1, 0.15),                # padding holds +100
    (25, 12288, 16384, 16400, 3.0, 7.0, 0.0, 0.0, 0.2),                # all-padding tile
    (40, 151936, 152064, 152064, 3.0, float("-inf"), 0.05, 0.05, 0.05),  # Qwen shape
    (3, 300, 300, 300, 40.0, float("-inf"), 0.0, 0.0, 0.0),            # very spread logits
    (11, 9001, 9001, 9008, 3.0, float("-inf"), 0.1, 0.1, 0.1),         # aligned ld, odd width
    (6, 20000, 20000, 20000, 30.0, float("-inf"), 0.0, 0.0, 0.0),      # subnormal gradients
]


@pytest.mark.parametrize("spec", SMALL, ids=[f"n{s[0]}_v{s[1]}_p{s[2]}_ld{s[3]}" for s in SMALL])
def test_small_shapes(spec):
    n, v, p, ld, sigma, fill, inact, ign, bad = spec
    case = random_case(n, v, p, ld=ld, sigma=sigma, seed=n * 7 + v, pad_fill=fill,
                       inactive_frac=inact, ignore_frac=ign, bad_target_frac=bad, device=DEV)
    full_check(case)


# Widths around the two forms of the flat backward (aligned 16-bit views): below 8192
# columns a wave takes 8 vectors per lane, from 8192 on 16, so its chunk is exactly one row
# at 8192 and crosses a row boundary above it.  Row counts leave a ragged last chunk.
FLAT_WIDTHS = [(7, 4096), (5, 8184), (6, 8192), (9, 8200), (3, 24584)]


@pytest.mark.parametrize("n,v", FLAT_WIDTHS, ids=[f"n{n}_v{v}" for n, v in FLAT_WIDTHS])
def test_flat_backward_chunk_geometry(n, v):
    case = random_case(n, v, sigma=3.0, seed=n + v, inactive_frac=0.2, ignore_frac=0.1,
                       device=DEV)
    _, _, stats, d, _, _ = full_check(case)  # aligned view: flat kernel, against the oracle
    # the same rows in a view 6 bytes off alignment take the (row, tile) kernel: same bits
    buf = torch.zeros((n, v + 11), dtype=case.logits.dtype, device=DEV)
    buf[:, 3:3 + v] = case.logits
    d2 = dst.logp_backward(buf[:, 3:3 + v], case.targets, case.grad, stats, v, v,
                           active=case.active)
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int16), d2.view(torch.int16))


UNIFORM = [(1024, "bf16"), (8200, "bf16"), (151936, "bf16"), (8200, "f16"), (8200, "f32"),
           (151936, "f32")]


@pytest.mark.parametrize("v,dt", UNIFORM, ids=[f"v{v}_{dt}" for v, dt in UNIFORM])
def test_uniform_rows_gradient_bits(v, dt):
    """On a row of equal logits every exp(z - M) is exp(0) = 1 and S = V exactly, so the
    backward's bits are fixed by float32 arithmetic alone: every column gets
    round(-fl32(g / V)) and the target round(fl32(g - fl32(g / V))), rounded to nearest even
    in the logits' dtype.  Rows with a negative maximum take the general path for FP32
    logits (the fast two-sum needs M >= 0), which must give the same bits."""
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
    n = 12
    rng = np.random.default_rng(v)
    c = torch.from_numpy(rng.normal(0.0, 3.0, size=(n, 1)).astype(np.float32))
    x = c.expand(n, v).to(tdt).contiguous()
    y = rng.integers(0, v, size=n)
    g = rng.normal(0.0, 1.0, size=n).astype(np.float32)
    say(f"uniform rows: n={n} V={v} {dt}")
    logits = x.to(DEV)
    yt = torch.from_numpy(y).to(DEV)
    gt = torch.from_numpy(g).to(DEV)
    _, _, stats = dst.logp_forward_ex(logits, yt)
    d = dst.logp_backward_ex(logits, yt, gt, stats)
    torch.cuda.synchronize()
    assert torch.all(stats[:, 1].cpu() == float(v))
    neg = -(g / np.float32(v))                       # float32 division, rounded once
    at_target = (g + neg).astype(np.float32)
    want = np.repeat(neg[:, None], v, axis=1)
    want[np.arange(n), y] = at_target
    want_t = torch.from_numpy(want).to(tdt)          # round to nearest even
    assert torch.equal(d.cpu().view(torch.int16 if dt != "f32" else torch.int32),
                       want_t.view(torch.int16 if dt != "f32" else torch.int32))


def test_rows_of_minus_inf_and_masked_tails():
    n, v = 6, 9000
    x = torch.randn((n, v)) * 3
    x[0, :] = float("-inf")                     # valid row with no finite logit
    x[1, :] = float("-inf")                     # invalid row with no finite logit
    x[2, 5000:] = float("-inf")                 # -inf masked vocab tail
    x[3, :4096] = float("-inf")                 # a whole -inf tile
    x[4, 1] = 50.0                              # dominant logit
    logits = x.to(torch.bfloat16).to(DEV)
    y = torch.tensor([3, -100, 17, 5000, 1, 8999], device=DEV)
    g = torch.tensor([1.0, 1.0, -2.0, 0.5, 3.0, 1e-3], device=DEV)
    say("minus-inf rows")
    logp, lse, stats = dst.logp_forward(logits, y)
    d = dst.logp_backward(logits, y, g, stats)
    torch.cuda.synchronize()
    assert float(logp[0]) == float("-inf") and float(lse[0]) == float("-inf")
    assert float(stats[0, 0]) == float("-inf") and float(stats[0, 1]) == 0.0
    assert float(logp[1]) == 0.0 and float(lse[1]) == float("-inf")
    assert torch.all(d[:2].view(torch.int16) == 0)
    assert torch.all(torch.isfinite(d.float()))
    assert torch.all(d[2, 5000:].view(torch.int16) == 0)
    host = logits.cpu()
    check_forward(host[2:], y[2:].cpu().numpy(), v, None, -100, logp[2:].cpu().numpy(),
                  lse[2:].cpu().numpy(), stats[2:].cpu().numpy(), "minus-inf rows")
    t = BackwardTally()
    t.add_block(host[2:], y[2:].cpu().numpy(), g[2:].cpu().numpy(), v, v, None, -100,
                bits_of(d[2:]), "minus-inf rows")


DEEP_ONE = [(8192, "bf16"), (8191, "bf16"), (8192, "f16"), (8191, "f16")]


@pytest.mark.parametrize("v,dt", DEEP_ONE, ids=[f"v{v}_{dt}" for v, dt in DEEP_ONE])
def test_one_deep_value_at_every_vector_position(v, dt):
    """A row whose only logit below M - 87 (or only -inf) sits at position e = 0..7 of its
    8-element vector: the test that sends a group of vectors to the general exponential path
    must see every position.  On the fast path a -inf gives NaN and exp(z - M) below 2^-126
    flushes to zero, where the BF16 result is a subnormal (g = 256 makes g/S about 1 here).
    Width 8192 takes the flat backward, 8191 the (row, tile) kernel."""
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    n = 16
    gen = torch.Generator().manual_seed(v)
    x = torch.randn((n, v), generator=gen)
    x[:, 100] = 12.0                          # a dominant logit: M = 12, S close to 1
    cols = [8 * (37 + 3 * r) + (r % 8) for r in range(n)]
    for r, c in enumerate(cols):
        x[r, c] = float("-inf") if r >= 8 else 12.0 - 90.0
    y = torch.randint(0, v, (n,), generator=gen)
    y[3] = cols[3]                            # targets on a deep value and on a -inf
    y[12] = cols[12]
    g = torch.full((n,), 256.0)
    logits = x.to(tdt).to(DEV)
    say(f"one deep value per row: V={v} {dt}")
    _, _, stats = dst.logp_forward_ex(logits, y.to(DEV))
    d = dst.logp_backward_ex(logits, y.to(DEV), g.to(DEV), stats)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(d.float()))
    t = BackwardTally()
    gpu_vals = bits_of(d) if dt == "bf16" else d.cpu().numpy()
    t.add_block(logits.cpu(), y.numpy(), g.numpy(), v, v, None, -100, gpu_vals,
                f"one deep value, V={v} {dt}")
    t.finish(f"one deep value, V={v} {dt}")


@pytest.mark.parametrize("v", [5000, 8200, 24584])
def test_invalid_rows_do_not_read_logits(v):
    # 5000 columns: 8 vectors per lane on the flat path; 8200 and 24584: 16, with chunks that
    # start in a valid row and end in a poisoned one and the reverse
    case = random_case(8, v, sigma=3.0, seed=3, device=DEV)
    case.targets[[1, 4]] = -100
    case.active = torch.ones(8, dtype=torch.uint8, device=DEV)
    case.active[6] = 0
    say("invalid rows hold NaN logits")
    _, _, stats = dst.logp_forward(case.logits, case.targets, active=case.active)
    poisoned = case.logits.clone()
    poisoned[[1, 4, 6]] = float("nan")
    d = dst.logp_backward(poisoned, case.targets, case.grad, stats, active=case.active)
    torch.cuda.synchronize()
    assert torch.all(d[[1, 4, 6]].view(torch.int16) == 0)
    clean = dst.logp_backward(case.logits, case.targets, case.grad, stats, active=case.active)
    assert torch.equal(d.view(torch.int16), clean.view(torch.int16))


# ------------------------------------------------------------------ configured workloads

def test_mid_config():
    """N=4096, V=151936 padded to 152064 (-inf pads), 5% inactive rows, g = 1/N_active."""
    case = mid_case(device=DEV)
    full_check(case)


def test_mid_config_garbage_padding_is_masked_by_index():
    a = mid_case(device=DEV)
    b = mid_case(device=DEV, pad_fill=100.0)
    say("mid config, +100 in the padding columns")
    ra, rb = run(a), run(b)
    for u, w in zip(ra, rb):
        assert torch.equal(u.view(torch.int32) if u.dtype == torch.float32 else
                           u.view(torch.int16), w.view(torch.int32) if w.dtype == torch.float32
                           else w.view(torch.int16))


def test_headline_config_sampled():
    """N=32768, V=151936: forward checked on every row, backward on 160 sampled rows
    (all 328 spike rows' share of them included) against the oracle."""
    case = headline_case(device=DEV)
    rng = np.random.default_rng(0)
    spike = np.asarray(case.meta["spike_row_index"][:32])
    rows = np.unique(np.concatenate([rng.choice(case.n, 128, replace=False), spike,
                                     [0, case.n - 1]]))
    full_check(case, rows=rows, block=64)


def test_pages_bench_workload_sampled():
    """sigma = 1 logits, uniform targets, g = 1: the pull request's benchmark workload."""
    case = headline_case(device=DEV, n=4096, pages_bench=True)
    full_check(case, rows=np.arange(0, 4096, 64))
