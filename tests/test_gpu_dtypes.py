"""FP16 / FP32 logits and temperature-scaled scoring on the GPU (the _ex entry points).

The fused-backward pull request checks FP32, BF16 and FP16 logits against an FP64
reference at V = 1, 255, 1031 and 151936 (its Tests section); the provider experiment in
its author reply scores at temperatures 1.0 and 0.7.  Scored logits are
z = fl32(x * inv_temperature); dlogits = inv_temperature * g * (onehot - softmax(z)) in the
logits' dtype.  Tolerances: logp / LSE 1e-4 absolute; BF16 and FP16 dlogits at least 99.99%
correctly rounded and every element within one spacing of the output dtype; FP32 dlogits
within 16 FP32 spacings (the FP32 row sum S alone carries a few).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst
from parity_checks import BackwardTally, check_forward, host_values
from workloads import random_case

pytestmark = pytest.mark.gpu
DEV = "cuda"
T = dst.TILE_COLS
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    view = {4: torch.int32, 2: torch.int16}[a.element_size()]
    return a.shape == b.shape and torch.equal(a.contiguous().view(view), b.contiguous().view(view))


def case_in(dtype: str, n, v, p=None, ld=None, sigma=3.0, seed=0, **kw):
    """random_case with its logits carried over to `dtype` (FP16 / FP32 values that are
    exactly the BF16 ones would not exercise the extra precision, so FP16/FP32 logits are
    drawn again in their own dtype from the same seed)."""
    c = random_case(n, v, p, ld=ld, sigma=sigma, seed=seed, **kw)
    if dtype != "bf16":
        gen = torch.Generator().manual_seed(seed + 12345)
        z = torch.randn((n, v), generator=gen) * sigma
        buf = torch.full((n, c.ld), kw.get("pad_fill", float("-inf")), dtype=TDT[dtype])
        buf[:, :v] = z.to(TDT[dtype])
        c.logits = buf
    return c.to(DEV)


def check_ex(case, inv_t=1.0, rows=None, ulps=1.0, min_cr=None, cr_skip_targets=False):
    x = case.logits[:, :case.vocab_padded]
    logp, lse, stats = dst.logp_forward_ex(x, case.targets, case.vocab_real, case.vocab_padded,
                                           active=case.active, inv_temperature=inv_t)
    d = dst.logp_backward_ex(x, case.targets, case.grad, stats, case.vocab_real,
                             case.vocab_padded, active=case.active, inv_temperature=inv_t)
    torch.cuda.synchronize()
    host = case.logits.cpu()
    y = case.targets.cpu().numpy()
    act = None if case.active is None else case.active.cpu().numpy()
    g = case.grad.cpu().numpy()
    rows = np.arange(case.n) if rows is None else np.asarray(rows)
    rt = torch.from_numpy(rows)
    fwd = check_forward_scaled(host[rt], y[rows], case.vocab_real, None if act is None
                               else act[rows], logp.cpu().numpy()[rows],
                               lse.cpu().numpy()[rows], stats.cpu().numpy()[rows], inv_t)
    t = BackwardTally(cr_skip_targets=cr_skip_targets)
    t.add_block(host[rt], y[rows], g[rows], case.vocab_real, case.vocab_padded,
                None if act is None else act[rows], -100, host_values(d[rt.to(DEV)]),
                case.name, inv_temperature=inv_t, ulps=ulps)
    bwd = t.finish(case.name, min_correctly_rounded=min_cr)
    return (logp, lse, stats, d), fwd, bwd


def check_forward_scaled(host, y, v, act, logp, lse, stats, inv_t):
    import oracle
    ref = oracle.forward(host, y, v, active=act, inv_temperature=inv_t)
    fin = np.isfinite(ref["lse"])
    assert np.abs(logp.astype(np.float64) - ref["logp"])[np.isfinite(ref["logp"])].max(
        initial=0.0) <= 1e-4
    assert np.abs(lse.astype(np.float64)[fin] - ref["lse"][fin]).max(initial=0.0) <= 1e-4
    assert np.array_equal(stats[:, 0].astype(np.float64), ref["max"])
    return {"logp_max_abs_err": float(np.abs(logp - ref["logp"])[np.isfinite(ref["logp"])]
                                      .max(initial=0.0))}


# ------------------------------------------------------------------ parity

DT_SHAPES = [(6, 1), (12, 255), (9, 1031), (16, 10000), (24, 151936)]


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("n,v", DT_SHAPES, ids=[f"v{v}" for _, v in DT_SHAPES])
def test_fp16_fp32_logits_parity(dtype, n, v):
    case = case_in(dtype, n, v, seed=v % 97, ignore_frac=0.1, bad_target_frac=0.1)
    say(f"{dtype} logits n={n} V={v}")
    ulps, min_cr = (16.0, 0.0) if dtype == "f32" else (1.0, None)
    _, fwd, bwd = check_ex(case, ulps=ulps, min_cr=min_cr)
    say(f"{dtype} V={v}: {fwd} {bwd}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("inv_t", [1.0 / 0.7, 0.5, 2.0])
def test_temperature_parity(dtype, inv_t):
    case = case_in(dtype, 20, 12345, 12800, sigma=2.0, seed=7, pad_fill=50.0,
                   inactive_frac=0.1, ignore_frac=0.1)
    say(f"{dtype} logits, inv_temperature={inv_t:.4f}")
    ulps, min_cr = (16.0, 0.0) if dtype == "f32" else (1.0, None)
    _, fwd, bwd = check_ex(case, inv_t=inv_t, ulps=ulps, min_cr=min_cr)
    say(f"{dtype} inv_t={inv_t:.4f}: {fwd} {bwd}")


def test_temperature_headline_shape_sampled():
    """N=4096 rows of Qwen width at temperature 0.7, sampled rows against the oracle."""
    case = case_in("bf16", 4096, 151936, seed=3)
    say("bf16, V=151936, temperature 0.7")
    _, fwd, bwd = check_ex(case, inv_t=float(np.float32(1.0) / np.float32(0.7)),
                           rows=np.arange(0, 4096, 97))
    say(f"temperature 0.7: {fwd} {bwd}")


# ------------------------------------------------------------------ bitwise contract

def test_ex_at_bf16_unit_temperature_equals_plain_entry_points():
    case = case_in("bf16", 40, 20000, 20480, seed=11, pad_fill=9.0, inactive_frac=0.2,
                   ignore_frac=0.1)
    say("_ex(bf16, 1.0) vs plain")
    a = dst.logp_forward(case.logits, case.targets, case.vocab_real, case.vocab_padded,
                         active=case.active)
    b = dst.logp_forward_ex(case.logits, case.targets, case.vocab_real, case.vocab_padded,
                            active=case.active, inv_temperature=1.0)
    assert all(same_bits(u, w) for u, w in zip(a, b))
    da = dst.logp_backward(case.logits, case.targets, case.grad, a[2], case.vocab_real,
                           case.vocab_padded, active=case.active)
    db = dst.logp_backward_ex(case.logits, case.targets, case.grad, a[2], case.vocab_real,
                              case.vocab_padded, active=case.active, inv_temperature=1.0)
    assert same_bits(da, db)


@pytest.mark.parametrize("dtype,inv_t", [("f16", 1.0), ("f32", 1.0), ("bf16", 1 / 0.7),
                                         ("f32", 0.5)])
def test_shards_merge_to_forward_ex_bitwise(dtype, inv_t):
    n, vr, vp = 64, 151936, 159744
    case = case_in(dtype, n, vr, vp, seed=13)
    say(f"shards {dtype} inv_t={inv_t:.3f}")
    ref = dst.logp_forward_ex(case.logits, case.targets, vr, vp, inv_temperature=inv_t)
    L = dst.logp_num_tiles(vp)
    for layout in ([39], [20, 19], [13, 13, 12, 1]):
        partials = torch.full((n, L, 3), float("nan"), dtype=torch.float32, device=DEV)
        c0 = 0
        for tiles in layout:
            c1 = min(vp, c0 + tiles * T)
            dst.logp_partials_ex(case.logits[:, c0:c1], case.targets, vr, vp, c0, c1, partials,
                                 inv_temperature=inv_t)
            c0 = c1
        got = dst.logp_merge(partials, case.targets, vr)
        assert all(same_bits(u, w) for u, w in zip(ref, got)), layout
    # padding invariance
    unpadded = case.logits[:, :vr].contiguous()
    got = dst.logp_forward_ex(unpadded, case.targets, vr, vr, inv_temperature=inv_t)
    assert all(same_bits(u, w) for u, w in zip(ref, got))


@pytest.mark.parametrize("dtype,inv_t", [("f16", 1.0), ("f32", 1.0), ("f32", 1 / 0.7),
                                         ("f16", 2.0)])
def test_batch_chunking_and_load_paths_bitwise(dtype, inv_t):
    case = case_in(dtype, 50, 10000, seed=17, inactive_frac=0.2)
    say(f"chunking / load paths {dtype} inv_t={inv_t:.3f}")

    def run(x, y, g, a):
        lp, ls, st = dst.logp_forward_ex(x, y, active=a, inv_temperature=inv_t)
        d = dst.logp_backward_ex(x, y, g, st, active=a, inv_temperature=inv_t)
        return lp, ls, st, d

    ref = run(case.logits, case.targets, case.grad, case.active)
    for chunk in (1, 7):
        for r0 in range(0, 50, chunk):
            s = slice(r0, min(50, r0 + chunk))
            got = run(case.logits[s], case.targets[s], case.grad[s], case.active[s])
            assert all(same_bits(u[s], w) for u, w in zip(ref, got)), chunk
    # misaligned view (element-wise loads, tile path) vs aligned (16-byte loads, flat path)
    buf = torch.zeros((50, 10013), dtype=case.logits.dtype, device=DEV)
    buf[:, 3:10003] = case.logits
    got = run(buf[:, 3:10003], case.targets, case.grad, case.active)
    assert all(same_bits(u, w) for u, w in zip(ref, got))


def test_subnormal_gradients_fp16_and_fp32():
    for dtype in ("f16", "f32"):
        case = case_in(dtype, 6, 20000, sigma=30.0, seed=19)
        say(f"{dtype} very spread logits")
        ulps, min_cr = (16.0, 0.0) if dtype == "f32" else (1.0, None)
        check_ex(case, ulps=ulps, min_cr=min_cr)


@pytest.mark.parametrize("dtype,inv_t", [("f32", 1.0), ("bf16", 1 / 0.7), ("f16", 0.5),
                                         ("f32", 2.0)])
def test_negative_max_and_wide_rows(dtype, inv_t):
    """Rows whose scored max is negative, and rows where most scored logits lie below -M:
    there z - M needs the general two-sum (FP32 logits, scaled logits)."""
    case = case_in(dtype, 16, 20000, sigma=3.0, seed=23)
    x = case.logits
    gen = torch.Generator().manual_seed(29)
    x[0:6, :20000] = (x[0:6, :20000].float() - 40.0).to(x.dtype)
    x[6:12, :20000] = (torch.rand((6, 20000), generator=gen) * 22.0 - 20.0).to(x.dtype).to(DEV)
    x[12, :20000] = (torch.rand(20000, generator=gen) * 0.5 - 0.25).to(x.dtype).to(DEV)
    say(f"negative max / wide rows {dtype} inv_t={inv_t:.3f}")
    ulps, min_cr = (16.0, 0.0) if dtype == "f32" else (1.0, None)
    _, fwd, bwd = check_ex(case, inv_t=inv_t, ulps=ulps, min_cr=min_cr)
    say(f"{dtype} inv_t={inv_t:.3f}: {fwd} {bwd}")
