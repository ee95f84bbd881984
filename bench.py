#!/usr/bin/env python3
"""Bench of the selected-token log-probability hot path on one MI355X.

One step = the whole path over one batch: logp_forward (tile loads, masking, tile max,
tile sum-exp, selected logit, canonical merge) then logp_backward (BF16 dlogits), on the
headline workload N=32768, V=151936, BF16 logits ~ N(0, 3^2) with 1% +30 spike rows,
70% argmax / 30% uniform targets and g ~ N(0, 0.01^2).  Inputs and output buffers are
resident in HBM before the timed region; the K timed steps are bracketed by
torch.cuda.synchronize() and timed with HIP events on the stream the kernels run on.

value = algorithmic bytes of one step / step time, in GB/s:
    forward  2*N*V (logits once) + 24*N (targets, logp, LSE, stats)
    backward 2*N_valid*V (logits once) + 2*N*V (dlogits) + 20*N (targets, g, stats)
The roofline object reports the dominant kernel (the backward) against 8 TB/s.  The
cpu_baseline object times the FP64 oracle on a bounded sample of the same rows.

Extra flags: --profile-copy adds a plain device copy of known size (for scaling the
hardware byte counters), --shard-path also times logp_partials + logp_merge.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 matrix-core peak
PAGES_FWD_BWD_MS = 27.2  # fused kernel, B200, N=32768, V=151936, BF16 (context, not target)
METRIC = "fwd+bwd ms and achieved HBM GB/s (% of peak), N=32768 V=151936 BF16"
KERNEL_SOURCES = [os.path.join(ROOT, "deterministic_selected_token_amd", "csrc", f)
                  for f in ("logp_kernels.hip", "logp_device.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bwd_kernels_headline_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def algorithmic_bytes(n: int, n_valid: int, vocab_real: int, width: int, has_mask: bool,
                      elem: int = 2):
    mask = 1 if has_mask else 0
    fwd = elem * n * vocab_real + (24 + mask) * n
    bwd = elem * n_valid * vocab_real + elem * n * width + (20 + mask) * n
    return fwd, bwd


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` ("fwd" or "bwd") from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE scaled by a 4 GiB copy), or None when the kernel sources have
    changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("kernels", {}).get(kernel, {}).get("scaled_bytes_per_launch")


def git_sha() -> str:
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT,
                              capture_output=True, text=True, timeout=10).stdout.strip()
    except Exception:
        return ""


def median(xs) -> float:
    ys = sorted(xs)
    k = len(ys) // 2
    return ys[k] if len(ys) % 2 else 0.5 * (ys[k - 1] + ys[k])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, target_seconds: float) -> dict:
    """The FP64 oracle (as it stands) on a bounded sample of the workload's rows."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    n = case.n
    v = case.vocab_real

    def run(rows, nthreads=threads):
        idx = np.linspace(0, n - 1, rows).astype(np.int64)
        host = case.logits[idx].cpu()
        y = case.targets[idx].cpu().numpy()
        g = case.grad[idx].cpu().numpy()
        t0 = time.perf_counter()
        oracle.forward(host, y, v, nthreads=nthreads)
        oracle.backward(host, y, g, v, want_f64=False, want_bf16=True, nthreads=nthreads)
        return time.perf_counter() - t0

    rows = 16
    dt = run(rows)
    if dt < target_seconds / 4:
        rows = int(min(n, max(rows, rows * target_seconds / max(dt, 1e-3))))
        dt = run(rows)
    fwd_b, bwd_b = algorithmic_bytes(rows, rows, v, v, False)
    full_fwd, full_bwd = algorithmic_bytes(n, n, v, v, False)
    gbs = (fwd_b + bwd_b) / dt / 1e9
    # one thread on 256 rows of the same workload
    rows1 = min(n, 256)
    dt1 = run(rows1, nthreads=1)
    f1, b1 = algorithmic_bytes(rows1, rows1, v, v, False)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {n} rows of the same workload, FP64 forward + backward "
                      f"(dlogits rounded to BF16), {dt:.2f} s wall",
            "ms_per_step_extrapolated": round((full_fwd + full_bwd) / (gbs * 1e9) * 1e3, 1),
            "one_thread": {"value": round((f1 + b1) / dt1 / 1e9, 4), "unit": "GB/s",
                           "rows": rows1, "seconds": round(dt1, 3)},
            "cpu_model": cpu_model()}


def time_pages_bench(dst, stream, steps: int) -> dict:
    """The headline shape on the pages' own bench inputs (randn logits, sigma 1; uniform
    targets; g = 1 on every row), for comparability with their timings."""
    import torch

    from workloads import headline_case

    case = headline_case(device=torch.device("cuda", 0), pages_bench=True)
    n, v = case.n, case.vocab_real
    x, y, g = case.logits, case.targets, case.grad
    d = torch.empty((n, v), dtype=torch.bfloat16, device=x.device)
    logp = torch.empty(n, dtype=torch.float32, device=x.device)
    lse = torch.empty_like(logp)
    stats = torch.empty((n, 2), dtype=torch.float32, device=x.device)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dst.logp_forward(x, y, v, v, logp=logp, lse=lse, stats=stats, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        dst.logp_backward(x, y, g, stats, v, v, dlogits=d, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(3):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    fwd = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
    bwd = sum(b.elapsed_time(c) for _, b, c in evs) / steps
    total = evs[0][0].elapsed_time(evs[-1][2]) / steps
    fb, bb = algorithmic_bytes(n, n, v, v, False)
    del case, x, d
    return {"fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4), "ms_per_step": round(total, 4),
            "gbs": round((fb + bb) / (total * 1e-3) / 1e9, 1)}


def time_variants(dst, case, stream, steps: int) -> dict:
    """fwd / bwd times of the _ex entry points for FP16, FP32 and a temperature of 0.7 on the
    headline rows (FP16 / FP32 logits are the BF16 values widened: the same data)."""
    import torch

    out = {}
    n, v = case.n, case.vocab_real
    y, g = case.targets, case.grad
    for name, tdt, inv_t in (("f16", torch.float16, 1.0), ("f32", torch.float32, 1.0),
                             ("bf16_temperature_0.7", torch.bfloat16, 1.0 / 0.7)):
        x = case.logits if tdt == torch.bfloat16 else case.logits.to(tdt)
        d = torch.empty((n, v), dtype=tdt, device=x.device)
        logp = torch.empty(n, dtype=torch.float32, device=x.device)
        lse = torch.empty_like(logp)
        stats = torch.empty((n, 2), dtype=torch.float32, device=x.device)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            dst.logp_forward_ex(x, y, v, v, inv_temperature=inv_t, logp=logp, lse=lse,
                                stats=stats, stream=stream)
            if ev is not None:
                ev[1].record(stream)
            dst.logp_backward_ex(x, y, g, stats, v, v, inv_temperature=inv_t, dlogits=d,
                                 stream=stream)
            if ev is not None:
                ev[2].record(stream)

        for _ in range(2):
            step()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        f_ms = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
        b_ms = sum(b.elapsed_time(c) for _, b, c in evs) / steps
        fb, bb = algorithmic_bytes(n, n, v, v, False, elem=x.element_size())
        out[name] = {"fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
                     "ms_per_step": round(f_ms + b_ms, 4),
                     "gbs": round((fb + bb) / ((f_ms + b_ms) * 1e-3) / 1e9, 1),
                     "fwd_gbs": round(fb / (f_ms * 1e-3) / 1e9, 1),
                     "bwd_gbs": round(bb / (b_ms * 1e-3) / 1e9, 1)}
        del x, d
        torch.cuda.empty_cache()
    return out


def time_grpo(dst, case, stream, steps: int) -> dict:
    """The GRPO rows: (1) one GRPO training step on the headline logits viewed as 32
    sequences x 1024 tokens -- logp_forward, grpo_loss (seq_mean, KL 0.04, 10% of tokens
    masked), logp_backward fed with d loss / d logp; (2) grpo_loss alone on 1024 sequences x
    4096 tokens, against its algorithmic bytes (logp, old_logp, ref_logp 4 B, mask 1 B read
    once, dlogp 4 B written; 4 B of advantage and 16 B of sums per sequence)."""
    import torch

    from deterministic_selected_token_amd import grpo

    dev = case.logits.device
    gen = torch.Generator(device=dev).manual_seed(7)

    def inputs(B, T):
        noise = lambda: 0.05 * torch.randn((B, T), generator=gen, device=dev)
        mask = (torch.rand((B, T), generator=gen, device=dev) >= 0.1).to(torch.uint8)
        adv = grpo.grpo_advantages(torch.randn(B, generator=gen, device=dev), 8)
        return noise, mask, adv

    def timed(fn):
        for _ in range(2):
            fn()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for e in evs:
            fn(e)
        torch.cuda.synchronize()
        a = sum(x.elapsed_time(y) for x, y, _ in evs) / steps
        b = sum(y.elapsed_time(z) for _, y, z in evs) / steps
        return a, b

    out = {}
    n, v = case.n, case.vocab_real
    B, T = 32, n // 32
    x, y = case.logits, case.targets
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse, stats = torch.empty_like(logp), torch.empty((n, 2), dtype=torch.float32, device=dev)
    d = torch.empty((n, v), dtype=torch.bfloat16, device=dev)
    dst.logp_forward(x, y, logp=logp, lse=lse, stats=stats, stream=stream)
    noise, mask, adv = inputs(B, T)
    old = (logp.view(B, T) + noise()).contiguous()
    ref = (logp.view(B, T) + noise()).contiguous()
    seq_stats = torch.empty((B, 4), dtype=torch.int32, device=dev)
    loss = torch.empty(6, dtype=torch.int64, device=dev)
    dlogp = torch.empty((B, T), dtype=torch.float32, device=dev)

    def step(ev=None):
        dst.logp_forward(x, y, logp=logp, lse=lse, stats=stats, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        grpo.grpo_loss(logp.view(B, T), old, adv, ref_logp=ref, mask=mask, mode="seq_mean",
                       beta=0.04, seq_stats=seq_stats, loss=loss, dlogp=dlogp, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        dst.logp_backward(x, y, dlogp.view(-1), stats, dlogits=d, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    for e in evs:
        e[3].record(stream)
        step(e)
    torch.cuda.synchronize()
    total = sum(e[3].elapsed_time(e[2]) for e in evs) / steps
    loss_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    out["grpo_step_headline"] = {"sequences": B, "tokens_per_sequence": T,
                                 "ms_per_step": round(total, 4), "grpo_loss_ms": round(loss_ms, 4),
                                 "loss": grpo.loss_fields(loss)["loss"]}
    del d
    torch.cuda.empty_cache()

    B, T = 1024, 4096
    noise, mask, adv = inputs(B, T)
    lp = -1.0 - torch.rand((B, T), generator=gen, device=dev)
    old, ref = lp + noise(), lp + noise()
    seq_stats = torch.empty((B, 4), dtype=torch.int32, device=dev)
    dlogp = torch.empty((B, T), dtype=torch.float32, device=dev)

    def loss_only(ev=None):
        if ev is not None:
            ev[0].record(stream)
        grpo.grpo_loss(lp, old, adv, ref_logp=ref, mask=mask, mode="token_mean", beta=0.04,
                       seq_stats=seq_stats, loss=loss, dlogp=dlogp, stream=stream)
        if ev is not None:
            ev[1].record(stream)
            ev[2].record(stream)

    ms, _ = timed(loss_only)
    nbytes = B * T * (4 * 3 + 1 + 4) + B * (4 + 16) + 48
    out["grpo_loss_1024x4096"] = {"ms": round(ms, 4), "algorithmic_bytes": nbytes,
                                  "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                  "launches": 4, "cpu_baseline": grpo_oracle_rate(
                                      lp, old, ref, adv, mask, nbytes)}
    return out


def grpo_oracle_rate(lp, old, ref, adv, mask, nbytes: int) -> dict:
    """The float64 GRPO oracle on the same tokens (numpy, as it stands), timed on the host."""
    from oracle import grpo_oracle

    host = [t.cpu().numpy() for t in (lp, old, ref, adv, mask)]
    t0 = time.perf_counter()
    grpo_oracle.loss(*host, mode="token_mean", beta=0.04)
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "kind": "oracle",
            "sample": f"all {lp.numel()} tokens, float64 numpy, {dt:.2f} s wall", "cores": 1}


def time_linear(dst, stream, steps: int, n: int = 8192, hidden: int = 4096,
                vocab: int = 151936, inv_temperature: float = 1.0,
                cpu_baseline: bool = True) -> dict:
    """linear_logp forward (linear_logp_partials + logp_merge) on n rows of a Qwen3-8B-shaped
    LM head (hidden 4096, vocabulary 151936), logits scored at inv_temperature: 2 n V H flops
    on the matrix cores."""
    import torch

    from deterministic_selected_token_amd import linear

    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(11)
    h = torch.randn((n, hidden), generator=gen, device=dev).to(torch.bfloat16)
    W = (torch.randn((vocab, hidden), generator=gen, device=dev) * (3.0 / hidden ** 0.5)) \
        .to(torch.bfloat16)
    y = torch.randint(0, vocab, (n,), generator=gen, device=dev)
    L = dst.logp_num_tiles(vocab)
    partials = torch.empty((n, L, 3), dtype=torch.float32, device=dev)
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse, stats = torch.empty_like(logp), torch.empty((n, 2), dtype=torch.float32, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        linear.linear_logp_partials(h, W, y, vocab, vocab, 0, vocab, partials, stream=stream,
                                    inv_temperature=inv_temperature)
        if ev is not None:
            ev[1].record(stream)
        dst.logp_merge(partials, y, vocab, logp=logp, lse=lse, stats=stats, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    k_ms = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
    m_ms = sum(b.elapsed_time(c) for _, b, c in evs) / steps
    flops = 2.0 * n * vocab * hidden
    out = {"rows": n, "hidden": hidden, "vocab": vocab, "inv_temperature": inv_temperature,
           "partials_ms": round(k_ms, 4), "merge_ms": round(m_ms, 4),
           "tflops": round(flops / (k_ms * 1e-3) / 1e12, 1),
           "frac_of_bf16_peak": round(flops / (k_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    if not cpu_baseline:
        return out
    # the float64 oracle on a few of the same rows (numpy float64 matmul + the C log-softmax)
    from oracle import linear_oracle

    rows = 4
    h_host, w_host, y_host = h[:rows].cpu(), W.cpu(), y[:rows].cpu().numpy()
    t0 = time.perf_counter()
    linear_oracle.forward(h_host, w_host, y_host, vocab, inv_temperature=inv_temperature)
    dt = time.perf_counter() - t0
    out["cpu_baseline"] = {
        "value": round(2.0 * rows * vocab * hidden / dt / 1e12, 4), "unit": "TFLOP/s",
        "kind": "oracle", "cores": len(os.sched_getaffinity(0)),
        "sample": f"{rows} of the {n} rows, float64 logits and log-softmax, {dt:.2f} s wall "
                  "(including the float64 copy of W)"}
    return out


def time_linear_backward(dst, stream, steps: int, n: int = 8192, hidden: int = 4096,
                         vocab: int = 151936, chunk_cols: int = 16384) -> dict:
    """linear_logp backward on the same LM-head shape: dz recomputed (2 n V H flops), then
    dh = dz W and dW = dz^T h (2 n V H flops each), 6 n V H flops per call."""
    import torch

    from deterministic_selected_token_amd import linear

    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(12)
    h = torch.randn((n, hidden), generator=gen, device=dev).to(torch.bfloat16)
    W = (torch.randn((vocab, hidden), generator=gen, device=dev) * (3.0 / hidden ** 0.5)) \
        .to(torch.bfloat16)
    y = torch.randint(0, vocab, (n,), generator=gen, device=dev)
    g = torch.randn((n,), generator=gen, device=dev) * 0.01
    _, _, stats = linear.linear_logp_forward(h, W, y, vocab, vocab, stream=stream)
    dh = torch.empty((n, hidden), dtype=torch.float32, device=dev)
    dW = torch.empty((vocab, hidden), dtype=torch.float32, device=dev)
    ws = torch.empty(linear.linear_logp_backward_workspace(n, hidden, chunk_cols),
                     dtype=torch.uint8, device=dev)

    def step():
        linear.linear_logp_backward(h, W, y, g, stats, vocab, vocab, chunk_cols=chunk_cols,
                                    dhidden=dh, dweight=dW, workspace=ws, stream=stream)

    step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    flops = 6.0 * n * vocab * hidden
    del h, W, dW, ws
    # the float64 oracle on a bounded sample: 4 rows against the first 16384 vocabulary rows
    import numpy as np

    from oracle import linear_oracle

    rows, cols = 4, 16384
    gen_c = torch.Generator().manual_seed(12)
    hs = torch.randn((rows, hidden), generator=gen_c).to(torch.bfloat16)
    Ws = (torch.randn((cols, hidden), generator=gen_c) * (3.0 / hidden ** 0.5)).to(torch.bfloat16)
    t0 = time.perf_counter()
    linear_oracle.backward(hs, Ws, np.arange(rows), np.ones(rows, dtype=np.float32), cols)
    dt = time.perf_counter() - t0
    cpu = {"value": round(6.0 * rows * cols * hidden / dt / 1e12, 4), "unit": "TFLOP/s",
           "kind": "oracle", "cores": len(os.sched_getaffinity(0)),
           "sample": f"{rows} rows x {cols} vocabulary rows, float64 dz, dh and dW, "
                     f"{dt:.2f} s wall"}
    return {"rows": n, "hidden": hidden, "vocab": vocab, "chunk_cols": chunk_cols,
            "ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "workspace_bytes": linear.linear_logp_backward_workspace(n, hidden, chunk_cols),
            "cpu_baseline": cpu}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample (0 disables it)")
    ap.add_argument("--shard-path", action="store_true",
                    help="also time logp_partials (4 shards) + logp_merge")
    ap.add_argument("--variants", action="store_true",
                    help="also time FP16 and FP32 logits and BF16 at temperature 0.7 on the "
                         "same shape, the same shape on the pages' bench inputs (sigma 1, "
                         "g = 1), a GRPO step and the GRPO loss alone (reported under "
                         "config.variants)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="run a 4 GiB device copy after the timed region (counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the path "
              "shards by rows, or by vocabulary tiles with one all-gather of the per-tile "
              "partials, and a several-GPU run is not part of this benchmark",
              file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: run as a single process (WORLD_SIZE > 1 is not supported)",
              file=sys.stderr)
        return 2

    import torch

    import deterministic_selected_token_amd as dst
    from workloads import headline_case

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print("bench: generating the headline workload", file=sys.stderr, flush=True)
    case = headline_case(device=dev)
    n, v = case.n, case.vocab_real
    x, y, g = case.logits, case.targets, case.grad
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    stats = torch.empty((n, 2), dtype=torch.float32, device=dev)
    dlogits = torch.empty((n, v), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dst.logp_forward(x, y, v, v, logp=logp, lse=lse, stats=stats, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        dst.logp_backward(x, y, g, stats, v, v, dlogits=dlogits, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # peak memory of one step beyond the resident inputs and preallocated outputs: zero
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    free_before = torch.cuda.mem_get_info(dev)[0]  # hipMemGetInfo: device-wide free bytes
    step()
    torch.cuda.synchronize()
    step_extra = torch.cuda.max_memory_allocated() - base
    free_change = free_before - torch.cuda.mem_get_info(dev)[0]

    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd_ms = [a.elapsed_time(b) for a, b, _ in evs]
    bwd_ms = [b.elapsed_time(c) for _, b, c in evs]
    total_ms = evs[0][0].elapsed_time(evs[-1][2]) / args.steps

    n_valid = n  # every headline row is active with an in-range target
    fwd_b, bwd_b = algorithmic_bytes(n, n_valid, v, v, False)
    value = (fwd_b + bwd_b) / (total_ms * 1e-3) / 1e9
    bwd_avg = sum(bwd_ms) / len(bwd_ms)
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    achieved = bwd_b / (bwd_avg * 1e-3) / 1e9

    extra = {}
    if args.shard_path:
        L = dst.logp_num_tiles(v)
        partials = torch.empty((n, L, 3), dtype=torch.float32, device=dev)
        layout = [(0, 13 * 4096), (13 * 4096, 26 * 4096), (26 * 4096, v)]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for rep in range(2):
            e[0].record(stream)
            for c0, c1 in layout:
                dst.logp_partials(x[:, c0:c1], y, v, v, c0, c1, partials, stream=stream)
            e[1].record(stream)
            dst.logp_merge(partials, y, v, stream=stream)
            e[2].record(stream)
        torch.cuda.synchronize()
        extra["shard_path"] = {"shards": len(layout),
                               "partials_ms": round(e[0].elapsed_time(e[1]), 4),
                               "merge_ms": round(e[1].elapsed_time(e[2]), 4)}
    if args.variants:
        extra["variants"] = time_variants(dst, case, stream, args.steps)
        extra["variants"]["bf16_pages_bench_inputs"] = time_pages_bench(dst, stream, args.steps)
        extra["variants"].update(time_grpo(dst, case, stream, args.steps))
        extra["variants"]["linear_logp_fwd"] = time_linear(dst, stream, max(3, args.steps // 4))
        extra["variants"]["linear_logp_fwd_temperature_0.7"] = time_linear(
            dst, stream, max(3, args.steps // 4), inv_temperature=1 / 0.7, cpu_baseline=False)
        extra["variants"]["linear_logp_bwd"] = time_linear_backward(
            dst, stream, max(2, args.steps // 8))
    if args.profile_copy:
        src = torch.empty(1 << 31, dtype=torch.int16, device=dev)  # 4 GiB
        dst_buf = torch.empty_like(src)
        dst_buf.copy_(src)
        torch.cuda.synchronize()
        extra["copy_bytes_each_way"] = src.numel() * 2

    cpu = None
    if args.cpu_seconds > 0:
        print("bench: timing the oracle sample on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(case, args.cpu_seconds)

    props = torch.cuda.get_device_properties(dev)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(PAGES_FWD_BWD_MS / total_ms, 3),
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "headline: N=32768 V=151936 bf16 logits ~N(0,3^2), 1% +30 "
                               "spike rows, targets 70% argmax / 30% uniform, g ~N(0,0.01^2)",
                   "n": n, "vocab": v, "logits_dtype": "bf16", "grad_dtype": "bf16",
                   "fwd_ms": round(fwd_avg, 4), "bwd_ms": round(bwd_avg, 4),
                   "wall_ms_per_step": round(wall_ms, 4),
                   "median_ms": {"fwd": round(median(fwd_ms), 4),
                                 "bwd": round(median(bwd_ms), 4),
                                 "step": round(median([f + b for f, b in zip(fwd_ms, bwd_ms)]),
                                               4)},
                   "algorithmic_bytes": {"fwd": fwd_b, "bwd": bwd_b},
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "step_extra_bytes_beyond_outputs": int(step_extra),
                   "device_free_bytes_change_over_step": int(free_change),
                   # the pages' peak-memory figure: from before the step, the returned BF16
                   # gradient included
                   "peak_gib_incl_returned_grad": round(
                       (step_extra + dlogits.numel() * dlogits.element_size()) / 2**30, 3),
                   "device": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                   "torch": torch.__version__, "hip": torch.version.hip, "git": git_sha(),
                   "vs_baseline_basis": "27.2 ms / ms_per_step: the pages' fused kernel, "
                                        "forward + backward at 32768 x 151936 BF16 on one "
                                        "B200 (randn logits, g = 1; the timing does not "
                                        "depend on the values); context, not a target",
                   **extra},
        "roofline": {"bound": "hbm", "kernel": "bwd_flat_kernel (logp_backward)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("bwd"),
                     "algorithmic_bytes_per_launch": bwd_b,
                     "avg_launch_ms": round(bwd_avg, 4),
                     "fwd_kernel": {"achieved": round(fwd_b / (fwd_avg * 1e-3) / 1e9, 2),
                                    "avg_launch_ms": round(fwd_avg, 4),
                                    "algorithmic_bytes_per_launch": fwd_b,
                                    "traffic": measured_traffic("fwd")}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
