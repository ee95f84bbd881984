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
The roofline object reports the dominant kernel (the backward) against 8 TB/s and against
the measured copy ceiling, the forward against 8 TB/s and the measured read ceiling (plain
read and copy kernels of tests/probes/hbm_ceiling.hip, timed in the same run).

Also in the default run, each under config: batch invariance of headline rows recomputed in
smaller batches; one tensor-parallel rank's share (5 of 38 tiles of the headline rows);
the mid-size workload (N=4096, padded vocabulary, 5% inactive rows); the vocab-shard
workload (N=8192, 39 tiles, 1/2/4 shards + merge against the fused forward); N=131072; and
the headline shape on the pages' bench inputs (sigma 1, g = 1); and linear_logp (forward and
BF16 backward at 8192 x 4096 x 151936, against the matrix-core ceiling measured in the same
run).  The oracle leg runs the
FP64 oracle on the headline rows and on the pages' inputs, compares the GPU's logp, LSE
and dlogits with it block by block (top-level "accuracy") and reports its own rate
("cpu_baseline").

Extra flags: --headline-only (the timed headline step alone), --variants (FP16, FP32,
temperature, GRPO, linear_logp, the matrix-core and LDS probes), --profile-copy (a 4 GiB copy of known size at the end, for
scaling the hardware byte counters).
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


CEILING_LIB = os.path.join(ROOT, "tests", "probes", "libhbm_ceiling.so")
# (vectors of 16 bytes per lane, waves per workgroup); the forward's pattern is 8 vectors in
# 4-wave workgroups, the backward's 16 vectors in 16-wave workgroups; smaller read footprints
# (2 or 4 vectors) read about 1% faster
READ_SHAPES = ((2, 4), (4, 8), (8, 4), (16, 4), (16, 16), (32, 8))
COPY_SHAPES = ((8, 16), (16, 16), (16, 8), (32, 8))
MFMA_CEILING_LIB = os.path.join(ROOT, "tests", "probes", "libmfma_ceiling.so")
LDS_CEILING_LIB = os.path.join(ROOT, "tests", "probes", "liblds_ceiling.so")


def load_ceiling_library():
    import ctypes

    lib = ctypes.CDLL(CEILING_LIB)  # built by __graft_entry__.build() with the test probes
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.hbm_read.argtypes = [P, I64, I32, I32, ctypes.c_uint32, P, P]
    lib.hbm_read.restype = I32
    lib.hbm_copy.argtypes = [P, P, I64, I32, I32, P]
    lib.hbm_copy.restype = I32
    lib.hbm_copy_nt.argtypes = [P, P, I64, P]
    lib.hbm_copy_nt.restype = I32
    lib.hbm_write.argtypes = [P, I64, ctypes.c_uint32, P]
    lib.hbm_write.restype = I32
    return lib


def hbm_ceiling(stream, gib: int = 10, reps: int = 6) -> dict:
    """Measured HBM ceilings: a plain streaming read of `gib` GiB and a plain copy of `gib`
    GiB each way (tests/probes/hbm_ceiling.hip, non-temporal 16-byte loads, the backward's
    `sc1 nt` 16-byte stores), in several wave shapes; GB/s counts the bytes read (read) or
    read + written (copy).  Beside them, for the record: a write-only fill (`write_gbs`) and
    the backward's copy shape with non-temporal-only stores."""
    import torch

    lib = load_ceiling_library()
    dev = torch.device("cuda", 0)
    nbytes = gib << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.view(torch.int32).random_()
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    h = stream.cuda_stream

    def timed(call) -> float:
        for _ in range(2):
            call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        return median([a.elapsed_time(b) for a, b in evs])

    def check(rc: int):
        if rc != 0:
            raise RuntimeError(f"hbm ceiling probe failed ({rc})")

    out = {"read_gbs": 0.0, "copy_gbs": 0.0, "write_gbs": 0.0, "bytes": nbytes,
           "kernels": "tests/probes/hbm_ceiling.hip (hbm_read, hbm_copy, hbm_copy_nt, "
                      "hbm_write)", "shapes": {}}
    for nv, waves in READ_SHAPES:
        ms = timed(lambda: check(lib.hbm_read(src.data_ptr(), nbytes, nv, waves, 0x9E3779B9,
                                              sink.data_ptr(), h)))
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["shapes"][f"read {nv} KiB/wave, {waves} waves/group"] = round(gbs, 1)
        out["read_gbs"] = max(out["read_gbs"], round(gbs, 1))
    for nv, waves in COPY_SHAPES:
        ms = timed(lambda: check(lib.hbm_copy(src.data_ptr(), dst.data_ptr(), nbytes, nv, waves,
                                              h)))
        gbs = 2 * nbytes / (ms * 1e-3) / 1e9
        out["shapes"][f"copy {nv} KiB/wave, {waves} waves/group"] = round(gbs, 1)
        out["copy_gbs"] = max(out["copy_gbs"], round(gbs, 1))
    ms = timed(lambda: check(lib.hbm_copy_nt(src.data_ptr(), dst.data_ptr(), nbytes, h)))
    out["shapes"]["copy 16 KiB/wave, 16 waves/group, nt-only stores"] = \
        round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    ms = timed(lambda: check(lib.hbm_write(dst.data_ptr(), nbytes, 0x5BD1E995, h)))
    out["write_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    out["shapes"]["write 16 KiB/wave, 16 waves/group"] = out["write_gbs"]
    del src, dst
    torch.cuda.empty_cache()
    return out


def mfma_ceiling(stream, reps: int = 5) -> dict:
    """Measured dense BF16 matrix-core ceiling (tests/probes/mfma_ceiling.hip): chains of
    independent v_mfma_f32_32x32x16_bf16 on register operands whose bits keep changing (the
    ceiling), and on fixed operands (`static_operands`: less switching, less power, a higher
    clock), no memory traffic, 1024 workgroups of the two wave shapes of the linear_logp
    kernels, about 6 ms per launch; TFLOP/s of the median launch."""
    import ctypes

    import torch

    lib = ctypes.CDLL(MFMA_CEILING_LIB)  # built by __graft_entry__.build() with the probes
    lib.mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                              ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.mfma_bf16.restype = ctypes.c_int
    lib.mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    lib.mfma_bf16_flops.restype = ctypes.c_double
    dev = torch.device("cuda", 0)
    groups, iters = 1024, 5000
    out = {"tflops": 0.0, "static_operands_tflops": 0.0,
           "kernel": "tests/probes/mfma_ceiling.hip (mfma_bf16)", "shapes": {}}
    for waves, toggle in ((4, 1), (8, 1), (4, 0), (8, 0)):
        sink = torch.empty(groups * waves * 64, dtype=torch.float32, device=dev)

        def call(seed):
            if lib.mfma_bf16(waves, groups, iters, seed, toggle, sink.data_ptr(),
                             stream.cuda_stream):
                raise RuntimeError("mfma ceiling probe failed")

        call(1)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            call(2 + i)
            b.record(stream)
        torch.cuda.synchronize()
        ms = median([a.elapsed_time(b) for a, b in evs])
        tf = lib.mfma_bf16_flops(waves, groups, iters) / (ms * 1e-3) / 1e12
        out["shapes"][f"{waves} waves/group, {'128 x 128' if waves == 4 else '64 x 128'} "
                      f"per wave, {'switching' if toggle else 'fixed'} operands"] = round(tf, 1)
        key = "tflops" if toggle else "static_operands_tflops"
        out[key] = max(out[key], round(tf, 1))
    return out


def lds_rates(stream, groups: int = 256) -> dict:
    """Per-CU LDS rates in bytes per core clock (tests/probes/lds_ceiling.hip; one workgroup
    per CU, cycles read in the kernel with s_memtime, median over the workgroups): LDS reads of
    4, 8 and 16 bytes per lane (the block product's fragment reads are 16-byte), and
    direct-to-LDS buffer loads from a 2 MiB source that stays in L2 (the block product's stage
    loads), with a workgroup on every CU and on one CU in eight (the L2 of each XCD is shared by
    its CUs)."""
    import ctypes

    import torch

    lib = ctypes.CDLL(LDS_CEILING_LIB)  # built by __graft_entry__.build() with the probes
    lib.lds_read.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.lds_read.restype = ctypes.c_int
    lib.lds_dma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.lds_dma.restype = ctypes.c_int
    lib.lds_read_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.lds_read_bytes.restype = ctypes.c_double
    lib.lds_dma_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.lds_dma_bytes.restype = ctypes.c_double
    dev = torch.device("cuda", 0)
    sink = torch.empty(groups * 16 * 64, dtype=torch.int32, device=dev)
    cycles = torch.empty(groups, dtype=torch.int64, device=dev)
    src = torch.randint(0, 256, (2 << 20,), dtype=torch.uint8, device=dev)
    out = {"kernels": "tests/probes/lds_ceiling.hip (lds_read, lds_dma)",
           "unit": "bytes per core clock per CU", "read": {}, "dma_from_l2": {}}

    def median_rate(call, nbytes, g=groups):
        for _ in range(2):  # the second launch is the one read
            if call():
                raise RuntimeError("lds probe failed")
        torch.cuda.synchronize()
        return round(nbytes / float(cycles[:g].double().median().item()), 1)

    for width in (4, 8, 16):
        for waves in (4, 8, 16):
            iters = 16000 // waves
            rate = median_rate(
                lambda: lib.lds_read(waves, groups, iters, width, sink.data_ptr(),
                                     cycles.data_ptr(), stream.cuda_stream),
                lib.lds_read_bytes(waves, iters, width))
            out["read"][f"{width}-byte reads, {waves} waves"] = rate
    for g in (groups, groups // 8):  # every CU loading, or one in eight
        for waves in (4, 8):
            iters = 4000 // waves

            def call():
                return lib.lds_dma(waves, g, iters, src.data_ptr(), src.numel(),
                                   sink.data_ptr(), cycles.data_ptr(), stream.cuda_stream)

            rate = median_rate(call, lib.lds_dma_bytes(waves, iters), g)
            out["dma_from_l2"][f"{waves} waves, {g} workgroups"] = rate
    return out


def vendor_gemm_reference(stream, reps: int = 7, n: int = 8192, hidden: int = 4096,
                          vocab: int = 151936) -> dict:
    """Context, not part of the path: the unfused logits GEMM h W^T -> BF16 [n, V] through
    torch.matmul (hipBLASLt) on the linear_logp shape; it forms and writes the logits and does
    no reduction.  Its choice of kernel, and so its summation order, may change with n."""
    import torch

    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(11)
    h = torch.randn((n, hidden), generator=gen, device=dev).to(torch.bfloat16)
    W = (torch.randn((vocab, hidden), generator=gen, device=dev) * (3.0 / hidden ** 0.5)) \
        .to(torch.bfloat16)
    out = torch.empty((n, vocab), dtype=torch.bfloat16, device=dev)
    with torch.cuda.stream(stream):
        for _ in range(2):
            torch.matmul(h, W.t(), out=out)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            torch.matmul(h, W.t(), out=out)
            b.record(stream)
    torch.cuda.synchronize()
    ms = median([a.elapsed_time(b) for a, b in evs])
    del h, W, out
    torch.cuda.empty_cache()
    return {"what": "torch.matmul(h, W.t()) -> bf16 logits (hipBLASLt), unfused, no reduction",
            "rows": n, "hidden": hidden, "vocab": vocab, "ms": round(ms, 4),
            "tflops": round(2.0 * n * vocab * hidden / (ms * 1e-3) / 1e12, 1)}


def n_valid_rows(case) -> int:
    """Rows that are active and whose target lies in [0, vocab_real), not ignore_index."""
    import torch

    y = case.targets
    ok = (y >= 0) & (y < case.vocab_real) & (y != case.ignore_index)
    if case.active is not None:
        ok &= case.active != 0
    return int(torch.count_nonzero(ok))


def time_case(dst, case, stream, steps: int, warmup: int = 2, keep: bool = False) -> dict:
    """Forward + backward of a workload through the library, HIP events on the launch
    stream; algorithmic bytes count the logits once for the forward and once (valid rows)
    for the backward, plus the dlogits write."""
    import torch

    n, v, p = case.n, case.vocab_real, case.vocab_padded
    x = case.logits[:, :p]
    dev = x.device
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty_like(logp)
    stats = torch.empty((n, 2), dtype=torch.float32, device=dev)
    d = torch.empty((n, p), dtype=x.dtype, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        dst.logp_forward(x, case.targets, v, p, active=case.active, logp=logp, lse=lse,
                         stats=stats, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        dst.logp_backward(x, case.targets, case.grad, stats, v, p, active=case.active,
                          dlogits=d, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    f_ms = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
    b_ms = sum(b.elapsed_time(c) for _, b, c in evs) / steps
    total = evs[0][0].elapsed_time(evs[-1][2]) / steps
    fb, bb = algorithmic_bytes(n, n_valid_rows(case), v, p, case.active is not None)
    out = {"n": n, "vocab_real": v, "vocab_padded": p, "fwd_ms": round(f_ms, 4),
           "bwd_ms": round(b_ms, 4), "ms_per_step": round(total, 4),
           "algorithmic_bytes": {"fwd": fb, "bwd": bb},
           "gbs": round((fb + bb) / (total * 1e-3) / 1e9, 1),
           "fwd_gbs": round(fb / (f_ms * 1e-3) / 1e9, 1),
           "bwd_gbs": round(bb / (b_ms * 1e-3) / 1e9, 1),
           "frac_of_hbm_peak": round((fb + bb) / (total * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "floor_ms_at_8tbs": round((fb + bb) / (HBM_PEAK_GBS * 1e9) * 1e3, 3)}
    if keep:
        out["_outputs"] = (logp, lse, stats, d)
    return out


SHARD_LAYOUTS = {1: (39,), 2: (20, 19), 4: (13, 13, 12, 1)}


def time_shard_config(dst, stream, steps: int) -> dict:
    """The vocab-parallel path on one GPU: N=8192 rows, vocabulary 151936 padded to 159744
    (39 tiles, the last all padding), logp_partials over 1, 2 and 4 tile-aligned shards
    (the last 4-shard slice is the all-padding identity) + logp_merge, against the fused
    forward; the outputs must be bitwise equal."""
    import torch

    from workloads import shard_case

    case = shard_case(device=torch.device("cuda", 0))
    n, v, p = case.n, case.vocab_real, case.vocab_padded
    x, y = case.logits, case.targets
    L = dst.logp_num_tiles(p)

    def timed(fn, reps):
        fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / reps

    ref = dst.logp_forward(x, y, v, p, stream=stream)
    fused_ms = timed(lambda: dst.logp_forward(x, y, v, p, logp=ref[0], lse=ref[1],
                                              stats=ref[2], stream=stream), steps)
    fused_bytes = 2 * n * v + 24 * n
    out = {"workload": "N=8192, vocabulary 151936 padded to 159744 (39 tiles), BF16 "
                       "~N(0,3^2), uniform targets",
           "fused_forward": {"ms": round(fused_ms, 4),
                             "gbs": round(fused_bytes / (fused_ms * 1e-3) / 1e9, 1)}}
    partials = torch.empty((n, L, 3), dtype=torch.float32, device=x.device)
    for k, tiles in SHARD_LAYOUTS.items():
        bounds, t0 = [], 0
        for t in tiles:
            bounds.append((t0 * dst.TILE_COLS, min((t0 + t) * dst.TILE_COLS, p)))
            t0 += t
        got = [torch.empty_like(r) for r in ref]

        def shards():
            for c0, c1 in bounds:
                dst.logp_partials(x[:, c0:c1], y, v, p, c0, c1, partials, stream=stream)

        def merge():
            dst.logp_merge(partials, y, v, logp=got[0], lse=got[1], stats=got[2],
                           stream=stream)

        part_ms = timed(shards, steps)
        merge_ms = timed(merge, steps)
        torch.cuda.synchronize()
        same = all(torch.equal(a.view(torch.int32), b.view(torch.int32))
                   for a, b in zip(ref, got))
        part_bytes = 2 * n * v + 12 * n * L + 8 * n * k
        out[f"k{k}"] = {"tiles": list(tiles), "partials_ms": round(part_ms, 4),
                        "merge_ms": round(merge_ms, 4),
                        "ms": round(part_ms + merge_ms, 4),
                        "partials_gbs": round(part_bytes / (part_ms * 1e-3) / 1e9, 1),
                        "bitwise_equal_to_fused": bool(same)}
    del case, x, partials
    torch.cuda.empty_cache()
    return out


def time_tp8_share(dst, case, stream, steps: int) -> dict:
    """One rank's share at tensor-parallel degree 8 over the headline rows: 5 of the 38
    tiles (20480 columns) of all 32768 rows, held contiguously as a rank holds its shard,
    reduced to its partials by logp_partials."""
    import torch

    n, v = case.n, case.vocab_real
    c1 = 5 * dst.TILE_COLS
    xs = case.logits[:, :c1].contiguous()
    partials = torch.empty((n, dst.logp_num_tiles(v), 3), dtype=torch.float32,
                           device=xs.device)

    def run():
        dst.logp_partials(xs, case.targets, v, v, 0, c1, partials, stream=stream)

    run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    nbytes = 2 * n * c1 + 12 * n * 5 + 8 * n
    del xs, partials
    torch.cuda.empty_cache()
    return {"rows": n, "tiles": 5, "columns": c1, "ms": round(ms, 4),
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def batch_invariance(dst, case, outputs, stream) -> dict:
    """Rows of the headline batch recomputed inside smaller batches (the first B rows, for
    B = 1, 9, 129, 1025), compared bit for bit with the full batch's logp and dlogits."""
    import torch

    logp, _, _, d = outputs
    v = case.vocab_real
    diff_logp = diff_d = rows = 0
    for b in (1, 9, 129, 1025):
        x = case.logits[:b].clone()
        lp, _, st = dst.logp_forward(x, case.targets[:b], v, v, stream=stream)
        db = dst.logp_backward(x, case.targets[:b], case.grad[:b], st, v, v, stream=stream)
        torch.cuda.synchronize()
        diff_logp += int((lp.view(torch.int32) != logp[:b].view(torch.int32)).sum())
        diff_d += int((db.view(torch.int16) != d[:b].view(torch.int16)).any(1).sum())
        rows += b
    return {"sub_batches": [1, 9, 129, 1025], "rows_compared": rows,
            "logp_rows_differing": diff_logp, "dlogits_rows_differing": diff_d}


def _pcts(err) -> dict:
    import numpy as np

    e = np.asarray(err, dtype=np.float64)
    if e.size == 0:
        return {"max": 0.0, "p99": 0.0, "p95": 0.0}
    return {"max": float(e.max()), "p99": float(np.percentile(e, 99)),
            "p95": float(np.percentile(e, 95))}


def _compare_dlogits(gpu_bits, d64, rounded, threads: int):
    """(elements, correctly rounded, max |gpu - d64|, max |d64|, max |RNE(d64) - d64|) of
    BF16 dlogits blocks; ±0 count as equal.  Row chunks go to a thread pool (numpy releases
    the GIL in these loops)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    def part(rs):
        g, r, x = gpu_bits[rs], rounded[rs], d64[rs]
        same = (g == r) | (((g | r) & 0x7FFF) == 0)
        gv = (g.astype(np.uint32) << 16).view(np.float32)
        rv = (r.astype(np.uint32) << 16).view(np.float32)
        return (g.size, int(same.sum()), float(np.abs(gv - x).max()),
                float(np.abs(x).max()), float(np.abs(rv - x).max()))

    rows = gpu_bits.shape[0]
    step = max(1, -(-rows // threads))
    with ThreadPoolExecutor(max_workers=threads) as pool:
        parts = list(pool.map(part, [slice(i, i + step) for i in range(0, rows, step)]))
    return (sum(p[0] for p in parts), sum(p[1] for p in parts), max(p[2] for p in parts),
            max(p[3] for p in parts), max(p[4] for p in parts))


def oracle_leg(case, outputs, bwd_rows: int, threads: int, block: int = 512) -> dict:
    """The FP64 oracle (as it stands) on the same inputs, compared with the GPU's outputs as
    it goes: the forward on every row, the backward on `bwd_rows` evenly spaced rows (plus
    every spike row of the headline workload), block by block.  Returns the oracle's wall
    times and the accuracy of the GPU outputs against it."""
    import numpy as np
    import torch

    import oracle

    logp_g, lse_g, _, d_g = outputs
    n, v = case.n, case.vocab_real
    y_all = case.targets.cpu().numpy()
    g_all = case.grad.cpu().numpy()
    logp_h = logp_g.cpu().numpy().astype(np.float64)
    lse_h = lse_g.cpu().numpy().astype(np.float64)
    # forward on every row
    t_fwd = 0.0
    d_logp, d_lse = [], []
    for r0 in range(0, n, 4 * block):
        idx = torch.arange(r0, min(n, r0 + 4 * block), device=case.logits.device)
        host = case.logits[idx].cpu()
        rows = idx.cpu().numpy()
        t0 = time.perf_counter()
        ref = oracle.forward(host, y_all[rows], v, nthreads=threads)
        t_fwd += time.perf_counter() - t0
        fin = np.isfinite(ref["logp"])
        d_logp.append(np.abs(logp_h[rows][fin] - ref["logp"][fin]))
        d_lse.append(np.abs(lse_h[rows] - ref["lse"]))
    # backward on a sample of rows
    spikes = case.meta.get("spike_row_index", [])
    sample = np.unique(np.concatenate([np.linspace(0, n - 1, bwd_rows).astype(np.int64),
                                       np.asarray(spikes, dtype=np.int64)]))
    t_bwd = 0.0
    tot = [0, 0, 0.0, 0.0, 0.0]
    for r0 in range(0, sample.size, block):
        rows = sample[r0:r0 + block]
        idx = torch.from_numpy(rows).to(case.logits.device)
        host = case.logits[idx].cpu()
        gpu_bits = d_g[idx].view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        ref = oracle.backward(host, y_all[rows], g_all[rows], v, want_f64=True,
                              want_bf16=True, nthreads=threads)
        t_bwd += time.perf_counter() - t0
        e, c, me, mr, fl = _compare_dlogits(gpu_bits[:, :v], ref["d64"][:, :v],
                                            ref["bf16"][:, :v], threads)
        tot[0] += e
        tot[1] += c
        tot[2], tot[3], tot[4] = max(tot[2], me), max(tot[3], mr), max(tot[4], fl)
    elements, correct, max_err, max_ref, floor = tot
    acc = {"rows_forward": n, "rows_backward": int(sample.size),
           "logp_abs_err": _pcts(np.concatenate(d_logp)),
           "lse_abs_err": _pcts(np.concatenate(d_lse)),
           "dlogits": {"elements": elements,
                       "correctly_rounded_pct": round(100.0 * correct / max(1, elements), 5),
                       "misrounded": elements - correct,
                       "max_err": max_err, "max_ref": max_ref, "floor": floor,
                       "max_err_over_max": max_err / max_ref if max_ref else 0.0,
                       "floor_over_max": floor / max_ref if max_ref else 0.0,
                       "max_err_over_floor": max_err / floor if floor else 0.0}}
    return {"fwd_seconds": t_fwd, "bwd_seconds": t_bwd, "fwd_rows": n,
            "bwd_rows": int(sample.size), "accuracy": acc}


def cpu_baseline(leg: dict, case, threads: int) -> dict:
    """Rate of the oracle legs (forward on every row, backward on the sample) under the
    same byte accounting as the GPU, plus a one-thread rate on 256 rows."""
    import numpy as np

    import oracle

    v = case.vocab_real
    fwd_b, _ = algorithmic_bytes(leg["fwd_rows"], leg["fwd_rows"], v, v, False)
    _, bwd_b = algorithmic_bytes(leg["bwd_rows"], leg["bwd_rows"], v, v, False)
    secs = leg["fwd_seconds"] + leg["bwd_seconds"]
    gbs = (fwd_b + bwd_b) / secs / 1e9
    full_fwd, full_bwd = algorithmic_bytes(case.n, case.n, v, v, False)
    rows1 = min(case.n, 256)
    idx = np.linspace(0, case.n - 1, rows1).astype(np.int64)
    host = case.logits[idx].cpu()
    y = case.targets[idx].cpu().numpy()
    g = case.grad[idx].cpu().numpy()
    t0 = time.perf_counter()
    oracle.forward(host, y, v, nthreads=1)
    oracle.backward(host, y, g, v, want_f64=False, want_bf16=True, nthreads=1)
    dt1 = time.perf_counter() - t0
    f1, b1 = algorithmic_bytes(rows1, rows1, v, v, False)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the same workload: FP64 forward on all {leg['fwd_rows']} rows "
                      f"({leg['fwd_seconds']:.2f} s) and FP64 backward on {leg['bwd_rows']} "
                      f"rows ({leg['bwd_seconds']:.2f} s), each compared with the GPU's "
                      "outputs block by block (comparison time excluded)",
            "ms_per_step_extrapolated": round((full_fwd + full_bwd) / (gbs * 1e9) * 1e3, 1),
            "one_thread": {"value": round((f1 + b1) / dt1 / 1e9, 4), "unit": "GB/s",
                           "rows": rows1, "seconds": round(dt1, 3)},
            "cpu_model": cpu_model()}


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
    4096 tokens (token_mean with a local normalizer: 4 launches), against its algorithmic
    bytes (logp, old_logp, ref_logp 4 B, mask 1 B read once, dlogp 4 B written; 4 B of
    advantage and 16 B of sums per sequence): calls issued back to back (GPU time per call,
    and the host's time per call through the Python binding), and one call bracketed on an
    idle GPU (which includes the host's launch work)."""
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

    single_ms, _ = timed(loss_only)
    # back to back, as a training loop issues them: the host runs ahead of the GPU, so the
    # per-call time is the GPU's (the bracketed single call above includes the host's work)
    calls = max(50, 10 * steps)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(calls):
        loss_only()
    b.record(stream)
    host_us = (time.perf_counter() - t0) / calls * 1e6
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / calls
    nbytes = B * T * (4 * 3 + 1 + 4) + B * (4 + 16) + 48
    out["grpo_loss_1024x4096"] = {"ms": round(ms, 4), "algorithmic_bytes": nbytes,
                                  "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                  "calls_back_to_back": calls,
                                  "host_us_per_call": round(host_us, 1),
                                  "ms_single_call_idle_gpu": round(single_ms, 4),
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
    """linear_logp forward (linear_logp_partials with its balancing workspace + logp_merge) on
    n rows of a Qwen3-8B-shaped LM head (hidden 4096, vocabulary 151936), logits scored at
    inv_temperature: 2 n V H flops on the matrix cores."""
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
    # the balanced launch (last rounds spread over every CU; the same bits)
    ws = torch.empty(linear.linear_logp_partials_workspace(n, vocab, 0, vocab),
                     dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        linear.linear_logp_partials(h, W, y, vocab, vocab, 0, vocab, partials, stream=stream,
                                    inv_temperature=inv_temperature, workspace=ws)
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
           "partials_workspace_bytes": ws.numel(),
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


def time_linear_shard(dst, stream, steps: int, n: int = 8192, hidden: int = 4096,
                      vocab: int = 151936, tiles: int = 5) -> dict:
    """linear_logp_partials of one tensor-parallel rank's share at degree 8 (5 of the 38
    4096-column tiles of W, 160 (row block, tile) workgroups for 256 CUs), with and without the
    balancing workspace (the same bits): ms and TFLOP/s of each."""
    import torch

    from deterministic_selected_token_amd import linear

    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(13)
    width = tiles * dst.TILE_COLS
    h = torch.randn((n, hidden), generator=gen, device=dev).to(torch.bfloat16)
    W = (torch.randn((width, hidden), generator=gen, device=dev) * (3.0 / hidden ** 0.5)) \
        .to(torch.bfloat16)
    y = torch.randint(0, vocab, (n,), generator=gen, device=dev)
    partials = torch.empty((n, dst.logp_num_tiles(vocab), 3), dtype=torch.float32, device=dev)
    ws = torch.empty(linear.linear_logp_partials_workspace(n, vocab, 0, width),
                     dtype=torch.uint8, device=dev)
    flops = 2.0 * n * width * hidden
    out = {"rows": n, "hidden": hidden, "columns": width, "tiles": tiles}
    for key, workspace in (("balanced", ws), ("one_launch", None)):
        def call():
            linear.linear_logp_partials(h, W, y, vocab, vocab, 0, width, partials,
                                        stream=stream, workspace=workspace)
        call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        ms = median([a.elapsed_time(b) for a, b in evs])
        out[key] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
    del h, W, ws
    torch.cuda.empty_cache()
    return out


def time_linear_backward(dst, stream, steps: int, n: int = 8192, hidden: int = 4096,
                         vocab: int = 151936, chunk_cols: int = 16384, out_dtype=None,
                         cpu_baseline: bool = True) -> dict:
    """linear_logp backward on the same LM-head shape: dz recomputed (2 n V H flops), then
    dh = dz W and dW = dz^T h (2 n V H flops each), 6 n V H flops per call; dh and dW written
    in ``out_dtype`` (float32, or bfloat16 by linear_logp_backward_bf16)."""
    import torch

    from deterministic_selected_token_amd import linear

    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(12)
    h = torch.randn((n, hidden), generator=gen, device=dev).to(torch.bfloat16)
    W = (torch.randn((vocab, hidden), generator=gen, device=dev) * (3.0 / hidden ** 0.5)) \
        .to(torch.bfloat16)
    y = torch.randint(0, vocab, (n,), generator=gen, device=dev)
    g = torch.randn((n,), generator=gen, device=dev) * 0.01
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    _, _, stats = linear.linear_logp_forward(h, W, y, vocab, vocab, stream=stream)
    dh = torch.empty((n, hidden), dtype=out_dtype, device=dev)
    dW = torch.empty((vocab, hidden), dtype=out_dtype, device=dev)
    ws_bytes = linear.linear_logp_backward_workspace(n, hidden, chunk_cols, out_dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        linear.linear_logp_backward(h, W, y, g, stats, vocab, vocab, chunk_cols=chunk_cols,
                                    dhidden=dh, dweight=dW, workspace=ws, stream=stream,
                                    out_dtype=out_dtype)

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
    out = {"rows": n, "hidden": hidden, "vocab": vocab, "chunk_cols": chunk_cols,
           "out_dtype": str(out_dtype).replace("torch.", ""), "ms": round(ms, 4),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "workspace_bytes": ws_bytes}
    if not cpu_baseline:
        return out
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
    out["cpu_baseline"] = cpu
    return out


def time_linear_kept(dst, stream, steps: int, n: int = 8192, hidden: int = 4096,
                     vocab: int = 151936, chunk_cols: int = 16384) -> dict:
    """linear_logp with kept logits on the same LM-head shape: the balanced forward that also
    writes the scored logits (linear_logp_partials_save, 4 bytes per logit) and the
    BF16-output backward that reads them (linear_logp_backward_saved: dh and dW on the matrix
    cores, 4 n V H flops, dz from the kept logits), each timed over ``steps`` calls."""
    import torch

    from deterministic_selected_token_amd import linear

    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(13)
    h = torch.randn((n, hidden), generator=gen, device=dev).to(torch.bfloat16)
    W = (torch.randn((vocab, hidden), generator=gen, device=dev) * (3.0 / hidden ** 0.5)) \
        .to(torch.bfloat16)
    y = torch.randint(0, vocab, (n,), generator=gen, device=dev)
    g = torch.randn((n,), generator=gen, device=dev) * 0.01
    z = torch.empty((n, vocab), dtype=torch.float32, device=dev)
    P = torch.empty((n, dst.logp_num_tiles(vocab), 3), dtype=torch.float32, device=dev)
    wsf = torch.empty(max(1, linear.linear_logp_partials_workspace(n, vocab, 0, vocab)),
                      dtype=torch.uint8, device=dev)
    dh = torch.empty((n, hidden), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((vocab, hidden), dtype=torch.bfloat16, device=dev)
    wsb = torch.empty(linear.linear_logp_backward_workspace(n, hidden, chunk_cols,
                                                            torch.bfloat16),
                      dtype=torch.uint8, device=dev)

    def fwd():
        linear.linear_logp_partials(h, W, y, vocab, vocab, 0, vocab, P, stream=stream,
                                    workspace=wsf, logits=z)

    fwd()
    _, _, stats = dst.logp_merge(P, y, vocab, stream=stream)

    def bwd():
        linear.linear_logp_backward(h, W, y, g, stats, vocab, vocab, chunk_cols=chunk_cols,
                                    dhidden=dh, dweight=dW, workspace=wsb, stream=stream,
                                    out_dtype=torch.bfloat16, logits=z)

    def timed(fn):
        fn()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / steps

    fwd_ms, bwd_ms = timed(fwd), timed(bwd)
    del h, W, z, dW, wsb
    torch.cuda.empty_cache()
    return {"logits_bytes": 4 * n * vocab, "forward_keeping_logits_ms": round(fwd_ms, 4),
            "backward_bf16_out_from_kept_logits_ms": round(bwd_ms, 4),
            "backward_tflops": round(4.0 * n * vocab * hidden / (bwd_ms * 1e-3) / 1e12, 1)}


def time_linear_default(dst, stream) -> dict:
    """The default run's linear_logp entry: the forward with its balancing workspace and the
    BF16-output backward at 8192 x 4096 x 151936, each as TFLOP/s and as a fraction of the
    dense BF16 matrix-core ceiling measured in the same run, and the same pair with kept
    logits (no oracle leg; --variants has the full set)."""
    import torch

    fwd = time_linear(dst, stream, 3, cpu_baseline=False)
    bwd = time_linear_backward(dst, stream, 2, out_dtype=torch.bfloat16, cpu_baseline=False)
    kept = time_linear_kept(dst, stream, 2)
    kept["forward_plus_backward_ms"] = round(kept["forward_keeping_logits_ms"]
                                             + kept["backward_bf16_out_from_kept_logits_ms"], 4)
    kept["recomputing_forward_plus_backward_ms"] = round(fwd["partials_ms"] + bwd["ms"], 4)
    mc = mfma_ceiling(stream, reps=3)
    return {"workload": "h [8192, 4096] x W [151936, 4096] BF16, unit temperature",
            "forward": {"ms": fwd["partials_ms"], "merge_ms": fwd["merge_ms"],
                        "tflops": fwd["tflops"], "frac_of_bf16_peak": fwd["frac_of_bf16_peak"],
                        "frac_of_measured_mfma_ceiling": round(fwd["tflops"] / mc["tflops"], 4)},
            "backward_bf16_out": {"ms": bwd["ms"], "tflops": bwd["tflops"],
                                  "frac_of_bf16_peak": bwd["frac_of_bf16_peak"],
                                  "frac_of_measured_mfma_ceiling": round(
                                      bwd["tflops"] / mc["tflops"], 4)},
            "kept_logits": kept,
            "mfma_bf16_ceiling_tflops": mc["tflops"]}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="0 disables the oracle leg (cpu_baseline and accuracy)")
    ap.add_argument("--bwd-rows", type=int, default=20480,
                    help="rows of each workload whose dlogits the oracle checks")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the headline step only (no ceilings, other workloads or "
                         "oracle leg): the short run the counter passes profile")
    ap.add_argument("--variants", action="store_true",
                    help="also time FP16 and FP32 logits and BF16 at temperature 0.7 on the "
                         "same shape, a GRPO step, the GRPO loss alone and linear_logp "
                         "(reported under config.variants)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="end with one 4 GiB hbm_copy of the ceiling probe (counter scaling)")
    ap.add_argument("--linear-forward-only", action="store_true",
                    help="only three linear_logp forward calls on the 8192 x 4096 x 151936 "
                         "shape, one JSON line (the short run the linear counter passes "
                         "profile)")
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
    from workloads import headline_case, long_case, mid_case

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.linear_forward_only:
        lin = time_linear(dst, stream, 3, cpu_baseline=False)
        print(json.dumps({"metric": "linear_logp forward TFLOP/s (8192 x 4096 x 151936)",
                          "value": lin["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": 3,
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": "linear_logp forward only", **lin}}),
              flush=True)
        return 0
    quick = args.headline_only
    extra_steps = max(3, args.steps // 4)

    ceiling = None
    if not quick:
        print("bench: measuring the HBM read and copy ceilings", file=sys.stderr, flush=True)
        ceiling = hbm_ceiling(stream)

    print("bench: generating the headline workload", file=sys.stderr, flush=True)
    case = headline_case(device=dev)
    n, v = case.n, case.vocab_real
    x, y, g = case.logits, case.targets, case.grad
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    stats = torch.empty((n, 2), dtype=torch.float32, device=dev)
    dlogits = torch.empty((n, v), dtype=torch.bfloat16, device=dev)

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
    fwd_achieved = fwd_b / (fwd_avg * 1e-3) / 1e9

    extra = {}
    accuracy = None
    cpu = None
    if not quick:
        print("bench: batch invariance, tensor-parallel share", file=sys.stderr, flush=True)
        extra["batch_invariance"] = batch_invariance(
            dst, case, (logp, lse, stats, dlogits), stream)
        extra["tp8_rank_share"] = time_tp8_share(dst, case, stream, extra_steps)
        print("bench: mid-size workload", file=sys.stderr, flush=True)
        mid = mid_case(device=dev)
        extra["mid"] = {"workload": "N=4096, vocabulary 151936 padded to 152064 (-inf "
                                    "pads), BF16 ~N(0,3^2), 5% inactive rows, g = 1/N_active",
                        **time_case(dst, mid, stream, extra_steps)}
        del mid
        print("bench: vocab-shard workload", file=sys.stderr, flush=True)
        extra["shards"] = time_shard_config(dst, stream, extra_steps)
        print("bench: 131072-row workload", file=sys.stderr, flush=True)
        long = long_case(device=dev)
        extra["long_131072"] = {"workload": "N=131072, V=151936, BF16 ~N(0,3^2), uniform "
                                            "targets, g ~N(0,1)",
                                **time_case(dst, long, stream, extra_steps)}
        del long
        torch.cuda.empty_cache()
        print("bench: the pages' bench inputs", file=sys.stderr, flush=True)
        pages = headline_case(device=dev, pages_bench=True)
        pages_t = time_case(dst, pages, stream, extra_steps, keep=True)
        pages_out = pages_t.pop("_outputs")
        extra["pages_bench_inputs"] = {"workload": "N=32768, V=151936, BF16 randn (sigma 1), "
                                                   "uniform targets, g = 1", **pages_t}
        if args.cpu_seconds > 0:
            import oracle

            threads = oracle.default_threads()
            print("bench: the oracle on the host, compared with the GPU outputs",
                  file=sys.stderr, flush=True)
            leg = oracle_leg(case, (logp, lse, stats, dlogits), args.bwd_rows, threads)
            leg_pages = oracle_leg(pages, pages_out, args.bwd_rows, threads)
            accuracy = {"headline": leg["accuracy"], "pages_bench_inputs": leg_pages["accuracy"],
                        "reference": "FP64 oracle; logp/LSE absolute errors over every row, "
                                     "dlogits over the sampled rows' N x V elements"}
            cpu = cpu_baseline(leg, case, threads)
        del pages, pages_out
        torch.cuda.empty_cache()
        print("bench: linear_logp (matrix cores)", file=sys.stderr, flush=True)
        extra["linear_logp"] = time_linear_default(dst, stream)
        torch.cuda.empty_cache()
    if args.variants:
        extra["variants"] = time_variants(dst, case, stream, args.steps)
        extra["variants"].update(time_grpo(dst, case, stream, args.steps))
        extra["variants"]["linear_logp_fwd"] = time_linear(dst, stream, max(3, args.steps // 4))
        extra["variants"]["linear_logp_fwd_temperature_0.7"] = time_linear(
            dst, stream, max(3, args.steps // 4), inv_temperature=1 / 0.7, cpu_baseline=False)
        extra["variants"]["linear_logp_partials_tp8_rank"] = time_linear_shard(
            dst, stream, max(5, args.steps // 4))
        extra["variants"]["linear_logp_bwd"] = time_linear_backward(
            dst, stream, max(2, args.steps // 8))
        extra["variants"]["linear_logp_bwd_bf16_out"] = time_linear_backward(
            dst, stream, max(2, args.steps // 8), out_dtype=torch.bfloat16, cpu_baseline=False)
        mc = mfma_ceiling(stream)
        extra["variants"]["mfma_bf16_ceiling"] = mc
        extra["variants"]["vendor_gemm_reference"] = vendor_gemm_reference(stream)
        extra["variants"]["lds_rates"] = lds_rates(stream)
        for key in ("linear_logp_fwd", "linear_logp_fwd_temperature_0.7", "linear_logp_bwd",
                    "linear_logp_bwd_bf16_out"):
            entry = extra["variants"][key]
            entry["frac_of_measured_mfma_ceiling"] = round(entry["tflops"] / mc["tflops"], 4)
    if args.profile_copy:
        lib = load_ceiling_library()
        nbytes = 4 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst_buf = torch.empty_like(src)
        if lib.hbm_copy(src.data_ptr(), dst_buf.data_ptr(), nbytes, 16, 16,
                        stream.cuda_stream) != 0:
            raise RuntimeError("hbm_copy failed")
        torch.cuda.synchronize()
        extra["copy_bytes_each_way"] = nbytes

    props = torch.cuda.get_device_properties(dev)
    roofline = {"bound": "hbm", "kernel": "bwd_flat_kernel (logp_backward)",
                "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("bwd"),
                "algorithmic_bytes_per_launch": bwd_b,
                "avg_launch_ms": round(bwd_avg, 4),
                "fwd_kernel": {"achieved": round(fwd_achieved, 2),
                               "frac": round(fwd_achieved / HBM_PEAK_GBS, 4),
                               "avg_launch_ms": round(fwd_avg, 4),
                               "algorithmic_bytes_per_launch": fwd_b,
                               "traffic": measured_traffic("fwd")}}
    if ceiling is not None:
        roofline["ceiling"] = ceiling
        roofline["frac_of_copy_ceiling"] = round(achieved / ceiling["copy_gbs"], 4)
        roofline["fwd_kernel"]["frac_of_read_ceiling"] = round(
            fwd_achieved / ceiling["read_gbs"], 4)
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
                   "floor_ms_at_8tbs": round((fwd_b + bwd_b) / (HBM_PEAK_GBS * 1e9) * 1e3, 3),
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
        "roofline": roofline,
        "accuracy": accuracy,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
