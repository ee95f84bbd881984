"""The forward's whole reduction order, bitwise, on inputs whose exponentials are exact.

FP32 logits x_c = t_c are chosen so that fl32(t_c * fl32(log2 e)) is an integer k_c in
[-40, 0], and every 4096-column tile holds one column with t = 0.  Then every tile maximum is
0, every term exp(x - m) = 2^(k_c) exactly (the hardware exp2 at an integer argument; the
test also checks that directly), and the only roundings left are the additions, whose result
depends on their order.  The expected bits come from a float32 emulation of the order the
numerical contract fixes (issue #241 "PR 3"; PR #314's Tensor Parallel doc: fixed global
tiles and a fixed merge order): lane l of a tile holds columns 512k + 8l + e and adds its 64
terms in (k, e) order from +0, the 64 lane sums combine pairwise (lane xor 1, 2, ..., 32); the
merge adds the tile sums (weights s_l * 2^0) the same way, lane i taking tiles i, i+64, ....
Both logp_partials' s_l and the fused forward's S must carry those exact bits; a plain
left-to-right sum differs on most rows, so the test sees the order.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest
import torch

import deterministic_selected_token_amd as dst

DEV = "cuda"
PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libexp2_probe.so")
T = 4096
LOG2E = np.float32(1.44269504088896340736)


def exact_exponent_args(lo: int = -40) -> dict[int, np.float32]:
    """k -> t with fl32(t * LOG2E) == k exactly (the k in [lo, 0] that have one nearby)."""
    out = {}
    for k in range(lo, 1):
        t = np.float32(np.float32(k) / LOG2E)
        for _ in range(16):
            p = np.float32(t * LOG2E)
            if p == k:
                out[k] = t
                break
            t = np.nextafter(t, np.float32(-np.inf) if p > k else np.float32(np.inf),
                             dtype=np.float32)
    return out


def lane_tree(lanes: np.ndarray) -> np.float32:
    lanes = lanes.astype(np.float32)
    o = 1
    while o < 64:
        lanes = (lanes + lanes[np.arange(64) ^ o]).astype(np.float32)
        o <<= 1
    return lanes[0]


def tile_sum(terms: np.ndarray) -> np.float32:
    """terms: float32 [4096] of one tile in column order (0 for masked columns)."""
    lanes = np.zeros(64, dtype=np.float32)
    for lane in range(64):
        acc = np.float32(0.0)
        for k in range(8):
            for e in range(8):
                acc = np.float32(acc + terms[512 * k + 8 * lane + e])
        lanes[lane] = acc
    return lane_tree(lanes)


def merge_sum(w: np.ndarray) -> np.float32:
    lanes = np.zeros(64, dtype=np.float32)
    for l, x in enumerate(w.astype(np.float32)):
        lanes[l % 64] = np.float32(lanes[l % 64] + x)
    return lane_tree(lanes)


def test_exact_arguments_exist_and_the_emulation_is_exact_where_order_cannot_matter():
    ks = exact_exponent_args()
    assert 0 in ks and ks[0] == 0.0 and len(ks) >= 30
    # all terms 1: every order gives 4096 exactly
    assert tile_sum(np.ones(T, dtype=np.float32)) == 4096.0
    assert merge_sum(np.full(100, 4096.0, dtype=np.float32)) == 409600.0


@pytest.mark.gpu
@pytest.mark.parametrize("V", [4096, 3 * 4096, 5 * 4096 + 1000])
def test_forward_reduction_order_is_the_contracts(V):
    n = 6
    ks = exact_exponent_args()
    kvals = np.array(sorted(ks), dtype=np.int64)
    tvals = np.array([ks[int(k)] for k in kvals], dtype=np.float32)
    rng = np.random.default_rng(V)
    pick = rng.integers(0, kvals.size, size=(n, V))
    L = -(-V // T)
    for l in range(L):  # one column per tile at t = 0, so every tile maximum is 0
        c0 = l * T
        width = min(T, V - c0)
        cols = c0 + rng.integers(0, width, size=n)
        pick[np.arange(n), cols] = int(np.searchsorted(kvals, 0))
    x = tvals[pick]
    terms = np.ldexp(np.float32(1.0), kvals[pick]).astype(np.float32)  # 2^k, exact
    want_s = np.zeros((n, L), dtype=np.float32)
    for r in range(n):
        for l in range(L):
            tile = np.zeros(T, dtype=np.float32)
            seg = terms[r, l * T:(l + 1) * T]
            tile[:seg.size] = seg
            want_s[r, l] = tile_sum(tile)
    want_S = np.array([merge_sum(want_s[r]) for r in range(n)], dtype=np.float32)

    print(f"[gpu] tile order: n={n} V={V} FP32 logits with exact exponentials", flush=True)
    logits = torch.from_numpy(x).to(DEV)
    y = torch.full((n,), -100, dtype=torch.int64, device=DEV)
    # the premise: the hardware exp2 (the probe library's v_exp_f32) is exact at each k
    probe = ctypes.CDLL(PROBE)
    probe.exp2_probe.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                 ctypes.c_int, ctypes.c_void_p]
    probe.exp2_probe.restype = ctypes.c_int
    out = torch.zeros(2, dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    for k in kvals:
        bits = int(np.float32(k).view(np.uint32))
        assert probe.exp2_probe(bits, 1, out.data_ptr(), 1, stream) == 0
        torch.cuda.synchronize()
        assert int(out[1]) == 0, f"hardware exp2({k}) is not 2^{k}"
    partials = torch.empty((n, L, 3), dtype=torch.float32, device=DEV)
    dst.logp_partials_ex(logits, y, V, V, 0, V, partials)
    _, _, stats = dst.logp_forward_ex(logits, y, V, V)
    torch.cuda.synchronize()
    p = partials.cpu().numpy()
    assert np.all(p[:, :, 0] == 0.0)
    got_s = np.ascontiguousarray(p[:, :, 1])
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), \
        np.argwhere(got_s != want_s)[:5]
    st = stats.cpu().numpy()
    assert np.all(st[:, 0] == 0.0)
    got_S = np.ascontiguousarray(st[:, 1])
    assert np.array_equal(got_S.view(np.uint32), want_S.view(np.uint32)), (got_S, want_S)
    # the order is visible: a left-to-right sum over the row's terms differs on most rows
    seq = []
    for r in range(n):
        acc = np.float32(0.0)
        for v in terms[r]:
            acc = np.float32(acc + v)
        seq.append(acc)
    assert np.mean(np.array(seq, dtype=np.float32) != want_S) > 0.5
