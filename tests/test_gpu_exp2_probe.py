"""The hardware exp2 (v_exp_f32) against the correctly rounded exp2, exhaustively over every
float in [-0.5, 0.5] (about 2.1e9 values).  The backward forms exp(t) as
exp2(u) (1 + delta) with the argument split exactly, so its accuracy is that of this
instruction on the fractional part; the forward's sum-exp uses it directly.  The probe is a
test library of its own (tests/probes), not part of the C ABI."""

from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "probes", "libexp2_probe.so")
BLOCKS = 4096


def test_hardware_exp2_is_within_one_ulp_on_the_unit_interval():
    lib = ctypes.CDLL(LIB)  # built by __graft_entry__.build(); missing means not built
    lib.exp2_probe.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int,
                               ctypes.c_void_p]
    lib.exp2_probe.restype = ctypes.c_int
    out = torch.zeros(2 * BLOCKS, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    half = 0x3F000000  # bit pattern of 0.5
    worst, off, total = 0, 0, 0
    for lo in (0x00000000, 0x80000000):  # [+0, 0.5] and [-0, -0.5]
        print(f"[gpu] exp2 probe from {lo:#010x}, {half + 1} values", flush=True)
        assert lib.exp2_probe(lo, half + 1, out.data_ptr(), BLOCKS, stream) == 0
        torch.cuda.synchronize()
        o = out.cpu().numpy().view(np.uint32)
        worst = max(worst, int(o[0::2].max()))
        off += int(o[1::2].astype(np.int64).sum())
        total += half + 1
    print(f"[gpu] exp2 on [-0.5, 0.5]: max {worst} ulp, {off} of {total} not correctly "
          f"rounded ({100.0 * off / total:.4f}%)", flush=True)
    assert worst <= 1, worst
