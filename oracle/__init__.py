"""FP64 CPU oracle for the selected-token log-probability path.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the bench's
``cpu_baseline`` leg are the only users.  The product path (the HIP library and its
binding) never imports, links or calls anything in this directory, and this directory
shares no code with it.

The arithmetic lives in ``logp_oracle.c`` (plain C, double precision, loops in column
order, one block of rows per thread).  This module only builds that file with gcc and
marshals numpy arrays into it.

Parity status of each function (what pins it is in ``tests/test_oracle_pins.py``):
  forward, backward, tile_partials (BF16, FP16 and FP32 logits; any inv_temperature),
  merge, rne_bf16, rne_f16, count_bad_targets, backward_elements: pinned.  Rows whose
  valid target logit is -inf while other logits are finite are pinned by the 50-digit
  brute force, whose alphabet holds -inf.
  Rows that hold NaN or +inf logits: parity unpinned (no closed form was written for them).

``grpo_oracle.py`` (plain numpy, float64) is the oracle of the GRPO loss on these
log-probabilities; its pins are in ``tests/test_grpo_oracle_pins.py``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

TILE = 4096  # tile width used by the partial checker (same numeric value as the kernels')

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "logp_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblogp_oracle.so")
_lib = None
_lock = threading.Lock()

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile ``logp_oracle.c`` into ``liblogp_oracle.so`` next to it (gcc, -O2)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", "-ffp-contract=off", "-fvisibility=hidden",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Load a compiled oracle shared object and declare its signatures."""
    lib = ctypes.CDLL(path)
    _declare(lib)
    return lib


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or \
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            _lib = load_library(_LIB_PATH)
    return _lib


def _declare(lib) -> None:
    lib.oracle_rne_bf16.restype = ctypes.c_uint16
    lib.oracle_rne_bf16.argtypes = [ctypes.c_double]
    lib.oracle_rne_bf16_array.restype = None
    lib.oracle_rne_bf16_array.argtypes = [_P, _P, _I64]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_forward.argtypes = [_P, _I64, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P,
                                   ctypes.c_int]
    lib.oracle_backward.restype = ctypes.c_int
    lib.oracle_backward.argtypes = [_P, _I64, _I64, _I64, _I64, _P, _P, _I64, _P, _P, _I64,
                                    _P, _I64, ctypes.c_int]
    lib.oracle_tile_partials.restype = ctypes.c_int
    lib.oracle_tile_partials.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _P, _P, _I64, _P,
                                         _P, _P, ctypes.c_int]
    lib.oracle_merge.restype = ctypes.c_int
    lib.oracle_merge.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _I64, _P, _P]
    lib.oracle_count_bad_targets.restype = ctypes.c_int64
    lib.oracle_count_bad_targets.argtypes = [_P, _P, _I64, _I64, _I64]
    lib.oracle_rne_f16_array.restype = None
    lib.oracle_rne_f16_array.argtypes = [_P, _P, _I64]
    _F = ctypes.c_float
    lib.oracle_forward_ex.restype = ctypes.c_int
    lib.oracle_forward_ex.argtypes = [ctypes.c_int, _F, _P, _I64, _I64, _I64, _P, _P, _I64, _P,
                                      _P, _P, _P, ctypes.c_int]
    lib.oracle_backward_ex.restype = ctypes.c_int
    lib.oracle_backward_ex.argtypes = [ctypes.c_int, _F, _P, _I64, _I64, _I64, _I64, _P, _P,
                                       _I64, _P, _P, _I64, _P, _I64, ctypes.c_int]
    lib.oracle_tile_partials_ex.restype = ctypes.c_int
    lib.oracle_tile_partials_ex.argtypes = [ctypes.c_int, _F, _P, _I64, _I64, _I64, _I64, _I64,
                                            _P, _P, _I64, _P, _P, _P, ctypes.c_int]


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


# ------------------------------------------------------------------ marshalling

DTYPES = {"bf16": 0, "f16": 1, "f32": 2, "f64": 3}  # f64: forward and partials only


def _logits(logits):
    """(C-contiguous array [n, ld], dtype name).  BF16 travels as raw uint16 bits."""
    try:
        import torch
        if isinstance(logits, torch.Tensor):
            t = logits.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16), "bf16"
            if t.dtype == torch.float16:
                return t.numpy(), "f16"
            if t.dtype == torch.float32:
                return t.numpy(), "f32"
            if t.dtype == torch.float64:
                return t.numpy(), "f64"
            raise TypeError(f"oracle: unsupported logits dtype {t.dtype}")
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(logits)
    if a.dtype == np.uint16:
        return a, "bf16"
    if a.dtype == np.float16:
        return a, "f16"
    if a.dtype == np.float32:
        return a, "f32"
    if a.dtype == np.float64:
        return a, "f64"
    raise TypeError("oracle expects BF16 bits (uint16), float16, float32 or float64 logits")


def _bits(logits) -> np.ndarray:
    """BF16 logits as a C-contiguous uint16 array of raw bits, shape [n, ld]."""
    a, dt = _logits(logits)
    if dt != "bf16":
        raise TypeError("oracle expects bfloat16 logits here")
    return a


def _np(x, dtype) -> Optional[np.ndarray]:
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=dtype)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


# ------------------------------------------------------------------ entry points

def rne_bf16(values, lib=None) -> np.ndarray:
    """Round FP64 values to BF16 (nearest, ties to even) directly; returns uint16 bits."""
    a = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load(lib).oracle_rne_bf16_array(_ptr(a), _ptr(out), a.size)
    return out


def rne_f16(values, lib=None) -> np.ndarray:
    """Round FP64 values to binary16 (nearest, ties to even) directly; returns uint16 bits."""
    a = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load(lib).oracle_rne_f16_array(_ptr(a), _ptr(out), a.size)
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def forward(logits, targets, vocab_real: int, active=None, ignore_index: int = -100,
            nthreads: Optional[int] = None, lib=None, inv_temperature: float = 1.0) -> dict:
    """FP64 logp, LSE, row max M and row sum-exp S for every row.

    ``logits``: BF16 (torch bfloat16 or raw uint16 bits), float16 or float32, [n, ld].
    The scored logits are fl32(x * inv_temperature)."""
    x, dt = _logits(logits)
    n, ld = (x.shape[0], x.shape[1]) if x.ndim == 2 else (0, vocab_real)
    y = _np(targets, np.int64)
    act = _np(active, np.uint8)
    out = {k: np.empty(n, dtype=np.float64) for k in ("logp", "lse", "max", "sumexp")}
    rc = _load(lib).oracle_forward_ex(DTYPES[dt], float(np.float32(inv_temperature)), _ptr(x),
                                      ld, n, vocab_real, _ptr(y), _ptr(act), ignore_index,
                                      _ptr(out["logp"]), _ptr(out["lse"]), _ptr(out["max"]),
                                      _ptr(out["sumexp"]), nthreads or default_threads())
    _check(rc, "forward")
    return out


def backward(logits, targets, grad, vocab_real: int, vocab_padded: Optional[int] = None,
             active=None, ignore_index: int = -100, want_f64: bool = True,
             want_bf16: bool = True, nthreads: Optional[int] = None, lib=None,
             inv_temperature: float = 1.0) -> dict:
    """FP64 dlogits [n, vocab_padded] and its direct rounding to the logits' dtype.

    Returns {"d64": float64 or None, "rounded": array in the logits' dtype (BF16 as uint16
    bits) or None, "bf16": the same as "rounded" for BF16 logits}."""
    x, dt = _logits(logits)
    n, ld = x.shape
    vocab_padded = vocab_real if vocab_padded is None else vocab_padded
    y = _np(targets, np.int64)
    act = _np(active, np.uint8)
    g = _np(grad, np.float32)
    d64 = np.empty((n, vocab_padded), dtype=np.float64) if want_f64 else None
    out_dtype = {"bf16": np.uint16, "f16": np.float16, "f32": np.float32}[dt]
    rounded = np.empty((n, vocab_padded), dtype=out_dtype) if want_bf16 else None
    rc = _load(lib).oracle_backward_ex(DTYPES[dt], float(np.float32(inv_temperature)), _ptr(x),
                                       ld, n, vocab_real, vocab_padded, _ptr(y), _ptr(act),
                                       ignore_index, _ptr(g), _ptr(d64), vocab_padded,
                                       _ptr(rounded), vocab_padded, nthreads or default_threads())
    _check(rc, "backward")
    return {"d64": d64, "rounded": rounded, "bf16": rounded if dt == "bf16" else None}


def backward_elements(logits_row, cols, target: int, grad: float, lse: float,
                      vocab_real: int, valid: bool = True) -> np.ndarray:
    """dlogits of one row at the given columns only, float64: g (1[c == y] - exp(x_c - LSE))
    for real columns of a valid row, 0 elsewhere -- the definition ``backward`` evaluates for
    whole rows, for rows too wide to expand in float64.  ``lse`` is the row's ``forward`` LSE;
    ``logits_row`` is one BF16 row (torch bfloat16 or raw uint16 bits)."""
    bits, dt = _logits(logits_row.reshape(1, -1) if hasattr(logits_row, "reshape")
                       else np.asarray(logits_row).reshape(1, -1))
    if dt != "bf16":
        raise TypeError("backward_elements expects a BF16 row")
    c = np.asarray(cols, dtype=np.int64)
    out = np.zeros(c.shape, dtype=np.float64)
    if not valid or not np.isfinite(lse):
        return out
    real = c < vocab_real
    x = bf16_bits_to_f64(bits[0, c[real]])
    d = -float(np.float32(grad)) * np.exp(x - lse)
    d[c[real] == target] += float(np.float32(grad))
    out[real] = d
    return out


def num_tiles(vocab_padded: int, tile: int = TILE) -> int:
    return -(-vocab_padded // tile)


def tile_partials(logits, targets, vocab_real: int, vocab_padded: Optional[int] = None,
                  active=None, ignore_index: int = -100, tile: int = TILE,
                  nthreads: Optional[int] = None, lib=None,
                  inv_temperature: float = 1.0) -> dict:
    """FP64 per-tile (m, s, sel), each [n, ceil(vocab_padded / tile)]."""
    x, dt = _logits(logits)
    n, ld = x.shape
    vocab_padded = vocab_real if vocab_padded is None else vocab_padded
    L = num_tiles(vocab_padded, tile)
    y = _np(targets, np.int64)
    act = _np(active, np.uint8)
    out = {k: np.empty((n, L), dtype=np.float64) for k in ("max", "sumexp", "sel")}
    rc = _load(lib).oracle_tile_partials_ex(DTYPES[dt], float(np.float32(inv_temperature)),
                                            _ptr(x), ld, n, vocab_real, vocab_padded, tile,
                                            _ptr(y), _ptr(act), ignore_index, _ptr(out["max"]),
                                            _ptr(out["sumexp"]), _ptr(out["sel"]),
                                            nthreads or default_threads())
    _check(rc, "tile_partials")
    return out


def merge(m, s, sel, targets, vocab_real: int, active=None, ignore_index: int = -100,
          tile: int = TILE, lib=None) -> dict:
    """FP64 merge of per-tile partials in tile order -> logp, LSE."""
    m = np.ascontiguousarray(m, dtype=np.float64)
    s = np.ascontiguousarray(s, dtype=np.float64)
    sel = np.ascontiguousarray(sel, dtype=np.float64)
    n, L = m.shape
    y = _np(targets, np.int64)
    act = _np(active, np.uint8)
    out = {k: np.empty(n, dtype=np.float64) for k in ("logp", "lse")}
    rc = _load(lib).oracle_merge(_ptr(m), _ptr(s), _ptr(sel), n, L, tile, vocab_real, _ptr(y),
                              _ptr(act), ignore_index, _ptr(out["logp"]), _ptr(out["lse"]))
    _check(rc, "merge")
    return out


def count_bad_targets(targets, vocab_real: int, active=None, ignore_index: int = -100,
                      lib=None) -> int:
    y = _np(targets, np.int64)
    act = _np(active, np.uint8)
    return int(_load(lib).oracle_count_bad_targets(_ptr(y), _ptr(act), y.size, vocab_real,
                                                ignore_index))
