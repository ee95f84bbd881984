"""Python binding of the gfx950 selected-token log-probability library.

Argument marshalling only: every entry point checks tensor dtypes and devices, allocates
outputs with torch when the caller passes none, and calls the C ABI declared in
``include/logp.h`` (``liblogp_mi355x.so`` next to this file).  Every step of the
computation runs in the HIP kernels; there is no CPU or PyTorch fallback, and importing
this package fails loudly when the library has not been built.

Tensor conventions:
  * logits: bfloat16 ``[n, width]`` with unit column stride; ``ld = logits.stride(0)``
    (the ``_ex`` functions also take float16 and float32 logits and a temperature).
    A vocab shard is a column slice of the full buffer (``full[:, c0:c1]``).
  * targets: int64 ``[n]``; active: uint8/bool ``[n]`` or None; grad_logp: float32 ``[n]``.
  * stats: float32 ``[n, 2]`` = (M, S) per row; partials: float32 ``[n, L, 3]`` =
    (m_l, s_l, sel_l) per global tile, ``L = logp_num_tiles(vocab_padded)``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loaded first so the library binds to the HIP runtime torch already uses

TILE_COLS = 4096
FWD_MAX_TILES = 4096

_HERE = os.path.dirname(os.path.abspath(__file__))
# DST_AMD_LIB selects another build of the same library (the tests' sanitizer build of the
# host code uses it); by default the in-tree build next to this file.
LIB_PATH = os.environ.get("DST_AMD_LIB") or os.path.join(_HERE, "liblogp_mi355x.so")

STATUS = {
    0: "LOGP_OK", 1: "LOGP_ERR_NULL", 2: "LOGP_ERR_SHAPE", 3: "LOGP_ERR_SHARD",
    4: "LOGP_ERR_DEVICE", 5: "LOGP_ERR_RANGE", 6: "LOGP_ERR_OVERLAP", 7: "LOGP_ERR_HIP",
    8: "LOGP_ERR_ARG", 9: "LOGP_ERR_SCRATCH",
}
DTYPES = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}  # logp_dtype_t values
EXPORTED = ("logp_forward", "logp_backward", "logp_partials", "logp_merge", "logp_num_tiles",
            "logp_check_targets", "logp_status_string", "logp_forward_ex", "logp_backward_ex",
            "logp_partials_ex")


class LogpError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({detail})")
        self.status = status


def _load_library() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -m "
            "deterministic_selected_token_amd.build, or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.logp_forward.argtypes = [P, I64, I64, I64, I64, P, P, I64, P, P, P, P]
    lib.logp_backward.argtypes = [P, I64, I64, I64, I64, I64, I64, P, P, I64, P, P, P, I64, P]
    lib.logp_partials.argtypes = [P, I64, I64, I64, I64, I64, I64, P, P, I64, P, I64, P]
    lib.logp_merge.argtypes = [P, I64, I64, I64, I64, P, P, I64, P, P, P, P]
    lib.logp_check_targets.argtypes = [P, P, I64, I64, I64, P, P]
    F = ctypes.c_float
    lib.logp_forward_ex.argtypes = [I32, F] + lib.logp_forward.argtypes
    lib.logp_backward_ex.argtypes = [I32, F] + lib.logp_backward.argtypes
    lib.logp_partials_ex.argtypes = [I32, F] + lib.logp_partials.argtypes
    for fn in ("logp_forward", "logp_backward", "logp_partials", "logp_merge",
               "logp_check_targets", "logp_forward_ex", "logp_backward_ex", "logp_partials_ex"):
        getattr(lib, fn).restype = I32
    lib.logp_num_tiles.argtypes = [I64]
    lib.logp_num_tiles.restype = I64
    lib.logp_status_string.argtypes = [I32]
    lib.logp_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load_library()


def library() -> ctypes.CDLL:
    """The loaded C-ABI library (``ctypes.CDLL``)."""
    return _lib


# ------------------------------------------------------------------ marshalling helpers

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    h = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return h or None


def _check(fn: str, status: int):
    if status != 0:
        raise LogpError(fn, status, _lib.logp_status_string(status).decode())


def _rows(name: str, t: torch.Tensor, dtype: torch.dtype, n: int, device) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, logits on {device}")
    if t.dim() != 1 or t.shape[0] != n or (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous [{n}] tensor")
    return t


def _active(active, n: int, device) -> Optional[torch.Tensor]:
    if active is None:
        return None
    if active.dtype == torch.bool:
        active = active.view(torch.uint8)
    return _rows("active", active, torch.uint8, n, device)


def _matrix(name: str, t: torch.Tensor, dtype) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    allowed = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in allowed:
        raise TypeError(f"{name} must be one of {allowed}, got {t.dtype}")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (device memory), got {t.device}")
    return t


def _ld(t: torch.Tensor) -> int:
    return int(t.stride(0)) if t.shape[0] > 1 else int(max(t.shape[1], t.stride(0)))


# ------------------------------------------------------------------ entry points

def logp_num_tiles(vocab_padded: int) -> int:
    return int(_lib.logp_num_tiles(int(vocab_padded)))


def logp_status_string(status: int) -> str:
    return _lib.logp_status_string(int(status)).decode()


def _forward(fn: str, logits, targets, vocab_real, vocab_padded, active, ignore_index, logp, lse,
             stats, stream, inv_temperature):
    ex = fn.endswith("_ex")
    logits = _matrix("logits", logits, tuple(DTYPES) if ex else torch.bfloat16)
    n, width = logits.shape
    dev = logits.device
    vocab_padded = width if vocab_padded is None else int(vocab_padded)
    vocab_real = vocab_padded if vocab_real is None else int(vocab_real)
    targets = _rows("targets", targets, torch.int64, n, dev)
    active = _active(active, n, dev)
    if logp is None:
        logp = torch.empty(n, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(n, dtype=torch.float32, device=dev)
    if stats is None:
        stats = torch.empty((n, 2), dtype=torch.float32, device=dev)
    _rows("logp", logp, torch.float32, n, dev)
    _rows("lse", lse, torch.float32, n, dev)
    if stats.shape != (n, 2) or stats.dtype != torch.float32 or not stats.is_contiguous():
        raise ValueError("stats must be a contiguous float32 [n, 2] tensor")
    args = (_ptr(logits), _ld(logits), n, vocab_real, vocab_padded, _ptr(targets), _ptr(active),
            int(ignore_index), _ptr(logp), _ptr(lse), _ptr(stats), _stream(dev, stream))
    if ex:
        st = _lib.logp_forward_ex(DTYPES[logits.dtype], float(inv_temperature), *args)
    else:
        st = _lib.logp_forward(*args)
    _check(fn, st)
    return logp, lse, stats


def logp_forward(logits: torch.Tensor, targets: torch.Tensor, vocab_real: Optional[int] = None,
                 vocab_padded: Optional[int] = None, active=None, ignore_index: int = -100,
                 logp: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 stats: Optional[torch.Tensor] = None, stream=None):
    """Selected-token logp, LSE and per-row (M, S) over whole BF16 rows -> (logp, lse, stats)."""
    return _forward("logp_forward", logits, targets, vocab_real, vocab_padded, active,
                    ignore_index, logp, lse, stats, stream, 1.0)


def logp_forward_ex(logits: torch.Tensor, targets: torch.Tensor,
                    vocab_real: Optional[int] = None, vocab_padded: Optional[int] = None,
                    active=None, ignore_index: int = -100, inv_temperature: float = 1.0,
                    logp: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    stats: Optional[torch.Tensor] = None, stream=None):
    """logp_forward for BF16 / FP16 / FP32 logits scored as fl32(x * inv_temperature)."""
    return _forward("logp_forward_ex", logits, targets, vocab_real, vocab_padded, active,
                    ignore_index, logp, lse, stats, stream, inv_temperature)


def _backward(fn: str, logits, targets, grad_logp, stats, vocab_real, vocab_padded, col_begin,
              col_end, active, ignore_index, dlogits, stream, inv_temperature):
    ex = fn.endswith("_ex")
    logits = _matrix("logits", logits, tuple(DTYPES) if ex else torch.bfloat16)
    n, width = logits.shape
    dev = logits.device
    col_end = col_begin + width if col_end is None else int(col_end)
    vocab_padded = col_end if vocab_padded is None else int(vocab_padded)
    vocab_real = vocab_padded if vocab_real is None else int(vocab_real)
    if col_end - col_begin > width:
        raise ValueError("logits view is narrower than [col_begin, col_end)")
    targets = _rows("targets", targets, torch.int64, n, dev)
    grad_logp = _rows("grad_logp", grad_logp, torch.float32, n, dev)
    active = _active(active, n, dev)
    if stats.shape != (n, 2) or stats.dtype != torch.float32 or not stats.is_contiguous() \
            or stats.device != dev:
        raise ValueError("stats must be a contiguous float32 [n, 2] tensor on the logits device")
    if dlogits is None:
        dlogits = torch.empty((n, col_end - col_begin), dtype=logits.dtype, device=dev)
    dlogits = _matrix("dlogits", dlogits, logits.dtype)
    if dlogits.shape[0] != n or dlogits.shape[1] < col_end - col_begin or dlogits.device != dev:
        raise ValueError("dlogits must be [n, >= col_end - col_begin] on the logits device")
    args = (_ptr(logits), _ld(logits), n, vocab_real, vocab_padded, int(col_begin), col_end,
            _ptr(targets), _ptr(active), int(ignore_index), _ptr(grad_logp), _ptr(stats),
            _ptr(dlogits), _ld(dlogits), _stream(dev, stream))
    if ex:
        st = _lib.logp_backward_ex(DTYPES[logits.dtype], float(inv_temperature), *args)
    else:
        st = _lib.logp_backward(*args)
    _check(fn, st)
    return dlogits


def logp_backward(logits: torch.Tensor, targets: torch.Tensor, grad_logp: torch.Tensor,
                  stats: torch.Tensor, vocab_real: Optional[int] = None,
                  vocab_padded: Optional[int] = None, col_begin: int = 0,
                  col_end: Optional[int] = None, active=None, ignore_index: int = -100,
                  dlogits: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """BF16 dlogits over columns [col_begin, col_end) (``logits`` is that column view)."""
    return _backward("logp_backward", logits, targets, grad_logp, stats, vocab_real,
                     vocab_padded, col_begin, col_end, active, ignore_index, dlogits, stream, 1.0)


def logp_backward_ex(logits: torch.Tensor, targets: torch.Tensor, grad_logp: torch.Tensor,
                     stats: torch.Tensor, vocab_real: Optional[int] = None,
                     vocab_padded: Optional[int] = None, col_begin: int = 0,
                     col_end: Optional[int] = None, active=None, ignore_index: int = -100,
                     inv_temperature: float = 1.0, dlogits: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """logp_backward for BF16 / FP16 / FP32 logits scored as fl32(x * inv_temperature);
    dlogits has the logits' dtype and includes the factor inv_temperature."""
    return _backward("logp_backward_ex", logits, targets, grad_logp, stats, vocab_real,
                     vocab_padded, col_begin, col_end, active, ignore_index, dlogits, stream,
                     inv_temperature)


def _shard_slot(partials: torch.Tensor, n: int, col_begin: int, col_end: int) -> int:
    """Slot of tile col_begin / TILE_COLS in the float32 [n, L, 3] partials buffer, after
    checking that every tile of the shard [col_begin, col_end) has its slot inside the
    buffer.  The C side sees only the first slot and the row stride, so a buffer with too
    few tiles per row would let one row's entries run into the next row's."""
    if not isinstance(partials, torch.Tensor) or partials.dim() != 3 \
            or partials.shape[0] != n or partials.shape[2] != 3 \
            or partials.dtype != torch.float32 or partials.stride(2) != 1 \
            or partials.stride(1) != 3:
        raise ValueError("partials must be float32 [n, L, 3] with packed triples")
    col_begin, col_end = int(col_begin), int(col_end)
    if col_begin < 0 or col_begin % TILE_COLS != 0:
        raise ValueError("col_begin must be a non-negative tile boundary")
    first = col_begin // TILE_COLS
    tiles = max(1, -(-(col_end - col_begin) // TILE_COLS))
    if first + tiles > partials.shape[1]:
        raise ValueError(f"the shard's tiles {first}..{first + tiles - 1} run past the "
                         f"{partials.shape[1]} tiles per row of the partials buffer")
    return first


def _partials(fn: str, logits, targets, vocab_real, vocab_padded, col_begin, col_end, partials,
              active, ignore_index, stream, inv_temperature):
    ex = fn.endswith("_ex")
    if not isinstance(logits, torch.Tensor):
        raise TypeError("logits must be a torch.Tensor")
    slot = _shard_slot(partials, logits.shape[0], col_begin, col_end)
    logits = _matrix("logits", logits, tuple(DTYPES) if ex else torch.bfloat16)
    n = logits.shape[0]
    dev = logits.device
    targets = _rows("targets", targets, torch.int64, n, dev)
    active = _active(active, n, dev)
    if partials.device != dev:
        raise ValueError(f"partials is on {partials.device}, logits on {dev}")
    first = partials[:, slot]
    ldp = partials.stride(0) // 3 if partials.stride(0) % 3 == 0 else -1
    args = (_ptr(logits), _ld(logits), n, int(vocab_real), int(vocab_padded), int(col_begin),
            int(col_end), _ptr(targets), _ptr(active), int(ignore_index), first.data_ptr(), ldp,
            _stream(dev, stream))
    if ex:
        st = _lib.logp_partials_ex(DTYPES[logits.dtype], float(inv_temperature), *args)
    else:
        st = _lib.logp_partials(*args)
    _check(fn, st)
    return partials


def logp_partials(logits: torch.Tensor, targets: torch.Tensor, vocab_real: int,
                  vocab_padded: int, col_begin: int, col_end: int, partials: torch.Tensor,
                  active=None, ignore_index: int = -100, stream=None) -> torch.Tensor:
    """Write the (m, s, sel) partials of the shard [col_begin, col_end) into ``partials``.

    ``logits`` is the shard's column view; ``partials`` is the full float32 [n, L, 3]
    buffer, whose tiles col_begin/TILE_COLS onward are written.
    """
    return _partials("logp_partials", logits, targets, vocab_real, vocab_padded, col_begin,
                     col_end, partials, active, ignore_index, stream, 1.0)


def logp_partials_ex(logits: torch.Tensor, targets: torch.Tensor, vocab_real: int,
                     vocab_padded: int, col_begin: int, col_end: int, partials: torch.Tensor,
                     active=None, ignore_index: int = -100, inv_temperature: float = 1.0,
                     stream=None) -> torch.Tensor:
    """logp_partials for BF16 / FP16 / FP32 logits scored as fl32(x * inv_temperature)."""
    return _partials("logp_partials_ex", logits, targets, vocab_real, vocab_padded, col_begin,
                     col_end, partials, active, ignore_index, stream, inv_temperature)


def logp_merge(partials: torch.Tensor, targets: torch.Tensor, vocab_real: int,
               num_tiles: Optional[int] = None, active=None, ignore_index: int = -100,
               logp: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               stats: Optional[torch.Tensor] = None, stream=None):
    """Fixed-order merge of float32 [n, L, 3] partials -> (logp, lse, stats)."""
    if partials.dim() != 3 or partials.shape[2] != 3 or partials.dtype != torch.float32 \
            or partials.stride(2) != 1 or partials.stride(1) != 3 \
            or partials.device.type != "cuda":
        raise ValueError("partials must be a float32 GPU tensor [n, L, 3] of packed triples")
    n, L, _ = partials.shape
    dev = partials.device
    num_tiles = L if num_tiles is None else int(num_tiles)
    targets = _rows("targets", targets, torch.int64, n, dev)
    active = _active(active, n, dev)
    if logp is None:
        logp = torch.empty(n, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(n, dtype=torch.float32, device=dev)
    if stats is None:
        stats = torch.empty((n, 2), dtype=torch.float32, device=dev)
    ldp = partials.stride(0) // 3 if partials.stride(0) % 3 == 0 else -1
    st = _lib.logp_merge(_ptr(partials), ldp, n, num_tiles, int(vocab_real), _ptr(targets),
                         _ptr(active), int(ignore_index), _ptr(logp), _ptr(lse), _ptr(stats),
                         _stream(dev, stream))
    _check("logp_merge", st)
    return logp, lse, stats


def logp_check_targets(targets: torch.Tensor, vocab_real: int, active=None,
                       ignore_index: int = -100, bad_count: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Device int64 [1]: active rows whose target is neither ignore_index nor in range."""
    if targets.dtype != torch.int64 or targets.dim() != 1 or targets.device.type != "cuda":
        raise ValueError("targets must be a 1-D int64 GPU tensor")
    dev = targets.device
    n = targets.shape[0]
    if n > 1 and targets.stride(0) != 1:
        raise ValueError("targets must be contiguous")
    active = _active(active, n, dev)
    if bad_count is None:
        bad_count = torch.empty(1, dtype=torch.int64, device=dev)
    st = _lib.logp_check_targets(_ptr(targets), _ptr(active), n, int(vocab_real),
                                 int(ignore_index), _ptr(bad_count), _stream(dev, stream))
    _check("logp_check_targets", st)
    return bad_count


__all__ = ["DTYPES", "EXPORTED", "LIB_PATH", "LogpError", "STATUS", "TILE_COLS",
           "FWD_MAX_TILES", "library", "logp_forward", "logp_forward_ex", "logp_backward",
           "logp_backward_ex", "logp_partials", "logp_partials_ex", "logp_merge",
           "logp_num_tiles", "logp_check_targets", "logp_status_string"]
