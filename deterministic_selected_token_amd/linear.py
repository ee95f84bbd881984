"""Python binding of the fused LM-head + selected-token logp (C ABI in include/linear_logp.h).

Argument marshalling only: tensors are checked, outputs allocated with torch when none are
passed, and the C entry points called on torch's current stream.  The logits h W^T are
formed and reduced inside the HIP kernel; the merge is the log-probability library's
``logp_merge``.

Tensor conventions:
  * hidden: bfloat16 ``[n, H]`` with unit column stride (row stride a multiple of 8 and at
    most 262144, start 16-byte aligned); weight: bfloat16 rows of the LM head ``[rows, H]``
    (a vocab shard is a row slice ``W[c0:c1]``); H a multiple of 8.
  * partials: float32 ``[n, L, 3]`` of (m_l, s_l, sel_l), ``L = logp_num_tiles(vocab_padded)``.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import (TILE_COLS, _active, _check, _lib, _ptr, _rows, _shard_slot, _stream,
               logp_merge, logp_num_tiles)

EXPORTED = ("linear_logp_partials", "linear_logp_partials_ex", "linear_logp_partials_ws",
            "linear_logp_partials_workspace", "linear_logp_backward",
            "linear_logp_backward_ex", "linear_logp_backward_workspace",
            "linear_logp_backward_noalloc", "linear_logp_backward_bf16",
            "linear_logp_backward_bf16_workspace", "linear_logp_partials_save",
            "linear_logp_backward_saved")
MAX_HIDDEN = 65536
MAX_LD = 262144
BWD_MAX_ROWS = 8388608
BWD_MAX_CHUNK = 1048576
NOALLOC_SCRATCH_BYTES = 128 << 20
MAX_SAVED_LD = 1 << 31
DEFAULT_CHUNK_COLS = 4 * TILE_COLS

_P, _I64 = ctypes.c_void_p, ctypes.c_int64
_lib.linear_logp_partials.argtypes = [_P, _I64, _I64, _I64, _P, _I64, _I64, _I64, _I64, _I64,
                                      _P, _P, _I64, _P, _I64, _P]
_lib.linear_logp_partials.restype = ctypes.c_int32
_lib.linear_logp_partials_ex.argtypes = [ctypes.c_float] + _lib.linear_logp_partials.argtypes
_lib.linear_logp_partials_ex.restype = ctypes.c_int32
_lib.linear_logp_partials_ws.argtypes = (_lib.linear_logp_partials_ex.argtypes[:-1]
                                         + [_P, _I64, _P])
_lib.linear_logp_partials_ws.restype = ctypes.c_int32
_lib.linear_logp_partials_workspace.argtypes = [_I64, _I64, _I64, _I64]
_lib.linear_logp_partials_workspace.restype = _I64
_lib.linear_logp_backward.argtypes = [_P, _I64, _I64, _I64, _P, _I64, _I64, _I64, _I64, _I64,
                                      _P, _P, _I64, _P, _P, _P, _I64, _P, _I64, _P, _I64, _I64,
                                      _P]
_lib.linear_logp_backward.restype = ctypes.c_int32
_lib.linear_logp_backward_ex.argtypes = [ctypes.c_float] + _lib.linear_logp_backward.argtypes
_lib.linear_logp_backward_ex.restype = ctypes.c_int32
_lib.linear_logp_backward_noalloc.argtypes = (_lib.linear_logp_backward_ex.argtypes[:20]
                                               + [_I64, _P])
_lib.linear_logp_backward_noalloc.restype = ctypes.c_int32
_lib.linear_logp_backward_workspace.argtypes = [_I64, _I64, _I64]
_lib.linear_logp_backward_workspace.restype = _I64
_lib.linear_logp_backward_bf16.argtypes = _lib.linear_logp_backward_ex.argtypes
_lib.linear_logp_backward_bf16.restype = ctypes.c_int32
_lib.linear_logp_backward_bf16_workspace.argtypes = [_I64, _I64, _I64]
_lib.linear_logp_backward_bf16_workspace.restype = _I64
_lib.linear_logp_partials_save.argtypes = (_lib.linear_logp_partials_ex.argtypes[:-1]
                                           + [_P, _I64, _P, _I64, _P])
_lib.linear_logp_partials_save.restype = ctypes.c_int32
_lib.linear_logp_backward_saved.argtypes = ([ctypes.c_float, _P, _I64]
                                            + _lib.linear_logp_backward.argtypes[:-4]
                                            + [ctypes.c_int32, _P, _I64, _I64, _P])
_lib.linear_logp_backward_saved.restype = ctypes.c_int32
_OUT_DTYPES = (torch.float32, torch.bfloat16)
_DTYPE_CODE = {torch.float32: 2, torch.bfloat16: 0}  # logp_dtype_t


def _bf16_rows(name: str, t: torch.Tensor, device=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a bfloat16 tensor")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t


def _row_stride(t: torch.Tensor) -> int:
    return int(t.stride(0)) if t.shape[0] > 1 else int(max(t.shape[1], t.stride(0), 8))


def kept_logits_buffer(n: int, width: int, device=None) -> torch.Tensor:
    """An uninitialised float32 [n, width] tensor laid out as linear_logp_partials(...,
    logits=) needs: rows 16-byte aligned (a row stride that is a multiple of 4 floats)."""
    return torch.empty((n, (int(width) + 3) // 4 * 4), dtype=torch.float32,
                       device=device)[:, :int(width)]


def _saved_logits(t: torch.Tensor, n: int, width: int, device) -> tuple:
    """(pointer, row stride) of a float32 [n, >= width] tensor of kept logits with unit column
    stride on ``device``."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != device:
        raise ValueError(f"logits must be a float32 tensor on {device}")
    if t.dim() != 2 or t.shape[0] != n or t.shape[1] < width or \
            (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"logits must be [{n}, >= {width}] with unit column stride")
    ld = int(t.stride(0)) if n > 1 else int(-(-max(t.shape[1], 4) // 4) * 4)
    return t.data_ptr(), ld


def linear_logp_partials_workspace(n: int, vocab_real: int, col_begin: int,
                                   col_end: int) -> int:
    """Workspace bytes with which linear_logp_partials can always balance its last rounds
    (-1 when out of range)."""
    return int(_lib.linear_logp_partials_workspace(int(n), int(vocab_real), int(col_begin),
                                                   int(col_end)))


def linear_logp_partials(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                         vocab_real: int, vocab_padded: int, col_begin: int, col_end: int,
                         partials: torch.Tensor, active=None, ignore_index: int = -100,
                         stream=None, inv_temperature: float = 1.0,
                         workspace: Optional[torch.Tensor] = None,
                         logits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Write the (m, s, sel) partials of vocab columns [col_begin, col_end) of the scored
    logits fl32(h W^T * inv_temperature) into the full ``partials`` buffer; ``weight`` is the
    row slice W[col_begin:col_end].  With a ``workspace`` (a contiguous uint8 GPU tensor,
    linear_logp_partials_workspace bytes always suffice) linear_logp_partials_ws balances the
    launch's last rounds over every CU, with bitwise the same partials; without one,
    inv_temperature = 1 calls the plain entry point.  With ``logits`` (float32 [n, >= col_end -
    col_begin], 16-byte aligned rows) linear_logp_partials_save also keeps the scored logits
    of the view's real columns there, for linear_logp_backward(..., logits=)."""
    if not isinstance(hidden, torch.Tensor):
        raise TypeError("hidden must be a torch.Tensor")
    slot = _shard_slot(partials, hidden.shape[0], col_begin, col_end)
    hidden = _bf16_rows("hidden", hidden)
    dev = hidden.device
    weight = _bf16_rows("weight", weight, dev)
    n, H = hidden.shape
    if weight.shape[1] != H:
        raise ValueError("hidden and weight must have the same hidden size")
    targets = _rows("targets", targets, torch.int64, n, dev)
    active = _active(active, n, dev)
    if partials.device != dev:
        raise ValueError(f"partials is on {partials.device}, hidden on {dev}")
    rows_needed = max(0, min(col_end, vocab_real) - col_begin)
    if weight.shape[0] < rows_needed:
        raise ValueError(f"weight holds {weight.shape[0]} rows, the range needs {rows_needed}")
    first = partials[:, slot]
    ldp = partials.stride(0) // 3 if partials.stride(0) % 3 == 0 else -1
    args = (_ptr(hidden), _row_stride(hidden), n, H, _ptr(weight), _row_stride(weight),
            int(vocab_real), int(vocab_padded), int(col_begin), int(col_end), _ptr(targets),
            _ptr(active), int(ignore_index), first.data_ptr(), ldp, _stream(dev, stream))
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or
                                  workspace.device != dev or workspace.dtype != torch.uint8 or
                                  not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 GPU tensor on the same device")
    if logits is not None:
        zp, ldz = _saved_logits(logits, n, int(col_end) - int(col_begin), dev)
        _check("linear_logp_partials_save", _lib.linear_logp_partials_save(
            float(inv_temperature), *args[:-1], zp, ldz,
            _ptr(workspace) if workspace is not None else None,
            workspace.numel() if workspace is not None else 0, args[-1]))
    elif workspace is not None:
        _check("linear_logp_partials_ws", _lib.linear_logp_partials_ws(
            float(inv_temperature), *args[:-1], _ptr(workspace), workspace.numel(), args[-1]))
    elif inv_temperature == 1.0:
        _check("linear_logp_partials", _lib.linear_logp_partials(*args))
    else:
        _check("linear_logp_partials_ex",
               _lib.linear_logp_partials_ex(float(inv_temperature), *args))
    return partials


def linear_logp_forward(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                        vocab_real: Optional[int] = None, vocab_padded: Optional[int] = None,
                        active=None, ignore_index: int = -100,
                        partials: Optional[torch.Tensor] = None,
                        logp: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        stats: Optional[torch.Tensor] = None, stream=None,
                        inv_temperature: float = 1.0,
                        workspace: Optional[torch.Tensor] = None, balance: bool = True,
                        logits: Optional[torch.Tensor] = None):
    """logp, LSE and (M, S) of the scored logits fl32(h W^T * inv_temperature) over the
    whole vocabulary: linear_logp_partials over all tiles, then logp_merge -> (logp, lse,
    stats).  balance=True (the default) passes a workspace, allocated with torch when none is
    given, so that the last rounds spread over every CU; the results are the same bits.
    ``logits`` (float32 [n, >= vocab_padded], rows 16-byte aligned: kept_logits_buffer(n,
    vocab_padded)) keeps the scored logits for the backward."""
    vocab_padded = weight.shape[0] if vocab_padded is None else int(vocab_padded)
    vocab_real = vocab_padded if vocab_real is None else int(vocab_real)
    n = hidden.shape[0]
    L = logp_num_tiles(vocab_padded)
    if partials is None:
        partials = torch.empty((n, L, 3), dtype=torch.float32, device=hidden.device)
    if balance and workspace is None and n > 0:
        need = linear_logp_partials_workspace(n, vocab_real, 0, vocab_padded)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=hidden.device)
    linear_logp_partials(hidden, weight, targets, vocab_real, vocab_padded, 0, vocab_padded,
                         partials, active=active, ignore_index=ignore_index, stream=stream,
                         inv_temperature=inv_temperature,
                         workspace=workspace if balance else None, logits=logits)
    return logp_merge(partials, targets, vocab_real, num_tiles=L, active=active,
                      ignore_index=ignore_index, logp=logp, lse=lse, stats=stats,
                      stream=stream)


def linear_logp_backward_workspace(n: int, hidden_size: int,
                                   chunk_cols: int = DEFAULT_CHUNK_COLS,
                                   out_dtype: torch.dtype = torch.float32) -> int:
    """Workspace bytes that linear_logp_backward needs for gradients of ``out_dtype`` (-1 when
    out of range)."""
    if out_dtype not in _OUT_DTYPES:
        raise ValueError(f"out_dtype must be one of {_OUT_DTYPES}")
    fn = _lib.linear_logp_backward_workspace if out_dtype == torch.float32 \
        else _lib.linear_logp_backward_bf16_workspace
    return int(fn(int(n), int(hidden_size), int(chunk_cols)))


def linear_logp_backward(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                         grad_logp: torch.Tensor, stats: torch.Tensor,
                         vocab_real: Optional[int] = None, vocab_padded: Optional[int] = None,
                         col_begin: int = 0, col_end: Optional[int] = None, active=None,
                         ignore_index: int = -100, inv_temperature: float = 1.0,
                         chunk_cols: int = DEFAULT_CHUNK_COLS,
                         dhidden: Optional[torch.Tensor] = None,
                         dweight: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None,
                         noalloc: bool = False, out_dtype: torch.dtype = torch.float32,
                         logits: Optional[torch.Tensor] = None):
    """(dhidden [n, H], dweight [col_end - col_begin, H]) of ``out_dtype``: the gradients of
    sum_t grad_logp[t] logp[t] with respect to hidden and to the weight rows
    W[col_begin:col_end] (``weight`` is that row slice), for the logits of linear_logp_forward
    with the same inv_temperature; ``stats`` is the forward's (M, S).  out_dtype float32 calls
    linear_logp_backward(_ex); bfloat16 calls linear_logp_backward_bf16, whose outputs are the
    FP32 results rounded once to nearest even inside the library.  The workspace (a uint8 GPU
    tensor of at least linear_logp_backward_workspace(n, H, chunk_cols, out_dtype) bytes) is
    allocated with torch when none is passed.  noalloc=True (float32 only) calls
    linear_logp_backward_noalloc instead, which stages in the library's static scratch array
    (at most NOALLOC_SCRATCH_BYTES of workspace) and allocates nothing; pass dhidden and
    dweight as well to keep torch from allocating them.  ``logits`` (float32 [n, >= col_end -
    col_begin], the scored logits linear_logp_partials(..., logits=) kept for this view)
    calls linear_logp_backward_saved, which reads them instead of forming h W^T again: the
    same bits, two products instead of three."""
    if out_dtype not in _OUT_DTYPES:
        raise ValueError(f"out_dtype must be one of {_OUT_DTYPES}")
    if noalloc and out_dtype != torch.float32:
        raise ValueError("noalloc writes float32 gradients only")
    if noalloc and logits is not None:
        raise ValueError("noalloc recomputes the logits; it takes no saved logits")
    hidden = _bf16_rows("hidden", hidden)
    dev = hidden.device
    weight = _bf16_rows("weight", weight, dev)
    n, H = hidden.shape
    if weight.shape[1] != H:
        raise ValueError("hidden and weight must have the same hidden size")
    vocab_padded = col_begin + weight.shape[0] if vocab_padded is None else int(vocab_padded)
    vocab_real = vocab_padded if vocab_real is None else int(vocab_real)
    col_end = vocab_padded if col_end is None else int(col_end)
    width = col_end - col_begin
    targets = _rows("targets", targets, torch.int64, n, dev)
    grad_logp = _rows("grad_logp", grad_logp, torch.float32, n, dev)
    active = _active(active, n, dev)
    if stats.shape != (n, 2) or stats.dtype != torch.float32 or stats.device != dev \
            or (n > 0 and stats.stride() != (2, 1)):
        raise ValueError("stats must be a contiguous float32 [n, 2] tensor")
    rows_needed = max(0, min(col_end, vocab_real) - col_begin)
    if weight.shape[0] < rows_needed:
        raise ValueError(f"weight holds {weight.shape[0]} rows, the range needs {rows_needed}")
    if dhidden is None:
        dhidden = torch.empty((n, H), dtype=out_dtype, device=dev)
    if dweight is None:
        dweight = torch.empty((width, H), dtype=out_dtype, device=dev)
    for name, t, rows in (("dhidden", dhidden, n), ("dweight", dweight, width)):
        if t.dtype != out_dtype or t.device != dev or t.dim() != 2 or \
                t.shape[0] != rows or t.shape[1] != H or (H > 1 and t.stride(1) != 1):
            raise ValueError(f"{name} must be {out_dtype} [{rows}, {H}] with unit column "
                             "stride")
    need = linear_logp_backward_workspace(n, H, chunk_cols, out_dtype)
    if need < 0:
        raise ValueError("n, hidden size or chunk_cols out of range")
    head = (_ptr(hidden), _row_stride(hidden), n, H, _ptr(weight) if weight.numel() else None,
            _row_stride(weight), vocab_real, vocab_padded, int(col_begin), col_end,
            _ptr(targets), _ptr(active), int(ignore_index), _ptr(grad_logp), _ptr(stats),
            _ptr(dhidden), _row_stride(dhidden) if n else H,
            _ptr(dweight) if dweight.numel() else None, _row_stride(dweight) if width else H)
    if noalloc:  # the library's static scratch array: no workspace, nothing allocated
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        _check("linear_logp_backward_noalloc",
               _lib.linear_logp_backward_noalloc(float(inv_temperature), *head, int(chunk_cols),
                                                 _stream(dev, stream)))
        return dhidden, dweight
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 GPU tensor")
    args = head + (_ptr(workspace), workspace.numel(), int(chunk_cols), _stream(dev, stream))
    if logits is not None:
        zp, ldz = _saved_logits(logits, n, width, dev)
        _check("linear_logp_backward_saved", _lib.linear_logp_backward_saved(
            float(inv_temperature), zp, ldz, *head, _DTYPE_CODE[out_dtype], *args[-4:]))
    elif out_dtype == torch.bfloat16:
        _check("linear_logp_backward_bf16",
               _lib.linear_logp_backward_bf16(float(inv_temperature), *args))
    elif inv_temperature == 1.0:
        _check("linear_logp_backward", _lib.linear_logp_backward(*args))
    else:
        _check("linear_logp_backward_ex",
               _lib.linear_logp_backward_ex(float(inv_temperature), *args))
    return dhidden, dweight
