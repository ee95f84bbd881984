"""Python binding of the deterministic GRPO loss (C ABI in ``include/grpo_loss.h``).

Argument marshalling only, like the log-probability binding: tensors are checked, outputs
allocated with torch when none are passed, and the C entry points called on torch's current
stream.  Every step runs in the HIP kernels.

Tensor conventions:
  * per-token arrays (logp, old_logp, ref_logp, dlogp): float32 ``[n_seqs, seq_len]`` views
    with unit column stride, all with the same row stride; mask: uint8/bool of the same
    shape and row stride, or None.
  * adv: float32 ``[n_seqs]`` (one advantage per sequence).
  * seq_stats / partials: int32 ``[..., 4]`` holding grpo_partial_t records
    (pg_sum and kl_sum as float32 bits, clipped, tokens); :func:`partial_fields` decodes.
  * loss: int64 ``[6]`` holding one grpo_loss_t; :func:`loss_fields` decodes.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _check, _ptr, _stream, library

TOKEN_TILE = 256
MAX_SEQ_LEN = TOKEN_TILE * 4096
MODES = {"token_mean": 0, "seq_mean": 1, "seq_sum_token_mean": 2}
EXPORTED = ("grpo_advantages", "grpo_token_counts", "grpo_loss", "grpo_loss_partials",
            "grpo_loss_merge", "grpo_loss_reduce")


class GrpoParams(ctypes.Structure):
    _fields_ = [("eps_low", ctypes.c_float), ("eps_high", ctypes.c_float),
                ("beta", ctypes.c_float), ("mode", ctypes.c_int32),
                ("norm_tokens", ctypes.c_int64), ("norm_seqs", ctypes.c_int64)]


def _declare(lib):
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    PP = ctypes.POINTER(GrpoParams)
    lib.grpo_advantages.argtypes = [P, I64, I64, F, I32, P, P]
    lib.grpo_token_counts.argtypes = [P, I64, I64, I64, I64, I64, P, P]
    lib.grpo_loss.argtypes = [P, P, P, P, P, I64, I64, I64, PP, P, P, P, P]
    lib.grpo_loss_partials.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, P, PP, P, I64,
                                       P, P]
    lib.grpo_loss_merge.argtypes = [P, I64, I64, I64, P, P]
    lib.grpo_loss_reduce.argtypes = [P, I64, PP, P, P]
    for fn in EXPORTED:
        getattr(lib, fn).restype = I32


_lib = library()
_declare(_lib)


def params(mode: str = "token_mean", eps_low: float = 0.2, eps_high: float = 0.2,
           beta: float = 0.0, norm_tokens: int = 0, norm_seqs: int = 0) -> GrpoParams:
    if mode not in MODES:
        raise ValueError(f"mode must be one of {tuple(MODES)}")
    return GrpoParams(float(eps_low), float(eps_high), float(beta), MODES[mode],
                      int(norm_tokens), int(norm_seqs))


def _tokens(name: str, t: Optional[torch.Tensor], dtype, shape, ld: Optional[int], device):
    if t is None:
        return None, ld
    if t.dtype == torch.bool and dtype == torch.uint8:
        t = t.view(torch.uint8)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if t.dim() != 2 or tuple(t.shape) != tuple(shape) or (shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a [{shape[0]}, {shape[1]}] view with unit column "
                         "stride")
    row = int(t.stride(0)) if shape[0] > 1 else (ld if ld is not None else int(shape[1]))
    if ld is not None and row != ld:
        raise ValueError(f"{name}: every per-token array must have the same row stride")
    return t, row


def _vector(name: str, t: torch.Tensor, dtype, n: int, device):
    if t.dtype != dtype or t.device != device or t.dim() != 1 or t.shape[0] != n or \
            (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous {dtype} [{n}] tensor on {device}")
    return t


def partial_fields(t: torch.Tensor) -> dict:
    """Decode grpo_partial_t records (an int32 [..., 4] tensor) into named tensors."""
    return {"pg_sum": t[..., 0].contiguous().view(torch.float32),
            "kl_sum": t[..., 1].contiguous().view(torch.float32),
            "clipped": t[..., 2], "tokens": t[..., 3]}


def loss_fields(t: torch.Tensor) -> dict:
    """Decode one grpo_loss_t (an int64 [6] tensor) into Python numbers (synchronizes)."""
    h = t.cpu()
    f = h[:2].view(torch.float32).tolist()
    i = h[2:].tolist()
    return {"loss": f[0], "pg_loss": f[1], "kl_loss": f[2], "clip_frac": f[3],
            "tokens": i[0], "sequences": i[1], "clipped": i[2], "norm": i[3]}


def grpo_advantages(rewards: torch.Tensor, group_size: int, eps: float = 1e-6,
                    scale_by_std: bool = True, adv: Optional[torch.Tensor] = None, stream=None):
    """Group-normalized advantages of float32 rewards [n] -> adv [n]."""
    n = rewards.shape[0]
    _vector("rewards", rewards, torch.float32, n, rewards.device)
    if adv is None:
        adv = torch.empty_like(rewards)
    _vector("adv", adv, torch.float32, n, rewards.device)
    _check("grpo_advantages", _lib.grpo_advantages(
        _ptr(rewards), n, int(group_size), float(eps), 1 if scale_by_std else 0, _ptr(adv),
        _stream(rewards.device, stream)))
    return adv


def grpo_token_counts(mask: torch.Tensor, t_begin: int = 0, t_end: Optional[int] = None,
                      counts: Optional[torch.Tensor] = None, stream=None):
    """Active tokens of each row of a uint8/bool mask [n_seqs, seq_len] in [t_begin, t_end)."""
    n, T = mask.shape
    mask, ld = _tokens("mask", mask, torch.uint8, (n, T), None, mask.device)
    t_end = T if t_end is None else int(t_end)
    if counts is None:
        counts = torch.empty(n, dtype=torch.int32, device=mask.device)
    _vector("counts", counts, torch.int32, n, mask.device)
    _check("grpo_token_counts", _lib.grpo_token_counts(
        _ptr(mask), n, T, ld, int(t_begin), t_end, _ptr(counts), _stream(mask.device, stream)))
    return counts


def grpo_loss(logp: torch.Tensor, old_logp: torch.Tensor, adv: torch.Tensor,
              ref_logp: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
              mode: str = "token_mean", eps_low: float = 0.2, eps_high: float = 0.2,
              beta: float = 0.0, norm_tokens: int = 0, norm_seqs: int = 0,
              need_grad: bool = True, seq_stats: Optional[torch.Tensor] = None,
              loss: Optional[torch.Tensor] = None, dlogp: Optional[torch.Tensor] = None,
              stream=None):
    """GRPO loss over whole sequences -> (loss int64[6], seq_stats int32[n,4], dlogp or None)."""
    n, T = logp.shape
    dev = logp.device
    logp, ld = _tokens("logp", logp, torch.float32, (n, T), None, dev)
    old_logp, ld = _tokens("old_logp", old_logp, torch.float32, (n, T), ld, dev)
    ref_logp, ld = _tokens("ref_logp", ref_logp, torch.float32, (n, T), ld, dev)
    mask, ld = _tokens("mask", mask, torch.uint8, (n, T), ld, dev)
    _vector("adv", adv, torch.float32, n, dev)
    if seq_stats is None:
        seq_stats = torch.empty((n, 4), dtype=torch.int32, device=dev)
    if loss is None:
        loss = torch.empty(6, dtype=torch.int64, device=dev)
    if need_grad and dlogp is None:
        dlogp = torch.empty_strided((n, T), (ld, 1), dtype=torch.float32, device=dev) \
            if ld == T else torch.zeros((n, ld), dtype=torch.float32, device=dev)[:, :T]
    if dlogp is not None:
        dlogp, ld = _tokens("dlogp", dlogp, torch.float32, (n, T), ld, dev)
    if seq_stats.shape != (n, 4) or seq_stats.dtype != torch.int32 or \
            not seq_stats.is_contiguous() or seq_stats.device != dev:
        raise ValueError("seq_stats must be a contiguous int32 [n, 4] tensor")
    if loss.shape != (6,) or loss.dtype != torch.int64 or loss.device != dev:
        raise ValueError("loss must be an int64 [6] tensor")
    p = params(mode, eps_low, eps_high, beta, norm_tokens, norm_seqs)
    _check("grpo_loss", _lib.grpo_loss(
        _ptr(logp), _ptr(old_logp), _ptr(ref_logp), _ptr(adv), _ptr(mask), n, T,
        ld if ld is not None else T, ctypes.byref(p), _ptr(seq_stats), _ptr(loss), _ptr(dlogp),
        _stream(dev, stream)))
    return loss, seq_stats, dlogp


def grpo_loss_partials(logp: torch.Tensor, old_logp: torch.Tensor, adv: torch.Tensor,
                       seq_len: int, t_begin: int, partials: torch.Tensor,
                       ref_logp: Optional[torch.Tensor] = None,
                       mask: Optional[torch.Tensor] = None,
                       seq_tokens: Optional[torch.Tensor] = None,
                       dlogp: Optional[torch.Tensor] = None, mode: str = "token_mean",
                       eps_low: float = 0.2, eps_high: float = 0.2, beta: float = 0.0,
                       norm_tokens: int = 0, norm_seqs: int = 0, stream=None):
    """Tile partials of the token range held by the column views (logp = full[:, t0:t1], ...)
    into the full int32 [n, L, 4] partials array (L = ceil(seq_len / 256)); writes dlogp."""
    n, width = logp.shape
    dev = logp.device
    logp, ld = _tokens("logp", logp, torch.float32, (n, width), None, dev)
    old_logp, ld = _tokens("old_logp", old_logp, torch.float32, (n, width), ld, dev)
    ref_logp, ld = _tokens("ref_logp", ref_logp, torch.float32, (n, width), ld, dev)
    mask, ld = _tokens("mask", mask, torch.uint8, (n, width), ld, dev)
    dlogp, ld = _tokens("dlogp", dlogp, torch.float32, (n, width), ld, dev)
    _vector("adv", adv, torch.float32, n, dev)
    if seq_tokens is not None:
        _vector("seq_tokens", seq_tokens, torch.int32, n, dev)
    L = -(-int(seq_len) // TOKEN_TILE)
    if partials.dim() != 3 or partials.shape[0] != n or partials.shape[2] != 4 or \
            partials.dtype != torch.int32 or not partials.is_contiguous() or \
            partials.device != dev or partials.shape[1] < L:
        raise ValueError(f"partials must be a contiguous int32 [{n}, >={L}, 4] tensor")
    ldp = partials.shape[1]
    tile0 = int(t_begin) // TOKEN_TILE
    base = partials.data_ptr() + tile0 * 16
    p = params(mode, eps_low, eps_high, beta, norm_tokens, norm_seqs)
    _check("grpo_loss_partials", _lib.grpo_loss_partials(
        _ptr(logp), _ptr(old_logp), _ptr(ref_logp), _ptr(adv), _ptr(mask), n, int(seq_len),
        ld if ld is not None else width, int(t_begin), int(t_begin) + width, _ptr(seq_tokens),
        ctypes.byref(p), base, ldp, _ptr(dlogp), _stream(dev, stream)))
    return partials


def grpo_loss_merge(partials: torch.Tensor, num_tiles: Optional[int] = None,
                    seq_stats: Optional[torch.Tensor] = None, stream=None):
    """Per-sequence sums from tile partials int32 [n, ldp, 4] -> seq_stats int32 [n, 4]."""
    n, ldp, _ = partials.shape
    dev = partials.device
    if partials.dtype != torch.int32 or not partials.is_contiguous():
        raise ValueError("partials must be a contiguous int32 [n, ldp, 4] tensor")
    num_tiles = ldp if num_tiles is None else int(num_tiles)
    if seq_stats is None:
        seq_stats = torch.empty((n, 4), dtype=torch.int32, device=dev)
    _check("grpo_loss_merge", _lib.grpo_loss_merge(
        _ptr(partials), ldp, n, num_tiles, _ptr(seq_stats), _stream(dev, stream)))
    return seq_stats


def grpo_loss_reduce(seq_stats: torch.Tensor, mode: str = "token_mean", beta: float = 0.0,
                     norm_tokens: int = 0, norm_seqs: int = 0,
                     loss: Optional[torch.Tensor] = None, stream=None):
    """The loss from per-sequence sums int32 [n, 4] -> loss int64 [6]."""
    n = seq_stats.shape[0]
    dev = seq_stats.device
    if seq_stats.dtype != torch.int32 or seq_stats.dim() != 2 or seq_stats.shape[1] != 4 or \
            not seq_stats.is_contiguous():
        raise ValueError("seq_stats must be a contiguous int32 [n, 4] tensor")
    if loss is None:
        loss = torch.empty(6, dtype=torch.int64, device=dev)
    p = params(mode, 0.2, 0.2, beta, norm_tokens, norm_seqs)
    _check("grpo_loss_reduce", _lib.grpo_loss_reduce(
        _ptr(seq_stats), n, ctypes.byref(p), _ptr(loss), _stream(dev, stream)))
    return loss
