"""vocab_sharded_embedding_amd: the vocab-parallel embedding and LM head on MI355X.

A thin Python binding over ``libvpe.so`` (C ABI declared in ``include/vpe.h``).
Functions here only marshal arguments: they check tensor placement, dtype and
layout, allocate outputs with ``torch.empty`` when none is given, and pass raw
device pointers plus the current HIP stream to the library.  Every step of the
computation runs in the library's HIP kernels; there is no fallback path, and
loading fails loudly when the library is missing or cannot be loaded.

Names follow the C ABI: ``vpe_shard_range``, ``vpe_embed``,
``vpe_sum_partials``, ``vpe_last_token_select``, ``vpe_lmhead``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvpe.so")

VPE_OK, VPE_ERR_NULL, VPE_ERR_SHAPE, VPE_ERR_DTYPE = 0, 1, 2, 3
VPE_ERR_ALIGN, VPE_ERR_SHARD, VPE_ERR_LAUNCH, VPE_ERR_RANGE = 4, 5, 6, 7
VPE_ERR_WORKSPACE = 8
VPE_NOALLOC_SCRATCH_BYTES = 16 << 20
VPE_F32, VPE_BF16 = 0, 1
VPE_I32, VPE_I64 = 0, 1
VPE_MAX_PARTS = 64

EXPORTED_SYMBOLS = ("vpe_shard_range", "vpe_embed", "vpe_sum_partials",
                    "vpe_last_token_select", "vpe_lmhead", "vpe_lmhead_prefill",
                    "vpe_argmax_init", "vpe_lmhead_argmax", "vpe_lmhead_prefill_argmax",
                    "vpe_argmax_decode", "vpe_argmax_decode_clear", "vpe_load_shard",
                    "vpe_lmhead_logsumexp_workspace", "vpe_lmhead_logsumexp",
                    "vpe_lmhead_prefill_logsumexp", "vpe_logsumexp_combine",
                    "vpe_lmhead_logsumexp_noalloc", "vpe_status_string")


class VpeError(RuntimeError):
    """A libvpe call returned a status other than VPE_OK."""

    def __init__(self, fn: str, status: int, name: str):
        super().__init__(f"{fn} failed: {name} ({status})")
        self.status = status
        self.status_name = name


_lib = None


class StaleLibraryError(RuntimeError):
    """libvpe.so was built from sources other than the ones next to it."""


def check_library_current(path: str = LIB_PATH) -> None:
    """Raise StaleLibraryError unless the digest recorded next to the library
    when it was built equals the digest of the sources in this tree."""
    from . import build as _build
    have, want = _build.built_digest(path), _build.source_digest()
    if have != want:
        raise StaleLibraryError(
            f"{path} does not match its sources (built from "
            f"{have[:12] or 'unrecorded sources'}, tree is {want[:12]}): rebuild it with "
            "`python -m vocab_sharded_embedding_amd.build` (or __graft_entry__.build()), "
            "or set VPE_REBUILD_STALE=1 to rebuild on load")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libvpe.so.  It is built first when missing; a library whose recorded
    source digest differs from the tree's sources is refused (StaleLibraryError),
    or rebuilt when the environment sets VPE_REBUILD_STALE=1."""
    global _lib
    if _lib is not None:
        return _lib
    from . import build as _build
    if not os.path.exists(path):
        _build.build()
    try:
        check_library_current(path)
    except StaleLibraryError:
        if os.environ.get("VPE_REBUILD_STALE") != "1" or path != LIB_PATH:
            raise
        _build.build()
        check_library_current(path)
    lib = ctypes.CDLL(path)
    i64, i32, vp, ci = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int
    lib.vpe_shard_range.argtypes = [i64, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.vpe_embed.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, vp, vp]
    lib.vpe_sum_partials.argtypes = [ctypes.POINTER(vp), i32, i64, ci, vp, vp]
    lib.vpe_last_token_select.argtypes = [vp, i64, i64, ci, vp, i64, vp, vp]
    lib.vpe_lmhead.argtypes = [vp, i64, i64, vp, i64, ci, vp, i64, i64, vp]
    lib.vpe_lmhead_prefill.argtypes = [vp, i64, i64, vp, i64, vp, i64, ci, vp, i64, i64, vp]
    lib.vpe_argmax_init.argtypes = [vp, i64, vp]
    lib.vpe_lmhead_argmax.argtypes = [vp, i64, i64, vp, i64, ci, i64, vp, vp]
    lib.vpe_lmhead_prefill_argmax.argtypes = [vp, i64, i64, vp, i64, vp, i64, ci, i64, vp, vp]
    lib.vpe_argmax_decode.argtypes = [vp, i64, vp, vp, vp]
    lib.vpe_argmax_decode_clear.argtypes = [vp, i64, vp, vp, vp]
    lib.vpe_load_shard.argtypes = [vp, i64, i64, ci, ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.vpe_lmhead_logsumexp_workspace.argtypes = [i64, i64, ctypes.POINTER(i64)]
    lib.vpe_lmhead_logsumexp.argtypes = [vp, i64, i64, vp, i64, ci, vp, i64, i64, vp, vp, i64, vp]
    lib.vpe_lmhead_prefill_logsumexp.argtypes = [vp, i64, i64, vp, i64, vp, i64, ci, vp, i64,
                                                 i64, vp, vp, i64, vp]
    lib.vpe_logsumexp_combine.argtypes = [ctypes.POINTER(vp), i32, i64, vp, vp]
    lib.vpe_lmhead_logsumexp_noalloc.argtypes = [vp, i64, i64, vp, i64, ci, vp, i64, i64, vp, vp]
    for name in EXPORTED_SYMBOLS[:-1]:
        getattr(lib, name).restype = ci
    lib.vpe_status_string.argtypes = [ci]
    lib.vpe_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_name(status: int) -> str:
    return load_library().vpe_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != VPE_OK:
        raise VpeError(fn, status, status_name(status))


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return VPE_F32
    if t.dtype == torch.bfloat16:
        return VPE_BF16
    raise TypeError(f"tensor dtype must be float32 or bfloat16, got {t.dtype}")


def _itype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.int32:
        return VPE_I32
    if t.dtype == torch.int64:
        return VPE_I64
    raise TypeError(f"token ids must be int32 or int64, got {t.dtype}")


def _need_device(name: str, t) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a HIP device tensor, got device {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _same_device(*ts) -> None:
    devs = {t.device for t in ts}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")


# ---------------------------------------------------------------------------
# the five calls
# ---------------------------------------------------------------------------
def vpe_shard_range(vocab: int, tp_size: int, tp_rank: int) -> Tuple[int, int]:
    """(vocab_start, vocab_end) owned by tp_rank: contiguous V/tp rows in rank order."""
    lib = load_library()
    s, e = ctypes.c_int64(), ctypes.c_int64()
    _check("vpe_shard_range", lib.vpe_shard_range(vocab, tp_size, tp_rank,
                                                  ctypes.byref(s), ctypes.byref(e)))
    return s.value, e.value


def vpe_embed(ids, weight, vocab_start: int, out=None):
    """One shard's masked lookup: ids [*] x weight [R, D] -> out [*, D].

    Rows for ids outside [vocab_start, vocab_start + R) are +0.0.
    """
    torch = _torch()
    _need_device("ids", ids)
    _need_device("weight", weight)
    if weight.dim() != 2:
        raise ValueError("weight must be [shard_rows, dim]")
    rows, dim = weight.shape
    if out is None:
        out = torch.empty((*ids.shape, dim), dtype=weight.dtype, device=weight.device)
    _need_device("out", out)
    if out.dtype != weight.dtype or out.numel() != ids.numel() * dim:
        raise ValueError("out must have the weight's dtype and ids.numel() * dim elements")
    _same_device(ids, weight, out)
    _check("vpe_embed", load_library().vpe_embed(
        ids.data_ptr(), _itype_code(ids), ids.numel(), weight.data_ptr(), _dtype_code(weight),
        rows, dim, int(vocab_start), out.data_ptr(), _stream_handle(weight.device)))
    return out


def vpe_sum_partials(partials: Sequence, out=None):
    """Elementwise sum of same-shape partials (rank order, fp32, one rounding)."""
    torch = _torch()
    parts = list(partials)
    if not parts:
        raise ValueError("need at least one partial")
    for i, p in enumerate(parts):
        _need_device(f"partials[{i}]", p)
        if p.shape != parts[0].shape or p.dtype != parts[0].dtype:
            raise ValueError("partials must share shape and dtype")
    if out is None:
        out = torch.empty_like(parts[0])
    _need_device("out", out)
    if out.dtype != parts[0].dtype or out.numel() != parts[0].numel():
        raise ValueError("out must match the partials' dtype and size")
    _same_device(out, *parts)
    arr = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    _check("vpe_sum_partials", load_library().vpe_sum_partials(
        arr, len(parts), parts[0].numel(), _dtype_code(parts[0]), out.data_ptr(),
        _stream_handle(out.device)))
    return out


def vpe_last_token_select(hidden, cu_seqlens, out=None):
    """hidden [T, D], cu_seqlens int32 [S+1] -> out [S, D] = hidden[cu[1:] - 1]."""
    torch = _torch()
    _need_device("hidden", hidden)
    _need_device("cu_seqlens", cu_seqlens)
    if hidden.dim() != 2:
        raise ValueError("hidden must be [n_tokens, dim]")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor with at least one entry")
    t, d = hidden.shape
    s = cu_seqlens.numel() - 1
    if out is None:
        out = torch.empty((s, d), dtype=hidden.dtype, device=hidden.device)
    _need_device("out", out)
    if out.dtype != hidden.dtype or out.numel() != s * d:
        raise ValueError("out must be [n_seqs, dim] of hidden's dtype")
    _same_device(hidden, cu_seqlens, out)
    _check("vpe_last_token_select", load_library().vpe_last_token_select(
        hidden.data_ptr(), t, d, _dtype_code(hidden), cu_seqlens.data_ptr(), s,
        out.data_ptr(), _stream_handle(hidden.device)))
    return out


def vpe_lmhead(x, weight, logits=None, col_offset: int = 0):
    """Shard logits x [M, D] . weight[R, D]^T into columns [col_offset, +R) of logits [M, ld]."""
    torch = _torch()
    _need_device("x", x)
    _need_device("weight", weight)
    if x.dim() != 2 or weight.dim() != 2 or x.shape[1] != weight.shape[1]:
        raise ValueError("x must be [m, dim] and weight [shard_rows, dim]")
    if x.dtype != weight.dtype:
        raise TypeError("x and weight must share a dtype")
    m, d = x.shape
    rows = weight.shape[0]
    if logits is None:
        logits = torch.empty((m, col_offset + rows), dtype=x.dtype, device=x.device)
    _need_device("logits", logits)
    if logits.dim() != 2 or logits.shape[0] != m or logits.dtype != x.dtype:
        raise ValueError("logits must be [m, ld] of x's dtype")
    _same_device(x, weight, logits)
    _check("vpe_lmhead", load_library().vpe_lmhead(
        x.data_ptr(), m, d, weight.data_ptr(), rows, _dtype_code(x), logits.data_ptr(),
        logits.shape[1], int(col_offset), _stream_handle(x.device)))
    return logits


def vpe_lmhead_prefill(hidden, cu_seqlens, weight, logits=None, col_offset: int = 0):
    """Logits of the last position of every packed sequence, select folded in.

    hidden [T, D], cu_seqlens int32 [S+1], weight [R, D] -> logits [S, ld]
    (columns [col_offset, col_offset + R) written).
    """
    torch = _torch()
    _need_device("hidden", hidden)
    _need_device("cu_seqlens", cu_seqlens)
    _need_device("weight", weight)
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.shape[1] != weight.shape[1]:
        raise ValueError("hidden must be [n_tokens, dim] and weight [shard_rows, dim]")
    if hidden.dtype != weight.dtype:
        raise TypeError("hidden and weight must share a dtype")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor with at least one entry")
    t, d = hidden.shape
    s = cu_seqlens.numel() - 1
    rows = weight.shape[0]
    if logits is None:
        logits = torch.empty((s, col_offset + rows), dtype=hidden.dtype, device=hidden.device)
    _need_device("logits", logits)
    if logits.dim() != 2 or logits.shape[0] != s or logits.dtype != hidden.dtype:
        raise ValueError("logits must be [n_seqs, ld] of hidden's dtype")
    _same_device(hidden, cu_seqlens, weight, logits)
    _check("vpe_lmhead_prefill", load_library().vpe_lmhead_prefill(
        hidden.data_ptr(), t, d, cu_seqlens.data_ptr(), s, weight.data_ptr(), rows,
        _dtype_code(hidden), logits.data_ptr(), logits.shape[1], int(col_offset),
        _stream_handle(hidden.device)))
    return logits


def vpe_load_shard(full, tp_size: int, tp_rank: int, out=None):
    """Rows [rank*R, rank*R + R) of the device table `full` [V, D] into `out` [R, D]."""
    torch = _torch()
    _need_device("full", full)
    if full.dim() != 2 or not full.is_contiguous():
        raise ValueError("full must be a contiguous [V, D] tensor")
    vocab, dim = full.shape
    if tp_size < 1 or vocab % tp_size != 0:
        raise ValueError(f"vocab {vocab} does not split evenly over tp_size {tp_size}")
    rows = vocab // tp_size
    if out is None:
        out = torch.empty((rows, dim), dtype=full.dtype, device=full.device)
    else:
        _need_device("out", out)
        if tuple(out.shape) != (rows, dim) or out.dtype != full.dtype or not out.is_contiguous():
            raise ValueError("out must be a contiguous [V/tp, D] tensor of the table's dtype")
        _same_device(full, out)
    _check("vpe_load_shard", load_library().vpe_load_shard(
        full.data_ptr(), vocab, dim, _dtype_code(full), tp_size, tp_rank, out.data_ptr(),
        _stream_handle(full.device)))
    return out


def vpe_argmax_init(best):
    """Reset the [m] uint64 (int64 tensor) greedy-pick keys to 0."""
    torch = _torch()
    _need_device("best", best)
    if best.dtype != torch.int64 or best.dim() != 1:
        raise ValueError("best must be a 1-D int64 tensor (uint64 keys)")
    _check("vpe_argmax_init", load_library().vpe_argmax_init(
        best.data_ptr(), best.numel(), _stream_handle(best.device)))
    return best


def vpe_lmhead_argmax(x, weight, vocab_start: int, best):
    """Fold this shard's greedy pick (largest logit, id = vocab_start + row) into best."""
    torch = _torch()
    _need_device("x", x)
    _need_device("weight", weight)
    _need_device("best", best)
    if x.dim() != 2 or weight.dim() != 2 or x.shape[1] != weight.shape[1]:
        raise ValueError("x must be [m, dim] and weight [shard_rows, dim]")
    if x.dtype != weight.dtype:
        raise TypeError("x and weight must share a dtype")
    if best.dtype != torch.int64 or best.numel() != x.shape[0]:
        raise ValueError("best must be an int64 tensor with one key per row of x")
    _same_device(x, weight, best)
    _check("vpe_lmhead_argmax", load_library().vpe_lmhead_argmax(
        x.data_ptr(), x.shape[0], x.shape[1], weight.data_ptr(), weight.shape[0],
        _dtype_code(x), int(vocab_start), best.data_ptr(), _stream_handle(x.device)))
    return best


def vpe_lmhead_prefill_argmax(hidden, cu_seqlens, weight, vocab_start: int, best):
    """Fold this shard's greedy pick for the last position of every packed sequence
    (hidden [T, D], cu_seqlens int32 [S+1]) into best [S], the select folded in."""
    torch = _torch()
    _need_device("hidden", hidden)
    _need_device("cu_seqlens", cu_seqlens)
    _need_device("weight", weight)
    _need_device("best", best)
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.shape[1] != weight.shape[1]:
        raise ValueError("hidden must be [n_tokens, dim] and weight [shard_rows, dim]")
    if hidden.dtype != weight.dtype:
        raise TypeError("hidden and weight must share a dtype")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor with at least one entry")
    s = cu_seqlens.numel() - 1
    if best.dtype != torch.int64 or best.dim() != 1 or best.numel() != s:
        raise ValueError("best must be an int64 tensor with one key per sequence")
    _same_device(hidden, cu_seqlens, weight, best)
    _check("vpe_lmhead_prefill_argmax", load_library().vpe_lmhead_prefill_argmax(
        hidden.data_ptr(), hidden.shape[0], hidden.shape[1], cu_seqlens.data_ptr(), s,
        weight.data_ptr(), weight.shape[0], _dtype_code(hidden), int(vocab_start),
        best.data_ptr(), _stream_handle(hidden.device)))
    return best


def _decode(name, best):
    torch = _torch()
    _need_device("best", best)
    if best.dtype != torch.int64 or best.dim() != 1:
        raise ValueError("best must be a 1-D int64 tensor (uint64 keys)")
    value = torch.empty(best.shape, dtype=torch.float32, device=best.device)
    token = torch.empty(best.shape, dtype=torch.int64, device=best.device)
    _check(name, getattr(load_library(), name)(
        best.data_ptr(), best.numel(), value.data_ptr(), token.data_ptr(),
        _stream_handle(best.device)))
    return value, token


def vpe_argmax_decode(best):
    """(max logit float32 [m], token id int64 [m]) from the keys."""
    return _decode("vpe_argmax_decode", best)


def vpe_argmax_decode_clear(best):
    """vpe_argmax_decode, then every key of best is 0 again (ready for the next folds)."""
    return _decode("vpe_argmax_decode_clear", best)


def vpe_lmhead_logsumexp_workspace(m: int, shard_rows: int) -> int:
    """Bytes of workspace vpe_lmhead_logsumexp needs at most for m rows of a shard."""
    n = ctypes.c_int64()
    _check("vpe_lmhead_logsumexp_workspace",
           load_library().vpe_lmhead_logsumexp_workspace(m, shard_rows, ctypes.byref(n)))
    return n.value


def vpe_lmhead_logsumexp(x, weight, logits=None, col_offset: int = 0, shard_lse=None,
                         workspace=None, store_logits: bool = True):
    """One shard's logits (as vpe_lmhead, unless store_logits is False) and every
    row's log-sum-exp over the shard's columns, shard_lse float32 [M].

    Returns (logits or None, shard_lse).  `workspace` is a device tensor of at
    least vpe_lmhead_logsumexp_workspace(M, R) bytes (allocated when None).
    """
    torch = _torch()
    _need_device("x", x)
    _need_device("weight", weight)
    if x.dim() != 2 or weight.dim() != 2 or x.shape[1] != weight.shape[1]:
        raise ValueError("x must be [m, dim] and weight [shard_rows, dim]")
    if x.dtype != weight.dtype:
        raise TypeError("x and weight must share a dtype")
    m, d = x.shape
    rows = weight.shape[0]
    if store_logits:
        if logits is None:
            logits = torch.empty((m, col_offset + rows), dtype=x.dtype, device=x.device)
        _need_device("logits", logits)
        if logits.dim() != 2 or logits.shape[0] != m or logits.dtype != x.dtype:
            raise ValueError("logits must be [m, ld] of x's dtype")
        _same_device(x, logits)
    elif logits is not None:
        raise ValueError("logits given with store_logits=False")
    if shard_lse is None:
        shard_lse = torch.empty(m, dtype=torch.float32, device=x.device)
    _need_device("shard_lse", shard_lse)
    if shard_lse.dtype != torch.float32 or shard_lse.numel() != m:
        raise ValueError("shard_lse must be a float32 tensor with one value per row of x")
    need = vpe_lmhead_logsumexp_workspace(m, rows)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=x.device)
    _need_device("workspace", workspace)
    _same_device(x, weight, shard_lse, workspace)
    nbytes = workspace.numel() * workspace.element_size()
    _check("vpe_lmhead_logsumexp", load_library().vpe_lmhead_logsumexp(
        x.data_ptr(), m, d, weight.data_ptr(), rows, _dtype_code(x),
        logits.data_ptr() if logits is not None else None,
        logits.shape[1] if logits is not None else rows, int(col_offset), shard_lse.data_ptr(),
        workspace.data_ptr(), nbytes, _stream_handle(x.device)))
    return logits, shard_lse


def vpe_lmhead_prefill_logsumexp(hidden, cu_seqlens, weight, logits=None, col_offset: int = 0,
                                 shard_lse=None, workspace=None, store_logits: bool = True):
    """vpe_lmhead_logsumexp over the last position of every packed sequence
    (hidden [T, D], cu_seqlens int32 [S+1]): the logits of those rows, unless
    store_logits is False, and each row's log-sum-exp over the shard's columns,
    shard_lse float32 [S].  Returns (logits or None, shard_lse)."""
    torch = _torch()
    _need_device("hidden", hidden)
    _need_device("cu_seqlens", cu_seqlens)
    _need_device("weight", weight)
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.shape[1] != weight.shape[1]:
        raise ValueError("hidden must be [n_tokens, dim] and weight [shard_rows, dim]")
    if hidden.dtype != weight.dtype:
        raise TypeError("hidden and weight must share a dtype")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor with at least one entry")
    t, d = hidden.shape
    s = cu_seqlens.numel() - 1
    rows = weight.shape[0]
    if store_logits:
        if logits is None:
            logits = torch.empty((s, col_offset + rows), dtype=hidden.dtype, device=hidden.device)
        _need_device("logits", logits)
        if logits.dim() != 2 or logits.shape[0] != s or logits.dtype != hidden.dtype:
            raise ValueError("logits must be [n_seqs, ld] of hidden's dtype")
        _same_device(hidden, logits)
    elif logits is not None:
        raise ValueError("logits given with store_logits=False")
    if shard_lse is None:
        shard_lse = torch.empty(s, dtype=torch.float32, device=hidden.device)
    _need_device("shard_lse", shard_lse)
    if shard_lse.dtype != torch.float32 or shard_lse.numel() != s:
        raise ValueError("shard_lse must be a float32 tensor with one value per sequence")
    need = vpe_lmhead_logsumexp_workspace(s, rows)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=hidden.device)
    _need_device("workspace", workspace)
    _same_device(hidden, cu_seqlens, weight, shard_lse, workspace)
    nbytes = workspace.numel() * workspace.element_size()
    _check("vpe_lmhead_prefill_logsumexp", load_library().vpe_lmhead_prefill_logsumexp(
        hidden.data_ptr(), t, d, cu_seqlens.data_ptr(), s, weight.data_ptr(), rows,
        _dtype_code(hidden), logits.data_ptr() if logits is not None else None,
        logits.shape[1] if logits is not None else rows, int(col_offset), shard_lse.data_ptr(),
        workspace.data_ptr(), nbytes, _stream_handle(hidden.device)))
    return logits, shard_lse


def vpe_lmhead_logsumexp_noalloc(x, weight, shard_lse, logits=None, col_offset: int = 0):
    """vpe_lmhead_logsumexp without a workspace: the library's static per-GPU
    array holds the tile pairs, so the call allocates nothing (outputs are the
    caller's: shard_lse float32 [M], and logits [M, ld] or None to store none).
    Calls that may overlap on one GPU race on that array."""
    torch = _torch()
    _need_device("x", x)
    _need_device("weight", weight)
    _need_device("shard_lse", shard_lse)
    if x.dim() != 2 or weight.dim() != 2 or x.shape[1] != weight.shape[1]:
        raise ValueError("x must be [m, dim] and weight [shard_rows, dim]")
    if x.dtype != weight.dtype:
        raise TypeError("x and weight must share a dtype")
    if shard_lse.dtype != torch.float32 or shard_lse.numel() != x.shape[0]:
        raise ValueError("shard_lse must be a float32 tensor with one value per row of x")
    if logits is not None:
        _need_device("logits", logits)
        if logits.dim() != 2 or logits.shape[0] != x.shape[0] or logits.dtype != x.dtype:
            raise ValueError("logits must be [m, ld] of x's dtype")
        _same_device(x, logits)
    _same_device(x, weight, shard_lse)
    _check("vpe_lmhead_logsumexp_noalloc", load_library().vpe_lmhead_logsumexp_noalloc(
        x.data_ptr(), x.shape[0], x.shape[1], weight.data_ptr(), weight.shape[0], _dtype_code(x),
        logits.data_ptr() if logits is not None else None,
        logits.shape[1] if logits is not None else weight.shape[0], int(col_offset),
        shard_lse.data_ptr(), _stream_handle(x.device)))
    return logits, shard_lse


def vpe_logsumexp_combine(shard_lse: Sequence, out=None):
    """log(sum_r exp(shard_lse[r])) per row: the ranks' values combined, in rank order."""
    torch = _torch()
    parts = list(shard_lse)
    if not parts:
        raise ValueError("need at least one shard's values")
    for i, p in enumerate(parts):
        _need_device(f"shard_lse[{i}]", p)
        if p.dtype != torch.float32 or p.shape != parts[0].shape:
            raise ValueError("shard values must be float32 tensors of one shape")
    if out is None:
        out = torch.empty_like(parts[0])
    _need_device("out", out)
    if out.dtype != torch.float32 or out.numel() != parts[0].numel():
        raise ValueError("out must be float32 with one value per row")
    _same_device(out, *parts)
    arr = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    _check("vpe_logsumexp_combine", load_library().vpe_logsumexp_combine(
        arr, len(parts), parts[0].numel(), out.data_ptr(), _stream_handle(out.device)))
    return out


from .layers import ParallelLMHead, VocabParallelEmbedding  # noqa: E402

__all__ = [
    "vpe_shard_range", "vpe_embed", "vpe_sum_partials", "vpe_last_token_select", "vpe_lmhead",
    "vpe_lmhead_prefill", "vpe_argmax_init", "vpe_lmhead_argmax", "vpe_lmhead_prefill_argmax",
    "vpe_argmax_decode", "vpe_argmax_decode_clear", "vpe_load_shard",
    "vpe_lmhead_logsumexp_workspace", "vpe_lmhead_logsumexp", "vpe_lmhead_prefill_logsumexp",
    "vpe_logsumexp_combine",
    "vpe_lmhead_logsumexp_noalloc", "VocabParallelEmbedding", "ParallelLMHead", "VpeError", "StaleLibraryError", "load_library",
    "check_library_current", "LIB_PATH",
]
