"""CPU oracle for the vocab-parallel embedding and LM-head path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It wraps the
plain C loops in ``oracle.c`` (built with gcc into ``liboracle.so``) and shares
no code with the HIP library: it does not import the product package, and the
product package does not import it.

Functions take and return numpy arrays.  bf16 data travels as uint16 bit
patterns (numpy has no bf16 type); fp32 data as float32.  Which passage of the
pages each function follows is stated in ``oracle.c`` next to its definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
I32, I64 = 0, 1

OK, ERR_ARG, ERR_SHARD, ERR_CUSEQ = 0, 1, 2, 3


class OracleError(RuntimeError):
    pass


_CMD = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
        "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra"]


def _digest() -> str:
    """sha256 of oracle.c and the compile command."""
    import hashlib
    with open(_SRC, "rb") as f:
        return hashlib.sha256(f.read() + " ".join(_CMD).encode()).hexdigest()


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no fast-math).
    Also rebuilds when the library was built from another oracle.c (the digest
    recorded next to it differs)."""
    digest = _digest()
    try:
        with open(_LIB + ".sha256") as f:
            current = f.read().strip() == digest and os.path.exists(_LIB)
    except OSError:
        current = False
    if force or not current:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(_CMD + [_SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB)
        with open(_LIB + ".sha256.tmp%d" % os.getpid(), "w") as f:
            f.write(digest + "\n")
        os.replace(_LIB + ".sha256.tmp%d" % os.getpid(), _LIB + ".sha256")
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        ci = ctypes.c_int
        lib.orc_shard_range.argtypes = [i64, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.orc_mask_shift.argtypes = [vp, ci, i64, i64, i64, vp, vp]
        lib.orc_embed.argtypes = [vp, ci, i64, vp, ci, i64, i64, i64, vp, ci]
        lib.orc_sum_partials.argtypes = [ctypes.POINTER(vp), i32, i64, ci, vp]
        lib.orc_last_token_select.argtypes = [vp, i64, i64, ci, vp, i64, vp]
        lib.orc_lmhead_f64.argtypes = [vp, i64, i64, vp, i64, ci, vp, i64, i64, ci]
        lib.orc_logit_f64.argtypes = [vp, i64, vp, ci, i64, i64]
        lib.orc_argmax_rows.argtypes = [vp, i64, i64, i64, vp, vp]
        lib.orc_logsumexp_rows.argtypes = [vp, i64, i64, i64, vp]
        lib.orc_logsumexp_rows.restype = ci
        lib.orc_load_shard.argtypes = [vp, i64, i64, ci, i32, i32, vp]
        lib.orc_load_shard.restype = ci
        lib.orc_argmax_rows.restype = ci
        lib.orc_logit_f64.restype = ctypes.c_double
        lib.orc_round_bf16.argtypes = [ctypes.c_float]
        lib.orc_round_bf16.restype = ctypes.c_uint16
        lib.orc_widen_bf16.argtypes = [ctypes.c_uint16]
        lib.orc_widen_bf16.restype = ctypes.c_float
        for name in ("orc_shard_range", "orc_mask_shift", "orc_embed", "orc_sum_partials",
                     "orc_last_token_select", "orc_lmhead_f64"):
            getattr(lib, name).restype = ci
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle data must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _itype_code(a: np.ndarray) -> int:
    if a.dtype == np.int32:
        return I32
    if a.dtype == np.int64:
        return I64
    raise TypeError(f"token ids must be int32 or int64, got {a.dtype}")


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise OracleError(f"{what} failed with code {rc}")


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


# ---------------------------------------------------------------------------
def shard_range(vocab: int, tp_size: int, tp_rank: int) -> Tuple[int, int]:
    lib = _load()
    s, e = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.orc_shard_range(vocab, tp_size, tp_rank, ctypes.byref(s), ctypes.byref(e)),
           "shard_range")
    return s.value, e.value


def load_shard(full: np.ndarray, tp_size: int, tp_rank: int) -> np.ndarray:
    """Rows [rank*R, rank*R + R) of the full [V, D] table, bits unchanged."""
    full = np.ascontiguousarray(full)
    if full.ndim != 2:
        raise ValueError("full table must be [V, D]")
    vocab, dim = full.shape
    rows = vocab // tp_size if tp_size > 0 else 0
    out = np.empty((rows, dim), dtype=full.dtype)
    _check(_load().orc_load_shard(_ptr(full), vocab, dim, _dtype_code(full), tp_size, tp_rank,
                                  _ptr(out)), "load_shard")
    return out


def mask_shift(ids: np.ndarray, vocab_start: int, vocab_end: int):
    """Steps 1-2: (mask[bool], local index[int64]) for flat ids."""
    ids = np.ascontiguousarray(ids).reshape(-1)
    n = ids.size
    mask = np.empty(n, dtype=np.uint8)
    local = np.empty(n, dtype=np.int64)
    _check(_load().orc_mask_shift(_ptr(ids), _itype_code(ids), n, vocab_start, vocab_end,
                                  _ptr(mask), _ptr(local)), "mask_shift")
    return mask.astype(bool), local


def embed(ids: np.ndarray, weight: np.ndarray, vocab_start: int,
          nthreads: int = 1) -> np.ndarray:
    """One shard's masked lookup: [n] ids x [R, D] shard -> [n, D]."""
    ids = np.ascontiguousarray(ids).reshape(-1)
    weight = np.ascontiguousarray(weight)
    if weight.ndim != 2:
        raise ValueError("weight must be [rows, dim]")
    rows, dim = weight.shape
    out = np.empty((ids.size, dim), dtype=weight.dtype)
    _check(_load().orc_embed(_ptr(ids), _itype_code(ids), ids.size, _ptr(weight),
                             _dtype_code(weight), rows, dim, vocab_start, _ptr(out),
                             nthreads), "embed")
    return out


def sum_partials(parts: Sequence[np.ndarray]) -> np.ndarray:
    """Elementwise sum of same-shape partials, rank order, fp32, one rounding."""
    parts = [np.ascontiguousarray(p) for p in parts]
    if not parts:
        raise ValueError("need at least one partial")
    shape, dt = parts[0].shape, parts[0].dtype
    for p in parts:
        if p.shape != shape or p.dtype != dt:
            raise ValueError("partials must share shape and dtype")
    out = np.empty(shape, dtype=dt)
    arr = (ctypes.c_void_p * len(parts))(*[_ptr(p) for p in parts])
    _check(_load().orc_sum_partials(arr, len(parts), out.size, _dtype_code(parts[0]),
                                    _ptr(out)), "sum_partials")
    return out


def last_token_select(hidden: np.ndarray, cu_seqlens: np.ndarray) -> np.ndarray:
    """Rows hidden[cu[s+1]-1] for every sequence s."""
    hidden = np.ascontiguousarray(hidden)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    t, d = hidden.shape
    s = cu.size - 1
    if s < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    out = np.empty((s, d), dtype=hidden.dtype)
    _check(_load().orc_last_token_select(_ptr(hidden), t, d, _dtype_code(hidden), _ptr(cu),
                                         s, _ptr(out)), "last_token_select")
    return out


def lmhead_f64(x: np.ndarray, weight: np.ndarray, out: Optional[np.ndarray] = None,
               col_offset: int = 0, nthreads: int = 1) -> np.ndarray:
    """Shard logits x . weight^T in fp64, written at columns [col_offset, +R) of out."""
    x = np.ascontiguousarray(x)
    weight = np.ascontiguousarray(weight)
    m, d = x.shape
    r, d2 = weight.shape
    if d != d2 or x.dtype != weight.dtype:
        raise ValueError("x and weight must share dim and dtype")
    if out is None:
        out = np.zeros((m, r + col_offset), dtype=np.float64)
    if out.dtype != np.float64 or not out.flags.c_contiguous or out.shape[0] != m:
        raise ValueError("out must be a C-contiguous float64 [m, ld] array")
    _check(_load().orc_lmhead_f64(_ptr(x), m, d, _ptr(weight), r, _dtype_code(x), _ptr(out),
                                  out.shape[1], col_offset, nthreads), "lmhead_f64")
    return out


def logit_f64(x: np.ndarray, weight: np.ndarray, m: int, j: int) -> float:
    """One logit x[m] . weight[j] in fp64 (for sampled checks of large products)."""
    x = np.ascontiguousarray(x)
    weight = np.ascontiguousarray(weight)
    return _load().orc_logit_f64(_ptr(x), x.shape[1], _ptr(weight), _dtype_code(x), m, j)


def argmax_rows(logits: np.ndarray):
    """(max value, first column holding it) of every row of an fp64 [m, n] array."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    m, n = logits.shape
    mx = np.empty(m, dtype=np.float64)
    idx = np.empty(m, dtype=np.int64)
    _check(_load().orc_argmax_rows(_ptr(logits), m, n, n, _ptr(mx), _ptr(idx)), "argmax_rows")
    return mx, idx


def logsumexp_rows(logits: np.ndarray) -> np.ndarray:
    """log(sum_j exp(logits[m, j])) of every row of an fp64 [m, n] array (the
    softmax normaliser of each row), in fp64."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    m, n = logits.shape
    out = np.empty(m, dtype=np.float64)
    _check(_load().orc_logsumexp_rows(_ptr(logits), m, n, n, _ptr(out)), "logsumexp_rows")
    return out


def round_bf16(values) -> np.ndarray:
    """fp32 -> bf16 bits, the oracle's own rounding (used by the sum of bf16 partials)."""
    lib = _load()
    v = np.asarray(values, dtype=np.float32).reshape(-1)
    return np.array([lib.orc_round_bf16(float(f)) for f in v], dtype=np.uint16)


def widen_bf16(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([lib.orc_widen_bf16(int(h)) for h in b], dtype=np.float32)
