"""Seeded synthetic inputs for the vocab-parallel embedding / LM-head path.

This module only draws numbers. It holds none of the method's arithmetic (no
masking, no lookup, no products, no sums): the kernels and the CPU oracle both
receive the same host bytes from here and compute on them independently.

Workloads are stand-ins for a Qwen3-0.6B checkpoint and a real token stream
(neither is available): tables are N(0, 0.02), hidden states N(0, 1), token
ids uniform over the vocabulary or Zipf(s=1.1) over token rank.  Shapes follow
the pages' Qwen3-0.6B figures (vocab 151936, hidden 1024, tp=2 shard of 75968
rows) plus a tiny fp32 case and a hidden-4096 tp=4 case.

Every generator is counter-seeded: a table row block ``b`` is drawn from
``numpy.random.default_rng([seed, b])`` so that any slice of a table can be
produced without drawing the rows before it.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

TABLE_BLOCK_ROWS = 1024


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration of the hot path.

    vocab, dim   full vocabulary size V and hidden size D
    dtype        "f32" or "bf16" (table, hidden states and logits)
    tp           tensor-parallel size; ranks own contiguous V/tp rows
    ranks        which ranks are run (each rank = one shard's embed + LM head)
    n_ids        number of token ids looked up
    id_dist      "uniform" over [0, V) or "zipf" (s = zipf_s over rank, id = rank-1)
    lm_rows      rows of hidden states fed to the LM head (M)
    seqs         number of packed sequences for prefill (0 = decode: no select)
    seq_len      tokens per sequence for prefill (n_ids == seqs * seq_len)
    concat       True: shard logits written into one [M, V] buffer at column
                 offset vocab_start; False: into a [M, V/tp] shard buffer
    seed         base seed; table = 100c+1, ids = 100c+2, hidden = 100c+3
    """

    name: str
    vocab: int
    dim: int
    dtype: str
    tp: int
    ranks: Tuple[int, ...]
    n_ids: int
    id_dist: str
    lm_rows: int
    seqs: int
    seq_len: int
    concat: bool
    seed: int
    zipf_s: float = 1.1
    note: str = ""

    @property
    def shard_rows(self) -> int:
        return self.vocab // self.tp

    def rank_start(self, rank: int) -> int:
        return rank * self.shard_rows

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            name="tiny_v4096_d64_f32_tp2",
            vocab=4096, dim=64, dtype="f32", tp=2, ranks=(0, 1), n_ids=256,
            id_dist="uniform", lm_rows=16, seqs=0, seq_len=0, concat=True,
            seed=100,
            note="tiny tp=2 emulated on one device, fp32, logits [16,4096] by shard concat",
        ),
        Workload(
            name="qwen3_0p6b_tp2_rank0",
            vocab=151936, dim=1024, dtype="bf16", tp=2, ranks=(0,), n_ids=8192,
            id_dist="uniform", lm_rows=256, seqs=0, seq_len=0, concat=False,
            seed=200,
            note="Qwen3-0.6B tp=2 rank-0 shard (rows [0,75968)); decode LM head M=256",
        ),
        Workload(
            name="qwen3_0p6b_tp1_prefill",
            vocab=151936, dim=1024, dtype="bf16", tp=1, ranks=(0,), n_ids=65536,
            id_dist="zipf", lm_rows=32, seqs=32, seq_len=2048, concat=True,
            seed=300,
            note="Qwen3-0.6B tp=1 prefill 32x2048 Zipf ids; last-token select; LM head M=32",
        ),
        Workload(
            name="qwen3_0p6b_tp2_all_ranks",
            vocab=151936, dim=1024, dtype="bf16", tp=2, ranks=(0, 1), n_ids=16384,
            id_dist="uniform", lm_rows=1024, seqs=0, seq_len=0, concat=True,
            seed=400,
            note="both tp=2 ranks on one GPU; partial sum == full lookup; logits [1024,151936]",
        ),
        Workload(
            name="large_v151936_d4096_tp4_rank2",
            vocab=151936, dim=4096, dtype="bf16", tp=4, ranks=(2,), n_ids=131072,
            id_dist="uniform", lm_rows=4096, seqs=0, seq_len=0, concat=False,
            seed=500,
            note="hidden 4096, tp=4 rank-2 shard rows [75968,113952); LM head [4096,37984]",
        ),
    ]
}

WORKLOAD_ORDER: List[str] = list(WORKLOADS.keys())


# --------------------------------------------------------------------------
# bf16 encoding of generated fp32 samples (input preparation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 samples to bf16 bit patterns (round to nearest, ties to even).

    Inputs here are finite normal samples; NaN handling is not needed and is
    rejected so that nothing silently changes meaning.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("generator produced a non-finite sample")
    u = a.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------
def table_rows(seed: int, vocab: int, dim: int, dtype: str, lo: int, hi: int,
               std: float = 0.02) -> np.ndarray:
    """Rows [lo, hi) of a vocab x dim N(0, std) table, drawn block by block.

    Returns float32 [hi-lo, dim] for "f32", uint16 bf16 bits for "bf16".
    The result does not depend on which slice is requested.

    A float32 normal draw is exactly +-0 with probability about 2**-23, so a
    Qwen3-sized table holds a few dozen zeros.  Their sign is cleared: tables
    hold no -0.0, the condition under which the sum of masked partials equals
    the full lookup bit for bit ((+0) + (-0) is +0).
    """
    if not (0 <= lo <= hi <= vocab):
        raise ValueError(f"bad row range [{lo},{hi}) for vocab {vocab}")
    out = np.empty((hi - lo, dim), dtype=np.float32 if dtype == "f32" else np.uint16)
    b0 = lo // TABLE_BLOCK_ROWS
    b1 = (hi + TABLE_BLOCK_ROWS - 1) // TABLE_BLOCK_ROWS
    for b in range(b0, b1):
        r0 = b * TABLE_BLOCK_ROWS
        r1 = min(r0 + TABLE_BLOCK_ROWS, vocab)
        rng = np.random.default_rng([seed, b])
        blk = rng.standard_normal((r1 - r0, dim), dtype=np.float32) * np.float32(std)
        s0, s1 = max(lo, r0), min(hi, r1)
        out[s0 - lo:s1 - lo] = _encode(blk[s0 - r0:s1 - r0], dtype)
    if dtype == "bf16":
        out[out == 0x8000] = 0
    else:
        out[out == 0] = 0.0  # -0.0 == 0 compares true: every zero becomes +0.0
    return out


def token_ids(seed: int, vocab: int, n: int, dist: str = "uniform",
              zipf_s: float = 1.1, dtype=np.int32) -> np.ndarray:
    """n token ids in [0, vocab): uniform, or Zipf(s) over rank with id = rank - 1.

    The Zipf law is taken on the finite support 1..vocab by inverse CDF, so the
    most frequent id is 0 and frequencies fall as rank**-s.
    """
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        ids = rng.integers(0, vocab, size=n, dtype=np.int64)
    elif dist == "zipf":
        ranks = np.arange(1, vocab + 1, dtype=np.float64)
        w = ranks ** (-zipf_s)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        u = rng.random(n)
        ids = np.searchsorted(cdf, u, side="right").astype(np.int64)
        np.minimum(ids, vocab - 1, out=ids)
    else:
        raise ValueError(f"unknown id distribution {dist!r}")
    return ids.astype(dtype)


def hidden_states(seed: int, rows: int, dim: int, dtype: str) -> np.ndarray:
    """rows x dim N(0, 1) hidden states (f32, or bf16 bits)."""
    rng = np.random.default_rng(seed)
    return _encode(rng.standard_normal((rows, dim), dtype=np.float32), dtype)


def cu_seqlens_uniform(seqs: int, seq_len: int) -> np.ndarray:
    """Cumulative sequence starts [0, L, 2L, ..., seqs*L] as int32."""
    return (np.arange(seqs + 1, dtype=np.int64) * seq_len).astype(np.int32)


def cu_seqlens_ragged(seed: int, seqs: int, min_len: int, max_len: int) -> np.ndarray:
    """Cumulative starts of `seqs` sequences with lengths uniform in [min_len, max_len]."""
    if min_len < 1:
        raise ValueError("sequence lengths must be >= 1")
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len + 1, size=seqs, dtype=np.int64)
    cu = np.zeros(seqs + 1, dtype=np.int64)
    np.cumsum(lens, out=cu[1:])
    return cu.astype(np.int32)


# --------------------------------------------------------------------------
# whole-workload inputs
# --------------------------------------------------------------------------
def table_seed(w: Workload) -> int:
    return w.seed + 1


def ids_seed(w: Workload) -> int:
    return w.seed + 2


def hidden_seed(w: Workload) -> int:
    return w.seed + 3


def shard_table(w: Workload, rank: int) -> np.ndarray:
    """The rank's shard: rows [rank*V/tp, (rank+1)*V/tp) of the full table."""
    lo = w.rank_start(rank)
    return table_rows(table_seed(w), w.vocab, w.dim, w.dtype, lo, lo + w.shard_rows)


def full_table(w: Workload) -> np.ndarray:
    return table_rows(table_seed(w), w.vocab, w.dim, w.dtype, 0, w.vocab)


def workload_ids(w: Workload, dtype=np.int32) -> np.ndarray:
    return token_ids(ids_seed(w), w.vocab, w.n_ids, w.id_dist, w.zipf_s, dtype=dtype)


def workload_hidden(w: Workload) -> np.ndarray:
    """Hidden states fed to the LM head path.

    Prefill workloads return the whole packed [seqs*seq_len, D] activation (the
    select step picks the last row of every sequence); decode workloads return
    [lm_rows, D] directly.
    """
    rows = w.seqs * w.seq_len if w.seqs else w.lm_rows
    return hidden_states(hidden_seed(w), rows, w.dim, w.dtype)


def workload_cu_seqlens(w: Workload) -> Optional[np.ndarray]:
    if not w.seqs:
        return None
    return cu_seqlens_uniform(w.seqs, w.seq_len)
