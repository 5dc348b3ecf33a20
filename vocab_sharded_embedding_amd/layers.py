"""Page-shaped layer objects over the C ABI (argument marshalling only).

``VocabParallelEmbedding`` and ``ParallelLMHead`` keep the constructor and
``weight_loader`` of the nano-vllm layers the pages walk through
(devpress.csdn.net/amd/6a3de260... sections 3-4; blog.xiaohansong.com
"从零实现 vLLM (1.1)" source analysis; AIInfraGuide 3.3 section 6): a rank
holds rows [vocab_start, vocab_end) of the [V, D] table as a [V/tp, D]
parameter.  Their ``forward`` calls the library; there is no collective here:
ranks emulated in one process combine their outputs with
``VocabParallelEmbedding.sum_partials`` (the embedding's all-reduce) and by
writing their logits at ``vocab_start`` into one [M, V] buffer (the LM head's
gather and concatenation).
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import (vpe_embed, vpe_lmhead, vpe_lmhead_argmax, vpe_lmhead_logsumexp, vpe_lmhead_prefill,
               vpe_lmhead_prefill_argmax, vpe_lmhead_prefill_logsumexp, vpe_load_shard,
               vpe_logsumexp_combine, vpe_shard_range, vpe_sum_partials)


class VocabParallelEmbedding(torch.nn.Module):
    def __init__(self, num_embeddings: int, embedding_dim: int, tp_size: int = 1,
                 tp_rank: int = 0, dtype: torch.dtype = torch.bfloat16,
                 device: Optional[torch.device] = None):
        super().__init__()
        self.num_embeddings = num_embeddings
        self.embedding_dim = embedding_dim
        self.tp_size = tp_size
        self.tp_rank = tp_rank
        self.vocab_start_idx, self.vocab_end_idx = vpe_shard_range(num_embeddings, tp_size,
                                                                   tp_rank)
        self.num_embeddings_per_partition = self.vocab_end_idx - self.vocab_start_idx
        self.weight = torch.nn.Parameter(
            torch.empty(self.num_embeddings_per_partition, embedding_dim, dtype=dtype,
                        device=device),
            requires_grad=False)
        self.weight.weight_loader = self.weight_loader

    def weight_loader(self, param: torch.nn.Parameter, loaded_weight: torch.Tensor) -> None:
        """Copy this rank's rows of the full [V, D] table into the shard (setup only).

        A full table already on the shard's device is copied by the library's
        own kernel (`vpe_load_shard`); a host table (e.g. read from disk) is
        narrowed and uploaded.
        """
        shard = param.data.size(0)
        full_shape = (self.num_embeddings, self.embedding_dim)
        if (loaded_weight.device == param.data.device and loaded_weight.is_cuda
                and tuple(loaded_weight.shape) == full_shape and loaded_weight.is_contiguous()
                and loaded_weight.dtype == param.data.dtype):
            vpe_load_shard(loaded_weight, self.tp_size, self.tp_rank, out=param.data)
            return
        piece = loaded_weight.narrow(0, self.vocab_start_idx, shard)
        if piece.shape != param.data.shape:
            raise ValueError(f"loaded table slice {tuple(piece.shape)} does not match "
                             f"shard {tuple(param.data.shape)}")
        param.data.copy_(piece)

    def forward(self, ids: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """This rank's partial embedding (zero rows for ids it does not own)."""
        return vpe_embed(ids, self.weight, self.vocab_start_idx, out=out)

    @staticmethod
    def sum_partials(partials: Sequence[torch.Tensor],
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The ranks' partials summed on one device (the all-reduce of the embedding)."""
        return vpe_sum_partials(partials, out=out)


class ParallelLMHead(VocabParallelEmbedding):
    def tie_to(self, embedding: VocabParallelEmbedding) -> "ParallelLMHead":
        """Share the embedding's shard as this head's weight (tied tables,
        AIInfraGuide 3.3 section 8): one [V/tp, D] buffer serves both calls."""
        same = (embedding.num_embeddings, embedding.embedding_dim, embedding.tp_size,
                embedding.tp_rank) == (self.num_embeddings, self.embedding_dim, self.tp_size,
                                       self.tp_rank)
        if not same:
            raise ValueError("a tied head needs the embedding's vocabulary, width and rank")
        self.weight = embedding.weight
        return self

    def forward(self, hidden: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                logits: Optional[torch.Tensor] = None) -> torch.Tensor:
        """This rank's logits.

        With ``cu_seqlens`` (prefill) only the last position of every sequence
        is projected.  ``logits`` may be this rank's [M, V/tp] buffer or the
        full [M, V] buffer, in which case the shard lands at its vocab_start.
        """
        if logits is None:
            col = 0
        elif logits.shape[1] == self.num_embeddings_per_partition:
            col = 0
        elif logits.shape[1] == self.num_embeddings:
            col = self.vocab_start_idx
        else:
            raise ValueError("logits must be [M, V/tp] (one shard) or [M, V] (all shards)")
        if cu_seqlens is not None:
            # the last-position select is folded into the LM-head kernel
            return vpe_lmhead_prefill(hidden, cu_seqlens, self.weight, logits, col_offset=col)
        return vpe_lmhead(hidden, self.weight, logits, col_offset=col)

    def fold_argmax(self, hidden: torch.Tensor, best: torch.Tensor,
                    cu_seqlens: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Fold this rank's greedy pick for every row of ``hidden`` (or, with
        ``cu_seqlens``, for the last position of every packed sequence) into
        ``best`` (keys reset by ``vpe_argmax_init``, or left cleared by
        ``vpe_argmax_decode_clear``; read with either decode)."""
        if cu_seqlens is not None:
            return vpe_lmhead_prefill_argmax(hidden, cu_seqlens, self.weight,
                                             self.vocab_start_idx, best)
        return vpe_lmhead_argmax(hidden, self.weight, self.vocab_start_idx, best)

    def logsumexp(self, hidden: torch.Tensor, logits: Optional[torch.Tensor] = None,
                  store_logits: bool = True, cu_seqlens: Optional[torch.Tensor] = None):
        """This rank's logits (into ``logits`` as ``forward`` places them, unless
        ``store_logits`` is False) and each row's log-sum-exp over this rank's
        vocabulary columns; with ``cu_seqlens`` (prefill) the rows are the last
        positions of the packed sequences.  Returns (logits or None,
        shard_lse).  The ranks' values combine with
        ``ParallelLMHead.combine_logsumexp``."""
        col = 0
        if logits is not None and logits.shape[1] == self.num_embeddings:
            col = self.vocab_start_idx
        elif logits is not None and logits.shape[1] != self.num_embeddings_per_partition:
            raise ValueError("logits must be [M, V/tp] (one shard) or [M, V] (all shards)")
        if cu_seqlens is not None:
            return vpe_lmhead_prefill_logsumexp(hidden, cu_seqlens, self.weight, logits,
                                                col_offset=col, store_logits=store_logits)
        return vpe_lmhead_logsumexp(hidden, self.weight, logits, col_offset=col,
                                    store_logits=store_logits)

    @staticmethod
    def combine_logsumexp(shard_lse: Sequence[torch.Tensor],
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The ranks' per-row values combined into the log-sum-exp of the full
        vocabulary rows (the exchange step, on one device)."""
        return vpe_logsumexp_combine(shard_lse, out=out)
