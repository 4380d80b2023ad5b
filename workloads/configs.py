"""The decode workloads, described by their sizes.

Every workload is one decode step of one attention layer: one new query token
per sequence, grouped-query attention (``num_q_heads`` query heads share each of
``num_kv_heads`` KV heads), a KV cache cut into blocks of ``block_size``
tokens.  The block sizes 64/128, the 90% sparsity and the 4K-token budget are
the operating points named in the SeerAttention-R abstract ("SeerAttention-R:
Sparse Attention Adaptation for Long Reasoning", Abstract).

Selection rules
---------------
``keep=(a, b)``     keep the smallest number of blocks that covers the fraction
                    a/b of the sequence's blocks (90% sparsity is (1, 10)).
``top_k=k``         keep exactly k blocks (clamped to the block count); a token
                    budget B is top_k = B // block_size.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "f32" or "bf16"
    context: int                    # context length (tokens, incl. the new one)
    keep: Optional[Tuple[int, int]] = None
    top_k: Optional[int] = None
    variable_context: Optional[Tuple[int, int]] = None   # inclusive range of lengths
    paged: bool = False
    planted_fraction: Optional[Tuple[int, int]] = None    # share of blocks planted
    heavy_tailed_keys: bool = False                       # Student-t(3) keys
    decode_steps: int = 0                                 # >0: an incremental decode loop
    query_tokens: int = 1                                 # new query tokens per sequence
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_context(self) -> int:
        if self.variable_context is not None:
            return self.variable_context[1]
        return self.context + self.decode_steps

    @property
    def max_blocks(self) -> int:
        return -(-self.max_context // self.block_size)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 1 sequence, 4 query heads on 1 KV head, d=64, 1024 tokens in 16 blocks of
    # 64, keep the top 4 blocks (75% sparsity), fp32.
    "tiny_1k": Workload("tiny_1k", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                        block_size=64, dtype="f32", context=1024, top_k=4, seed=29001),
    # 8 sequences, 32/8 heads, d=128, 8192 tokens in 128 blocks of 64, 90%
    # sparsity (13 blocks), bf16, 5% of blocks planted along the query.
    "planted_8k": Workload("planted_8k", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=64, dtype="bf16", context=8192, keep=(1, 10),
                           planted_fraction=(1, 20), seed=29002),
    # 16 sequences, 32/8 heads, d=128, 32768 tokens in 256 blocks of 128, a
    # 4096-token budget (32 blocks), bf16.
    "budget_32k": Workload("budget_32k", batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=128, dtype="bf16", context=32768, top_k=4096 // 128,
                           seed=29003),
    # The same shape at 90% sparsity (26 of 256 blocks).
    "sparse90_32k": Workload("sparse90_32k", batch=16, num_q_heads=32, num_kv_heads=8,
                             head_dim=128, block_size=128, dtype="bf16", context=32768,
                             keep=(1, 10), seed=29003),
    # 64 sequences of 2048..16384 tokens, 40/8 heads (5:1), d=128, 64-token
    # pages behind a shuffled int32 page table, 90% sparsity per sequence.
    "paged_var": Workload("paged_var", batch=64, num_q_heads=40, num_kv_heads=8, head_dim=128,
                          block_size=64, dtype="bf16", context=16384,
                          variable_context=(2048, 16384), paged=True, keep=(1, 10),
                          seed=29004),
    # 4 sequences, 64/8 heads, d=128, 131072 tokens (1024 blocks of 128),
    # Student-t(3) keys, 95% sparsity, 256 decode steps with incremental pooling.
    "long_131k": Workload("long_131k", batch=4, num_q_heads=64, num_kv_heads=8, head_dim=128,
                          block_size=128, dtype="bf16", context=131072, keep=(1, 20),
                          heavy_tailed_keys=True, decode_steps=256, seed=29005),
    # sparse90_32k with 4 new query tokens per sequence (speculative or chunked
    # decode): 16 query rows per KV head, one selection for the 4 tokens.
    "spec4_32k": Workload("spec4_32k", batch=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
                          block_size=128, dtype="bf16", context=32768, keep=(1, 10),
                          query_tokens=4, seed=29006),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
