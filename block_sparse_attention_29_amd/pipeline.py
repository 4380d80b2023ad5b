"""One gated block-sparse decode step, wired from the libseer calls.

``DecodeState`` owns the device buffers of one attention layer (pooled-key
table, open-block sums, scores, selection, outputs, workspace) and enqueues:

    build_pool(lens)             bulk key pooling after prefill
    append(lens_old, lens_new)   incremental pooling of newly cached tokens
    select(q, lens)              gate scores + top-k block selection (the learned
                                 gate network when gate weights are given)
    attend(q, lens)              sparse (or dense) decode attention
    step(q, lens)                select + attend, the gate fused into the attention
                                 kernel (two launches; with a learned gate, its
                                 score launch, then the attention kernel selecting
                                 from those scores where that applies, then the merge)
    step_append(q, old, new)     append, then step (the append inside the gate's score
                                 kernel where there is one)
    step_unfused(q, lens)        select, then attend (three launches)

all on torch's current stream, with no host synchronisation.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import seer


class DecodeState:
    def __init__(self, *, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, max_blocks: int, dtype: torch.dtype, k: torch.Tensor,
                 v: torch.Tensor, page_table: Optional[torch.Tensor] = None,
                 k_max: Optional[int] = None, keep: Optional[tuple] = None,
                 top_k: Optional[torch.Tensor] = None, threshold: Optional[float] = None,
                 force_first: bool = False, force_last: bool = False, unified: bool = False,
                 gate_weights=None, query_tokens: int = 1, fuse=None,
                 combine: int = seer.SEER_COMBINE_AUTO):
        self.shape = seer.make_shape(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                     max_blocks, dtype)
        self.k, self.v, self.page_table = k, v, page_table
        self.kv = seer.make_kv(k, v, page_table)
        self.keep = keep
        self.top_k = top_k
        # learned gate: device tensors w1, w1_scale, b1, wq (or None: parameter-free gate)
        self.gate_weights = gate_weights
        # new query tokens per sequence (q [B][T][Hq][d] when T > 1)
        self.T = int(query_tokens)
        if self.T > 1 and gate_weights is not None:
            raise ValueError("the learned gate takes one query token per sequence")
        self.rule = seer.make_select(top_k=top_k, keep=keep, threshold=threshold,
                                     force_first=force_first, force_last=force_last,
                                     unified=unified, fuse=fuse)
        # single-token combine: the library's choice, or one kernel forced
        self.combine = int(combine)
        if k_max is None:
            if keep is not None and threshold is None:
                k_max = seer.keep_blocks(max_blocks, keep[0], keep[1])
                k_max = min(max_blocks, k_max + int(force_first) + int(force_last))
            else:
                k_max = max_blocks
        self.k_max = int(k_max)
        dev = k.device
        U = batch * num_kv_heads
        self.pooled = torch.zeros(U * head_dim * max_blocks, dtype=torch.float32, device=dev)
        self.open_sum = torch.zeros(U * head_dim, dtype=torch.float64, device=dev)
        self.scores = torch.zeros(U * max_blocks, dtype=torch.float64, device=dev)
        self.sel_idx = torch.full((U, self.k_max), -1, dtype=torch.int32, device=dev)
        self.sel_cnt = torch.zeros(U, dtype=torch.int32, device=dev)
        tok = (self.T,) if self.T > 1 else ()
        self.out = torch.zeros((batch, *tok, num_q_heads, head_dim), dtype=torch.float32,
                               device=dev)
        self.lse = torch.zeros((batch, *tok, num_q_heads), dtype=torch.float32, device=dev)
        if self.T > 1:
            self.workspace = torch.empty(seer.multi_decode_workspace_size(self.shape, self.T),
                                         dtype=torch.uint8, device=dev)
        else:
            self.workspace = seer.alloc_workspace(self.shape, dev)

    # pooling ---------------------------------------------------------------
    def build_pool(self, lens: torch.Tensor):
        seer.block_pool_keys(self.shape, self.kv, None, lens, self.pooled, self.open_sum)

    def append(self, lens_old: torch.Tensor, lens_new: torch.Tensor):
        seer.block_pool_keys(self.shape, self.kv, lens_old, lens_new, self.pooled, self.open_sum)

    # selection -------------------------------------------------------------
    def select(self, q: torch.Tensor, lens: torch.Tensor):
        if self.T > 1:
            seer.multi_gate_select(self.shape, self.T, q, self.pooled, lens, self.rule,
                                   self.k_max, self.scores, self.sel_idx, self.sel_cnt)
        elif self.gate_weights is not None:
            seer.learned_gate_select(self.shape, q, self.pooled, lens, self.gate_weights,
                                     self.rule, self.k_max, self.scores, self.sel_idx,
                                     self.sel_cnt)
        else:
            seer.gate_select(self.shape, q, self.pooled, lens, self.rule, self.k_max,
                             self.scores, self.sel_idx, self.sel_cnt)

    # attention -------------------------------------------------------------
    def attend(self, q: torch.Tensor, lens: torch.Tensor, dense: bool = False,
               sel_idx: Optional[torch.Tensor] = None, sel_cnt: Optional[torch.Tensor] = None,
               k_max: Optional[int] = None):
        if dense:
            si, sc, km = None, None, self.shape.max_blocks
        elif sel_idx is not None:
            si, sc, km = sel_idx, sel_cnt, int(k_max if k_max is not None else sel_idx.shape[-1])
        else:
            si, sc, km = self.sel_idx, self.sel_cnt, self.k_max
        if self.T > 1:
            seer.multi_sparse_decode(self.shape, self.T, q, self.kv, lens, si, sc, km, self.out,
                                     self.lse, self.workspace)
        elif self.combine != seer.SEER_COMBINE_AUTO:
            seer.sparse_decode_partial(self.shape, q, self.kv, lens, si, sc, km, self.workspace)
            seer.sparse_decode_combine(self.shape, self.out, self.lse, self.workspace,
                                       self.combine)
        else:
            seer.sparse_decode(self.shape, q, self.kv, lens, si, sc, km, self.out, self.lse,
                               self.workspace)
        return self.out, self.lse

    def step(self, q: torch.Tensor, lens: torch.Tensor):
        """Gate, select and attend: one decode step over a built pooled table
        (the parameter-free gate fused into the attention kernel where that
        pays, for one or several query tokens)."""
        if self.gate_weights is not None:
            auto = self.combine == seer.SEER_COMBINE_AUTO
            seer.learned_gated_sparse_decode(self.shape, q, self.kv, lens, self.pooled,
                                             self.gate_weights, self.rule, self.k_max,
                                             self.scores, self.sel_idx, self.sel_cnt,
                                             self.out if auto else None, self.lse if auto else None,
                                             self.workspace)
            if not auto:
                seer.sparse_decode_combine(self.shape, self.out, self.lse, self.workspace,
                                           self.combine)
            return self.out, self.lse
        if self.T > 1:
            seer.multi_gated_sparse_decode(self.shape, self.T, q, self.kv, lens, self.pooled,
                                           self.rule, self.k_max, self.scores, self.sel_idx,
                                           self.sel_cnt, self.out, self.lse, self.workspace)
            return self.out, self.lse
        if self.combine != seer.SEER_COMBINE_AUTO:
            seer.gated_sparse_decode(self.shape, q, self.kv, lens, self.pooled, self.rule,
                                     self.k_max, self.scores, self.sel_idx, self.sel_cnt, None,
                                     None, self.workspace)
            seer.sparse_decode_combine(self.shape, self.out, self.lse, self.workspace,
                                       self.combine)
            return self.out, self.lse
        seer.gated_sparse_decode(self.shape, q, self.kv, lens, self.pooled, self.rule,
                                 self.k_max, self.scores, self.sel_idx, self.sel_cnt, self.out,
                                 self.lse, self.workspace)
        return self.out, self.lse

    def step_append(self, q: torch.Tensor, lens_old: torch.Tensor, lens_new: torch.Tensor):
        """append(lens_old, lens_new) then step(q, lens_new), as one call (the
        pooling append inside the gate's score kernel where it has one)."""
        if self.gate_weights is not None or self.T > 1 or self.combine != seer.SEER_COMBINE_AUTO:
            self.append(lens_old, lens_new)
            return self.step(q, lens_new)
        seer.gated_sparse_decode_append(self.shape, q, self.kv, lens_old, lens_new, self.pooled,
                                        self.open_sum, self.rule, self.k_max, self.scores,
                                        self.sel_idx, self.sel_cnt, self.out, self.lse,
                                        self.workspace)
        return self.out, self.lse

    def step_unfused(self, q: torch.Tensor, lens: torch.Tensor):
        """The same step as three launches: gate kernel, then attention."""
        self.select(q, lens)
        return self.attend(q, lens)
