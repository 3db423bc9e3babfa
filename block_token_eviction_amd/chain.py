"""One denoising step of the token-eviction hot path on preallocated buffers.

FOCUS mode (FOCUS paper Section 4.2 and Figure 5's flow: delta from layers 0
and 1, top-K under the budget, gather of the kept rows; then, for every later
layer, the KV scatter and the reduced-query attention):

    focus_importance_delta -> topk_select -> gather_rows -> kv_scatter
        -> attention_order (longest first) -> reduced_attention

Extended FOCUS step (FOCUS paper Section 4.1 budget, Section 4.2 selection
with its structural constraints, Section 4.3 delayed commit; App. E.2.2 to
E.3.1 for the fused selection, the one-launch compaction, the paged pool
and the per-sequence history):

    focus_importance_delta -> focus_budget -> focus_select -> gather_rows_multi
        -> kv_scatter_paged -> attention_order -> reduced_attention_paged
        -> focus_commit_mask -> focus_history_update

ES-dLLM mode (ES-dLLM notes page, key designs 1 and 2: score the survivors,
keep the top ones, gather their rows, scatter their new K/V in place):

    esdllm_score -> topk_select -> gather_rows -> kv_scatter

In both FOCUS steps the KV scatter and the attention can run as one launch
(kv_scatter_attention / kv_scatter_attention_paged, bitwise the same caches
and outputs): the attention takes the kept positions' K/V from the new rows
and writes them into the cache, so the scattered bytes ride in the
attention's stream instead of a separate short launch.

ES-dLLM skip layer (the same page: at a skip layer the survivors are scored,
the layer's hidden-state cache is updated in place at every survivor, and
only the top (1 - r)|S| survivors go on to the next layer):

    esdllm_score_update (score + hidden-cache update in one pass) -> topk_select
        -> gather_rows_multi (kept hidden rows + their positions)

ES-dLLM iteration (the same page, key design 2: the initial full pass and a
periodic refresh run without skipping; every iteration starts from the whole
block). Per-sequence counters make survivor sets ragged within a batch, so the
survivors of each layer are compacted by sequence (count, cu):

    esdllm_schedule -> [esdllm_score_update -> topk_select
        -> gather_rows_multi_ragged] per skip layer

Every call enqueues HIP kernels on the current stream; nothing here reads
device data back or synchronises. Per-sequence counts stay on the device, so
the output buffers are sized by the host-side bound batch * k_max rows.
"""
from __future__ import annotations

import math

import torch

from . import (attention_order, esdllm_schedule, esdllm_score, esdllm_score_update, focus_budget,
               focus_commit_mask, focus_history_update, focus_importance_delta, focus_select,
               gather_rows, gather_rows_multi, gather_rows_multi_ragged, kv_scatter,
               kv_scatter_attention, kv_scatter_attention_paged, kv_scatter_paged,
               reduced_attention, reduced_attention_paged, topk_select)


class FocusStep:
    def __init__(self, batch: int, block: int, hidden: int, hq: int, head_dim: int, k_max: int,
                 dtype: torch.dtype, device, hkv: int | None = None):
        """hkv (KV heads): when given, the attention order weighs each sequence's length
        by its query passes (attention_order with the kept counts)."""
        self.batch, self.block, self.k_max = batch, block, k_max
        self.group = None if hkv is None else hq // hkv
        self.scale = 1.0 / math.sqrt(head_dim)
        i32 = dict(dtype=torch.int32, device=device)
        self.delta = torch.empty((batch, block), dtype=torch.float32, device=device)
        self.idx = torch.empty((batch, k_max), **i32)
        self.count = torch.empty((batch,), **i32)
        self.cu = torch.empty((batch + 1,), **i32)
        self.gathered = torch.empty((batch * k_max, hidden), dtype=dtype, device=device)
        self.out = torch.empty((batch * k_max, hq, head_dim), dtype=dtype, device=device)
        self.order = torch.empty((batch,), **i32)

    def score(self, q0, k0, q1, k1, decoded, pool_kernel):
        return focus_importance_delta(q0, k0, q1, k1, decoded, pool_kernel, out=self.delta)

    def select(self, k):
        return topk_select(self.delta, k, self.k_max, self.idx, self.count, self.cu)

    def gather(self, hidden_rows):
        return gather_rows(hidden_rows, self.idx, self.count, self.cu, out=self.gathered)

    def scatter(self, new_k, new_v, row_base, cache_k, cache_v):
        return kv_scatter(new_k, new_v, self.idx, self.count, self.cu, row_base, cache_k, cache_v)

    def schedule(self, kv_len):
        """Largest-first work order of the step's attention calls (one per step:
        every layer of the step sees the same lengths and kept counts)."""
        if self.group is None:
            return attention_order(kv_len, out=self.order)
        return attention_order(kv_len, out=self.order, count=self.count, group=self.group)

    def attend(self, q_kept, cache_k, cache_v, seq_start, kv_len):
        return reduced_attention(q_kept, self.count, self.cu, cache_k, cache_v, seq_start, kv_len,
                                 self.k_max, self.scale, out=self.out, order=self.order)

    def scatter_attend(self, q_kept, new_k, new_v, pos_base, cache_k, cache_v, seq_start, kv_len):
        """scatter (into rows seq_start + pos_base + idx) and attend in one launch."""
        return kv_scatter_attention(q_kept, self.count, self.cu, self.idx, self.block, pos_base,
                                    new_k, new_v, cache_k, cache_v, seq_start, kv_len, self.k_max,
                                    self.scale, out=self.out, order=self.order)

    def run(self, *, q0, k0, q1, k1, decoded, k, hidden_rows, pool_kernel, new_k, new_v, q_kept,
            cache_k, cache_v, seq_start, kv_len, row_base=None, pos_base=None, fused=False):
        """fused: one scatter + attention launch (needs pos_base, int32 [batch], the block's
        first KV position); otherwise kv_scatter into row_base, then reduced_attention."""
        self.score(q0, k0, q1, k1, decoded, pool_kernel)
        self.select(k)
        self.gather(hidden_rows)
        if fused:
            self.schedule(kv_len)
            self.scatter_attend(q_kept, new_k, new_v, pos_base, cache_k, cache_v, seq_start, kv_len)
        else:
            self.scatter(new_k, new_v, row_base, cache_k, cache_v)
            self.schedule(kv_len)
            self.attend(q_kept, cache_k, cache_v, seq_start, kv_len)
        return self.out


class FocusFullStep:
    """The FOCUS step with the device-side budget and history, the constrained
    selection (|S| up to B rows per sequence), one compaction launch for the
    per-token tensors, a paged KV pool and the delayed commit mask. The
    per-sequence state (token_sum, total_steps, rightmost_processed, cached)
    is the caller's and is updated in place."""

    def __init__(self, batch: int, block: int, hq: int, head_dim: int, row_shapes, dtype: torch.dtype,
                 device, hkv: int | None = None):
        """row_shapes: (shape of one row, dtype) of each per-token tensor to compact.
        hkv (KV heads): when given, the attention order weighs lengths by query passes."""
        self.batch, self.block = batch, block
        self.group = None if hkv is None else hq // hkv
        self.scale = 1.0 / math.sqrt(head_dim)
        i32 = dict(dtype=torch.int32, device=device)
        cap = batch * block
        self.delta = torch.empty((batch, block), dtype=torch.float32, device=device)
        self.k = torch.empty((batch,), **i32)
        self.idx = torch.empty((batch, block), **i32)
        self.count = torch.empty((batch,), **i32)
        self.cu = torch.empty((batch + 1,), **i32)
        self.rows = [torch.empty((cap,) + tuple(shape), dtype=dt, device=device)
                     for shape, dt in row_shapes]
        self.order = torch.empty((batch,), **i32)
        self.out = torch.empty((cap, hq, head_dim), dtype=dtype, device=device)
        self.commit = torch.empty((batch, block), dtype=torch.uint8, device=device)
        self.block_done = torch.empty((batch,), **i32)

    def score(self, q0, k0, q1, k1, decoded, pool_kernel):
        return focus_importance_delta(q0, k0, q1, k1, decoded, pool_kernel, out=self.delta)

    def budget(self, token_sum, total_steps, alpha, threshold_mode=0):
        return focus_budget(self.delta, token_sum, total_steps, alpha, threshold_mode, out=self.k)

    def select(self, decoded, rightmost_processed):
        return focus_select(self.delta, self.k, decoded, rightmost_processed, self.idx, self.count,
                            self.cu)

    def compact(self, per_token):
        return gather_rows_multi(per_token, self.idx, self.count, self.cu, outs=self.rows)

    def scatter(self, new_k, new_v, pos_base, block_table, page_size, pool_k, pool_v):
        return kv_scatter_paged(new_k, new_v, self.idx, self.count, self.cu, pos_base, block_table,
                                page_size, pool_k, pool_v)

    def schedule(self, kv_len):
        if self.group is None:
            return attention_order(kv_len, out=self.order)
        return attention_order(kv_len, out=self.order, count=self.count, group=self.group)

    def attend(self, q_kept, pool_k, pool_v, block_table, page_size, kv_len):
        return reduced_attention_paged(q_kept, self.count, self.cu, pool_k, pool_v, block_table,
                                       page_size, kv_len, self.block, self.scale, out=self.out,
                                       order=self.order)

    def scatter_attend(self, q_kept, new_k, new_v, pos_base, block_table, page_size, pool_k,
                       pool_v, kv_len):
        """scatter (logical positions pos_base + idx) and attend in one launch."""
        return kv_scatter_attention_paged(q_kept, self.count, self.cu, self.idx, self.block,
                                          pos_base, new_k, new_v, pool_k, pool_v, block_table,
                                          page_size, kv_len, self.block, self.scale, out=self.out,
                                          order=self.order)

    def commit_mask(self, decoded, cached):
        return focus_commit_mask(decoded, cached, self.commit, self.block_done)

    def history(self, decoded, decoded_now, token_sum, total_steps):
        return focus_history_update(decoded, decoded_now, token_sum, total_steps)

    def run(self, *, q0, k0, q1, k1, decoded, decoded_now, pool_kernel, alpha, token_sum,
            total_steps, rightmost_processed, cached, per_token, new_k, new_v, q_kept, pos_base,
            block_table, page_size, pool_k, pool_v, kv_len, threshold_mode=0, fused=False):
        self.score(q0, k0, q1, k1, decoded, pool_kernel)
        self.budget(token_sum, total_steps, alpha, threshold_mode)
        self.select(decoded, rightmost_processed)
        self.compact(per_token)
        if fused:
            self.schedule(kv_len)
            self.scatter_attend(q_kept, new_k, new_v, pos_base, block_table, page_size, pool_k,
                                pool_v, kv_len)
        else:
            self.scatter(new_k, new_v, pos_base, block_table, page_size, pool_k, pool_v)
            self.schedule(kv_len)
            self.attend(q_kept, pool_k, pool_v, block_table, page_size, kv_len)
        self.commit_mask(decoded, cached)
        self.history(decoded, decoded_now, token_sum, total_steps)
        return self.out


class EsStep:
    def __init__(self, batch: int, n_surv: int, hidden: int, k_max: int, dtype: torch.dtype, device):
        self.k_max = k_max
        i32 = dict(dtype=torch.int32, device=device)
        self.score = torch.empty((batch, n_surv), dtype=torch.float32, device=device)
        self.idx = torch.empty((batch, k_max), **i32)
        self.count = torch.empty((batch,), **i32)
        self.cu = torch.empty((batch + 1,), **i32)
        self.gathered = torch.empty((batch * k_max, hidden), dtype=dtype, device=device)

    def run(self, *, h_new, h_prev, surv_pos, conf, alpha, k, new_k, new_v, row_base, cache_k,
            cache_v):
        esdllm_score(h_new, h_prev, surv_pos, conf, alpha, out=self.score)
        topk_select(self.score, k, self.k_max, self.idx, self.count, self.cu)
        gather_rows(h_new, self.idx, self.count, self.cu, out=self.gathered)
        kv_scatter(new_k, new_v, self.idx, self.count, self.cu, row_base, cache_k, cache_v,
                   pos_map=surv_pos)
        return self.gathered


class EsSkipLayer:
    """One ES-dLLM skip layer on preallocated buffers. h_cache is the layer's
    hidden-state cache [batch, seq_len, hidden] from the previous iteration,
    updated in place; the kept survivors (ascending) and their hidden rows are
    returned for the next layer."""

    def __init__(self, batch: int, n_surv: int, keep: int, seq_len: int, hidden: int,
                 dtype: torch.dtype, device):
        self.batch, self.n_surv, self.keep, self.seq_len = batch, n_surv, keep, seq_len
        i32 = dict(dtype=torch.int32, device=device)
        self.score = torch.empty((batch, n_surv), dtype=torch.float32, device=device)
        self.k = torch.full((batch,), keep, **i32)
        self.idx = torch.empty((batch, keep), **i32)
        self.count = torch.empty((batch,), **i32)
        self.cu = torch.empty((batch + 1,), **i32)
        self.h_next = torch.empty((batch * keep, hidden), dtype=dtype, device=device)
        self.surv_next = torch.empty((batch * keep,), **i32)

    def run(self, h_surv, h_cache, surv_pos, conf, alpha: float):
        """h_surv [batch, n_surv, hidden] this iteration's states of the survivors."""
        b = self.batch
        esdllm_score_update(h_surv, h_cache, surv_pos, conf, alpha, out=self.score)
        topk_select(self.score, self.k, self.keep, self.idx, self.count, self.cu)
        gather_rows_multi([h_surv, surv_pos], self.idx, self.count, self.cu,
                          outs=[self.h_next, self.surv_next])
        return self.h_next.view(b, self.keep, -1), self.surv_next.view(b, self.keep)


class EsIteration:
    """One iteration of ES-dLLM's skip pipeline with its device-side bookkeeping,
    on preallocated buffers. The caller owns the per-sequence iteration counters
    (`iter`, int32 [batch], advanced in place) and the block starts; each skip
    layer l has its hidden-state cache h_caches[l] [batch, seq_len, hidden],
    updated in place. keep: the skip iterations' keep counts per skip layer
    (floor((1 - r_l)|S_l|)); refresh iterations keep every survivor."""

    def __init__(self, batch: int, block_len: int, hidden: int, keep, period: int,
                 dtype: torch.dtype, device):
        self.batch, self.block_len, self.keep, self.period = batch, block_len, list(keep), period
        i32 = dict(dtype=torch.int32, device=device)
        n_l = len(self.keep)
        cap = batch * block_len
        self.surv0 = torch.empty((batch, block_len), **i32)
        self.count0 = torch.empty((batch,), **i32)
        self.cu0 = torch.empty((batch + 1,), **i32)
        self.keep_out = torch.empty((max(n_l, 1), batch), **i32)
        self.refresh = torch.empty((batch,), dtype=torch.uint8, device=device)
        self.score = [torch.empty((batch, block_len), dtype=torch.float32, device=device)
                      for _ in range(n_l)]
        self.idx = [torch.empty((batch, block_len), **i32) for _ in range(n_l)]
        self.count = [torch.empty((batch,), **i32) for _ in range(n_l)]
        self.cu = [torch.empty((batch + 1,), **i32) for _ in range(n_l)]
        self.h_next = [torch.empty((cap, hidden), dtype=dtype, device=device) for _ in range(n_l)]
        self.surv_next = [torch.empty((cap,), **i32) for _ in range(n_l)]

    def schedule(self, iter_, block_start):
        return esdllm_schedule(iter_, block_start, self.block_len, self.period, self.keep,
                               self.surv0, self.count0, self.cu0, self.keep_out, self.refresh)

    def layer(self, l: int, h_rows, surv_rows, count, cu, h_cache, conf, alpha: float):
        """Skip layer l on survivors compacted by (count, cu): h_rows [rows, hidden] their
        states, surv_rows int32 [rows] their positions. Returns the kept survivors
        (h_next, surv_next, count, cu), compacted the same way."""
        esdllm_score_update(h_rows, h_cache, surv_rows, conf, alpha, count=count, cu=cu,
                            cap=self.block_len, out=self.score[l])
        topk_select(self.score[l], self.keep_out[l], self.block_len, self.idx[l], self.count[l],
                    self.cu[l])
        gather_rows_multi_ragged([h_rows, surv_rows], cu, self.idx[l], self.count[l], self.cu[l],
                                 outs=[self.h_next[l], self.surv_next[l]])
        return self.h_next[l], self.surv_next[l], self.count[l], self.cu[l]

    def run(self, iter_, block_start, layer_states, h_caches, conf, alpha: float):
        """layer_states(l, surv_rows, count, cu) -> h_rows: the model's output of the layer
        before skip layer l for the survivors (outside this library)."""
        surv, count, cu, _, _ = self.schedule(iter_, block_start)
        rows = surv.view(-1)
        h = None
        for l in range(len(self.keep)):
            h_rows = layer_states(l, rows, count, cu)
            h, rows, count, cu = self.layer(l, h_rows, rows, count, cu, h_caches[l], conf, alpha)
        return h, rows, count, cu
