"""One denoising step of the token-eviction hot path on preallocated buffers.

FOCUS mode (FOCUS paper Section 4.2 and Figure 5's flow: delta from layers 0
and 1, top-K under the budget, gather of the kept rows; then, for every later
layer, the KV scatter and the reduced-query attention):

    focus_importance_delta -> topk_select -> gather_rows -> kv_scatter -> reduced_attention

ES-dLLM mode (ES-dLLM notes page, key designs 1 and 2: score the survivors,
keep the top ones, gather their rows, scatter their new K/V in place):

    esdllm_score -> topk_select -> gather_rows -> kv_scatter

Every call enqueues HIP kernels on the current stream; nothing here reads
device data back or synchronises. Per-sequence counts stay on the device, so
the output buffers are sized by the host-side bound batch * k_max rows.
"""
from __future__ import annotations

import math

import torch

from . import (attention_order, esdllm_score, focus_importance_delta, gather_rows, kv_scatter,
               reduced_attention, topk_select)


class FocusStep:
    def __init__(self, batch: int, block: int, hidden: int, hq: int, head_dim: int, k_max: int,
                 dtype: torch.dtype, device):
        self.batch, self.block, self.k_max = batch, block, k_max
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
        """Longest-first work order of the step's attention calls (one per step:
        every layer of the step sees the same lengths)."""
        return attention_order(kv_len, out=self.order)

    def attend(self, q_kept, cache_k, cache_v, seq_start, kv_len):
        return reduced_attention(q_kept, self.count, self.cu, cache_k, cache_v, seq_start, kv_len,
                                 self.k_max, self.scale, out=self.out, order=self.order)

    def run(self, *, q0, k0, q1, k1, decoded, k, hidden_rows, pool_kernel, new_k, new_v, q_kept,
            cache_k, cache_v, seq_start, kv_len, row_base):
        self.score(q0, k0, q1, k1, decoded, pool_kernel)
        self.select(k)
        self.gather(hidden_rows)
        self.scatter(new_k, new_v, row_base, cache_k, cache_v)
        self.schedule(kv_len)
        self.attend(q_kept, cache_k, cache_v, seq_start, kv_len)
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
