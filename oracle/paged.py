"""Paged KV cache: scatter and reduced attention through a page table (oracle;
test use only).

Followed: FOCUS paper App. E.2.4 (FOCUS runs on a PagedAttention memory pool:
a sparse KV fill writes the processed positions' K/V to their physical
block offsets; ragged attention reads each sequence's KV through the page
mapping); FOCUS paper Section 5 (the LMDeploy engine with PagedAttention).

A sequence's logical KV position p lives in physical cache row
    block_table[b, p // page_size] * page_size + p % page_size
of a pool of pages of page_size rows. Both operations are defined through
this mapping by the contiguous ones: the scatter writes the same rows the
contiguous scatter would, at their mapped places; the attention reads the
sequence's rows 0 .. kv_len-1 in logical order through the mapping and
computes exactly the contiguous attention on them.
"""
from __future__ import annotations

import numpy as np

from .attention import reduced_attention
from .rows import _bytes


def physical_row(block_table, b: int, p: int, page_size: int) -> int:
    return int(block_table[b, p // page_size]) * page_size + p % page_size


def kv_scatter_paged(new_k, new_v, idx, count, cu, pos_base, block_table, page_size: int,
                     cache_k, cache_v, pos_map=None):
    """cache[physical_row(b, pos_base[b] + pos)] = new[cu[b] + t], pos = idx or pos_map[b, idx].
    Returns updated copies; the inputs are not modified."""
    out = []
    for new, cache in ((new_k, cache_k), (new_v, cache_v)):
        c = _bytes(cache, cache.shape[0]).copy()
        nb = _bytes(new, new.shape[0])
        for b in range(len(count)):
            for t in range(int(count[b])):
                j = int(idx[b, t])
                pos = j if pos_map is None else int(pos_map[b, j])
                c[physical_row(block_table, b, int(pos_base[b]) + pos, page_size)] = nb[int(cu[b]) + t]
        out.append(c.view(cache.dtype).reshape(cache.shape))
    return out[0], out[1]


def gather_sequences(cache, block_table, page_size: int, kv_len):
    """The sequences' KV rows in logical order, laid out contiguously, and
    their starts: (rows [sum kv_len, ...], seq_start [batch])."""
    rows = []
    for b in range(len(kv_len)):
        rows.extend(physical_row(block_table, b, p, page_size) for p in range(int(kv_len[b])))
    seq_start = np.zeros(len(kv_len), np.int64)
    seq_start[1:] = np.cumsum(np.asarray(kv_len, np.int64))[:-1]
    return np.asarray(cache)[np.asarray(rows, np.int64)], seq_start


def reduced_attention_paged(q, count, cu, cache_k, cache_v, block_table, page_size: int, kv_len,
                            hq: int, hkv: int, scale: float, rows=None) -> np.ndarray:
    k, ss = gather_sequences(cache_k, block_table, page_size, kv_len)
    v, _ = gather_sequences(cache_v, block_table, page_size, kv_len)
    return reduced_attention(q, count, cu, k, v, ss, kv_len, hq, hkv, scale, rows=rows)
