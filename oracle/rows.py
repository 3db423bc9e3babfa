"""Row gather (compaction) and row scatter into the KV cache (oracle; test use only).

Gather — FOCUS paper Section 4.2: the block hidden states H (B x h) are
gathered at the index set into H_reduced (|S| x h); App. E.2.3: the
destination of each kept row is given by a prefix sum over sequences.
Here: dst[cu[b] + t] = src[b, idx[b, t]] for t < count[b].

Scatter — ES-dLLM notes page, key design 2: the new K/V of the surviving
positions is written in place into the full KV cache and every other slot
keeps its old contents; FOCUS paper App. E.2.4 (sparse KV cache filling at
pre-computed processing indices). Here: cache[row_base[b] + pos] =
new[cu[b] + t] with pos = idx[b, t], or pos_map[b, idx[b, t]] when a
position map is given.

Both are byte copies: they work on uint8 views, so the result is exact for
any element type.
"""
from __future__ import annotations

import numpy as np


def _bytes(a: np.ndarray, rows: int) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.size == 0:                    # no rows to copy (e.g. a sequence with nothing kept)
        return np.zeros((rows, 0), dtype=np.uint8)
    return a.view(np.uint8).reshape(rows, -1)


def gather_rows(src: np.ndarray, idx, count, cu) -> np.ndarray:
    """src [batch, n, ...] -> dst [cu[-1], ...] (same dtype)."""
    batch, n = src.shape[0], src.shape[1]
    s = _bytes(src, batch * n)
    total = int(cu[batch])
    d = np.zeros((total, s.shape[1]), dtype=np.uint8)
    for b in range(batch):
        for t in range(int(count[b])):
            d[int(cu[b]) + t] = s[b * n + int(idx[b, t])]
    return d.view(src.dtype).reshape((total,) + src.shape[2:])


def gather_rows_ragged(src: np.ndarray, src_cu, idx, count, cu) -> np.ndarray:
    """Gather from rows that are themselves compacted by sequence (a skip
    layer's output exists only for its survivors, ES-dLLM notes page, key
    design 2): dst[cu[b] + t] = src[src_cu[b] + idx[b, t]] for t < count[b]."""
    rows = src.shape[0]
    s = _bytes(src, rows)
    batch = len(count)
    total = int(cu[batch])
    d = np.zeros((total, s.shape[1]), dtype=np.uint8)
    for b in range(batch):
        for t in range(int(count[b])):
            d[int(cu[b]) + t] = s[int(src_cu[b]) + int(idx[b, t])]
    return d.view(src.dtype).reshape((total,) + src.shape[1:])


def gather_rows_multi(srcs, idx, count, cu):
    """Each src [batch, n, ...] gathered with the same index set (FOCUS paper
    App. E.2.3: hidden states, residual, RoPE positions and cache indices are
    compacted together)."""
    return [gather_rows(s, idx, count, cu) for s in srcs]


def kv_scatter(new_k: np.ndarray, new_v: np.ndarray, idx, count, cu, row_base,
               cache_k: np.ndarray, cache_v: np.ndarray, pos_map=None):
    """Returns updated copies (cache_k', cache_v'); the inputs are not modified."""
    out = []
    for new, cache in ((new_k, cache_k), (new_v, cache_v)):
        rows = cache.shape[0]
        c = _bytes(cache, rows).copy()
        nb = _bytes(new, new.shape[0])
        for b in range(len(count)):
            for t in range(int(count[b])):
                j = int(idx[b, t])
                pos = j if pos_map is None else int(pos_map[b, j])
                c[int(row_base[b]) + pos] = nb[int(cu[b]) + t]
        out.append(c.view(cache.dtype).reshape(cache.shape))
    return out[0], out[1]
