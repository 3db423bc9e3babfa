"""Per-sequence top-K selection (oracle; test use only).

Followed: FOCUS paper Section 4.2 (indices of the top-K masked tokens by
Delta-I); ES-dLLM notes page, key design 1 (keep the top-(1 - r_l)|S|
positions by score); FOCUS paper App. E.2.3 (destinations of the compacted
rows come from a prefix sum of the per-sequence kept counts).

Readings: a score that is NaN or -inf is not eligible (decoded positions
carry -inf). Order is score descending, then index ascending; -0.0 and +0.0
are equal. K_eff = min(max(K, 0), #eligible, k_max). The kept indices are
written in ascending index order, padded with -1; cu is the exclusive
prefix sum of the kept counts. Under these readings the result is unique.
"""
from __future__ import annotations

import math

import numpy as np


def topk_select(scores, k, k_max: int):
    """scores [batch, n] float, k [batch] int -> (idx [batch, k_max] int32,
    count [batch] int32, cu [batch + 1] int32)."""
    scores = np.asarray(scores)
    k = np.asarray(k)
    batch, n = scores.shape
    idx = np.full((batch, k_max), -1, dtype=np.int32)
    count = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        row = [float(x) for x in scores[b]]
        eligible = [j for j in range(n) if not math.isnan(row[j]) and row[j] > -math.inf]
        ranked = sorted(eligible, key=lambda j: (-row[j], j))
        keff = min(max(int(k[b]), 0), len(ranked), k_max)
        chosen = sorted(ranked[:keff])
        idx[b, :keff] = chosen
        count[b] = keff
    cu = np.zeros(batch + 1, dtype=np.int32)
    cu[1:] = np.cumsum(count)
    return idx, count, cu
