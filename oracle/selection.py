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


def focus_select(delta, k, decoded, rightmost_processed):
    """The kept index set S of FOCUS token eviction, per sequence.

    Followed: FOCUS paper Section 4.2 (top-K masked tokens by delta, then two
    structural constraints: AR-context preservation keeps each candidate's
    immediate predecessor; placeholder integrity keeps the unprocessed masked
    tokens preceding any selected candidate); App. E.2.2 (the same
    constraints in one kernel, placeholder integrity as retaining tokens up
    to the maximum selected index, and |S| >= 1); App. E.3.1
    (rightmost_processed = max(previous, the position processed now)); FOCUS
    notes page, key design 3.

    Readings: candidates are the top-K of the eligible (not decoded, not NaN,
    not -inf) positions in the top-K order of ``topk_select``; the
    predecessor i-1 of every candidate i >= 1 is kept whatever its state;
    placeholders are the masked positions j with rightmost_processed < j <
    max(candidates); if S is still empty, it holds the single first position
    of the order (score descending, index ascending) over all positions,
    with -inf ranked above NaN; the new rightmost_processed is
    max(old, max(S)).

    delta [batch, B] float; k [batch] int; decoded [batch, B] bool;
    rightmost_processed [batch] int -> (idx [batch, B] int32 ascending,
    -1 padded; count [batch]; cu [batch + 1]; new rightmost_processed).
    """
    delta = np.asarray(delta)
    dec = np.asarray(decoded).astype(bool)
    batch, block = delta.shape
    idx = np.full((batch, block), -1, dtype=np.int32)
    count = np.zeros(batch, dtype=np.int32)
    rp_new = np.asarray(rightmost_processed, dtype=np.int32).copy()
    for b in range(batch):
        row = [float(x) for x in delta[b]]
        elig = [j for j in range(block)
                if not dec[b, j] and not math.isnan(row[j]) and row[j] > -math.inf]
        ranked = sorted(elig, key=lambda j: (-row[j], j))
        keff = min(max(int(k[b]), 0), len(ranked))
        cand = ranked[:keff]
        s = set(cand)
        s.update(i - 1 for i in cand if i >= 1)
        if cand:
            rp = int(rightmost_processed[b])
            s.update(j for j in range(rp + 1, max(cand)) if not dec[b, j])
        if not s:
            def rank_key(j):
                x = row[j]
                return (1, j) if math.isnan(x) else (0, -x, j)
            s = {min(range(block), key=rank_key)}
        chosen = sorted(s)
        idx[b, :len(chosen)] = chosen
        count[b] = len(chosen)
        rp_new[b] = max(int(rightmost_processed[b]), chosen[-1])
    cu = np.zeros(batch + 1, dtype=np.int32)
    cu[1:] = np.cumsum(count)
    return idx, count, cu, rp_new
