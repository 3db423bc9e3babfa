"""FOCUS dynamic budget and its history update (oracle; test use only).

Followed: FOCUS notes page, key design 2 (the budget
K = min(B, max(ceil(alpha * N_bar), N_sigma)), with N_sigma the number of
masked block positions whose importance delta is at least one standard
deviation, and N_bar = 1 before any history) and its worked example; FOCUS
paper Section 4.1 (the same budget), App. E.3.1 (per-sequence history:
token_sum += n_decoded, total_steps += 1, N_bar = token_sum / total_steps),
App. E.2.2 (the selection kernel's variant threshold: delta > mu + sigma)
and App. D.2 (eviction iff delta < sigma).

Readings: the masked positions are those whose delta is finite (decoded
positions carry -inf); mean and standard deviation are the population ones
over the masked positions of the block, summed in ascending position order
in float64; "delta >= sigma" is decided exactly as delta >= 0 and
delta^2 >= variance (mode 0), "delta > mu + sigma" as d = delta - mu > 0 and
d^2 > variance (mode 1); no masked position gives N_sigma = 0; the history
average is token_sum / total_steps in float64, and 1 when total_steps is 0.
These are the GPU kernel's decisions in the same precision and order, so the
budgets agree exactly.
"""
from __future__ import annotations

import math

import numpy as np


def _sigma_count(row, mode: int) -> int:
    xs = [float(x) for x in row if math.isfinite(float(x))]
    n = len(xs)
    if n == 0:
        return 0
    total = 0.0
    for x in xs:
        total += x
    mu = total / n
    ss = 0.0
    for x in xs:
        d = x - mu
        ss += d * d
    var = ss / n
    if mode == 0:
        return sum(1 for x in xs if x >= 0.0 and x * x >= var)
    count = 0
    for x in xs:
        d = x - mu
        if d > 0.0 and d * d > var:
            count += 1
    return count


def focus_budget(delta, token_sum, total_steps, alpha: float, mode: int = 0) -> np.ndarray:
    """delta [batch, B] float32 (-inf = decoded); token_sum, total_steps [batch] int
    -> K [batch] int32."""
    delta = np.asarray(delta)
    batch, block = delta.shape
    a = float(np.float32(alpha))
    out = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        steps = int(total_steps[b])
        nbar = int(token_sum[b]) / steps if steps > 0 else 1.0
        k_hist = math.ceil(a * nbar)
        out[b] = min(block, max(k_hist, _sigma_count(delta[b], mode)))
    return out


def history_update(decoded_prev, decoded_now, token_sum, total_steps):
    """Tokens decoded this step (positions decoded now but not before) added to
    token_sum; total_steps + 1. Returns the new (token_sum, total_steps)."""
    prev = np.asarray(decoded_prev).astype(bool)
    now = np.asarray(decoded_now).astype(bool)
    n_new = (now & ~prev).sum(axis=1)
    return (np.asarray(token_sum, np.int64) + n_new).astype(np.int32), \
        (np.asarray(total_steps, np.int64) + 1).astype(np.int32)
