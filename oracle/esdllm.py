"""ES-dLLM early-skip importance score, in float64 (oracle; test use only).

Definition followed (ES-dLLM notes page, key design 1): for layer l and
position i,

    I = alpha * c_i^(t-1) + (1 - alpha) * ||H^(t) - H^(t-1)||_1 / (sqrt(d) * ||H^(t-1)||_2)

where c^(t-1) is the previous iteration's maximum softmax probability at
that position and H are the layer's hidden states of this and the previous
iteration.

Readings: d is the hidden size of H. c is indexed by the absolute position
of the survivor. 0/0 (an unchanged all-zero row) is 0; x/0 with x > 0 is +inf.
"""
from __future__ import annotations

import numpy as np


def esdllm_score(h_new, h_prev, surv_pos, conf, alpha: float) -> np.ndarray:
    """h_new [batch, n_surv, h], h_prev [batch, L, h], surv_pos [batch, n_surv],
    conf [batch, L] -> score [batch, n_surv] float64."""
    h_new = np.asarray(h_new, dtype=np.float64)
    h_prev = np.asarray(h_prev, dtype=np.float64)
    conf = np.asarray(conf, dtype=np.float64)
    surv_pos = np.asarray(surv_pos)
    alpha = float(alpha)
    batch, n_surv, hidden = h_new.shape
    out = np.empty((batch, n_surv), dtype=np.float64)
    for b in range(batch):
        for s in range(n_surv):
            p = int(surv_pos[b, s])
            x, y = h_new[b, s], h_prev[b, p]
            l1 = np.sum(np.abs(x - y))
            l2 = np.sqrt(np.sum(y * y))
            if l1 == 0.0:
                v = 0.0
            elif l2 == 0.0:
                v = np.inf
            else:
                v = l1 / (np.sqrt(hidden) * l2)
            out[b, s] = alpha * conf[b, p] + (1.0 - alpha) * v
    return out


def esdllm_skip_layer(h_surv, h_cache, surv_pos, conf, alpha: float, keep: int, row_base=None):
    """One skip layer of ES-dLLM's early skipping (ES-dLLM notes page, key
    designs 1 and 2), composed of the oracle's own steps:

    1. score every survivor against the layer's cached previous-iteration
       hidden state (``esdllm_score``);
    2. update the layer's hidden-state cache in place at every survivor's
       position (partial cache update: skipped positions keep their state);
    3. keep the top ``keep`` survivors by score (``topk_select``; the pages'
       top-(1 - r_l)|S| with keep = floor((1 - r_l)|S|) passed in);
    4. the next layer's survivors and their hidden rows are the kept ones, in
       ascending survivor order.

    h_surv [batch, n_surv, h]; h_cache [batch, L, h] (viewed as rows); surv_pos
    [batch, n_surv]; conf [batch, L]. Returns (score, idx, count, cu, h_next
    [sum(count), h], surv_next [sum(count)], h_cache updated copy).
    """
    from .selection import topk_select
    from .rows import gather_rows, kv_scatter

    h_surv = np.asarray(h_surv)
    h_cache = np.asarray(h_cache)
    surv_pos = np.asarray(surv_pos)
    batch, n_surv = surv_pos.shape
    L = h_cache.shape[1]
    score = esdllm_score(h_surv, h_cache, surv_pos, conf, alpha)
    ident = np.tile(np.arange(n_surv, dtype=np.int32), (batch, 1))
    all_cnt = np.full(batch, n_surv, np.int32)
    all_cu = np.arange(batch + 1, dtype=np.int32) * n_surv
    rb = np.arange(batch, dtype=np.int64) * L if row_base is None else row_base
    rows = h_surv.reshape(batch * n_surv, -1)
    cache_rows = h_cache.reshape(batch * L, -1)
    new_cache, _ = kv_scatter(rows, rows, ident, all_cnt, all_cu, rb, cache_rows, cache_rows,
                              pos_map=surv_pos)
    idx, count, cu = topk_select(score, np.full(batch, keep, np.int32), keep)
    h_next = gather_rows(h_surv, idx, count, cu)
    surv_next = gather_rows(surv_pos[:, :, None], idx, count, cu)[:, 0]
    return score, idx, count, cu, h_next, surv_next, new_cache.reshape(h_cache.shape)
