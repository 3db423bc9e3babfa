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


def esdllm_schedule(iter_, block_start, block_len: int, period: int, keep):
    """Iteration bookkeeping of ES-dLLM's skipping (ES-dLLM notes page, key
    design 2): generation starts with one full forward that initialises the
    caches, and after it a full refresh without skipping runs at a fixed
    period, so that skip errors do not pile up over the iterations.

    Reading taken: a sequence's iteration counter counts the iterations it
    has run; iteration 0 is the initial full pass, and with period > 0 every
    iteration whose count is a multiple of the period is a refresh (period 0:
    only the initial pass). A refresh skips nothing, so every skip layer keeps
    all of its survivors (keep = |S| = the block length); other iterations
    keep the given counts floor((1 - r_l) |S_l|). Every iteration starts from
    the whole current block: the first skip layer's survivors are positions
    block_start .. block_start + block_len - 1.

    Returns dict(surv_pos [batch, block_len], count [batch], cu [batch + 1],
    keep [n_layers, batch], refresh [batch] bool, iter [batch] advanced).
    """
    iter_ = np.asarray(iter_, dtype=np.int64)
    block_start = np.asarray(block_start, dtype=np.int64)
    batch = iter_.shape[0]
    refresh = np.array([it == 0 or (period > 0 and it % period == 0) for it in iter_], dtype=bool)
    surv = block_start[:, None] + np.arange(block_len)[None, :]
    keep_out = np.array([[block_len if refresh[b] else int(kl) for b in range(batch)]
                         for kl in keep], dtype=np.int64).reshape(len(keep), batch)
    return dict(surv_pos=surv, count=np.full(batch, block_len), cu=np.arange(batch + 1) * block_len,
                keep=keep_out, refresh=refresh, iter=iter_ + 1)


def esdllm_skip_layer_ragged(h_rows, h_cache, surv_rows, count, cu, conf, alpha: float, k,
                             cap: int):
    """One skip layer on survivor sets of different sizes per sequence (a
    sequence refreshing this iteration keeps every survivor while another
    skips half): the same steps as ``esdllm_skip_layer``.

    h_rows [rows, h]: the survivors' states of this iteration, sequence b's at
    rows cu[b] .. cu[b] + count[b] - 1; surv_rows [rows] their positions;
    h_cache [batch, L, h]; k [batch] the keep counts; cap: survivor slots per
    sequence. Returns (score [batch, cap] with -inf past count, idx, count',
    cu', h_next [sum(count'), h], surv_next [sum(count')], h_cache updated copy).
    """
    from .selection import topk_select
    from .rows import gather_rows_ragged

    h_rows = np.asarray(h_rows)
    h_cache = np.asarray(h_cache)
    surv_rows = np.asarray(surv_rows)
    batch = len(count)
    score = np.full((batch, cap), -np.inf)
    new_cache = h_cache.copy()
    for b in range(batch):
        lo, n = int(cu[b]), int(count[b])
        if n == 0:
            continue
        score[b, :n] = esdllm_score(h_rows[lo:lo + n][None], h_cache[b][None],
                                    surv_rows[lo:lo + n][None], np.asarray(conf)[b][None], alpha)[0]
        for s in range(n):
            new_cache[b, int(surv_rows[lo + s])] = h_rows[lo + s]
    idx, count2, cu2 = topk_select(score, np.asarray(k), cap)
    h_next = gather_rows_ragged(h_rows, cu, idx, count2, cu2)
    surv_next = gather_rows_ragged(surv_rows[:, None], cu, idx, count2, cu2)[:, 0]
    return score, idx, count2, cu2, h_next, surv_next, new_cache


def esdllm_iteration(iter_, block_start, block_len: int, period: int, keep, layer_states,
                     h_caches, conf, alpha: float):
    """One iteration of the skip pipeline: the bookkeeping, then each skip
    layer in turn on the survivors the previous one kept. layer_states(l,
    surv_rows, count, cu) stands for the model's layer output for the
    survivors (compacted rows). Returns (schedule dict, per-layer results of
    ``esdllm_skip_layer_ragged``)."""
    sch = esdllm_schedule(iter_, block_start, block_len, period, keep)
    rows, cnt, cu = sch["surv_pos"].reshape(-1), sch["count"], sch["cu"]
    out = []
    for l in range(len(keep)):
        h = layer_states(l, rows, cnt, cu)
        res = esdllm_skip_layer_ragged(h, h_caches[l], rows, cnt, cu, conf, alpha, sch["keep"][l],
                                       block_len)
        out.append(res)
        rows, cnt, cu = res[5], res[2], res[3]
    return sch, out
