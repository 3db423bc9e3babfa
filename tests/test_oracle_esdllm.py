"""Pins of the ES-dLLM score oracle (CPU only): closed forms, special cases,
scale invariance and a library cross-check (ES-dLLM notes page, key design 1);
the skip layers, their ragged form and the iteration bookkeeping (key design 2)
against a hand-worked schedule, the uniform layer and torch's index_select."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle


def _case(seed, batch=2, n_surv=5, L=9, h=64):
    r = np.random.default_rng(seed)
    h_prev = r.standard_normal((batch, L, h))
    surv = np.stack([r.choice(L, n_surv, replace=False) for _ in range(batch)])
    h_new = np.stack([h_prev[b, surv[b]] for b in range(batch)]) + r.standard_normal((batch, n_surv, h))
    conf = r.uniform(size=(batch, L))
    return h_new, h_prev, surv, conf


def test_exact_copy_gives_alpha_times_conf():
    h_new, h_prev, surv, conf = _case(0)
    h_new = np.stack([h_prev[b, surv[b]] for b in range(2)])
    out = oracle.esdllm_score(h_new, h_prev, surv, conf, 0.5)
    np.testing.assert_array_equal(out, 0.5 * np.take_along_axis(conf, surv, 1))


def test_one_element_closed_form():
    """H_prev = ones(4096); H_new = ones with one element +0.5: l1 = 0.5, sqrt(h)*l2 = 64*64."""
    h = 4096
    h_prev = np.ones((1, 1, h)); h_new = np.ones((1, 1, h)); h_new[0, 0, 17] += 0.5
    out = oracle.esdllm_score(h_new, h_prev, np.zeros((1, 1), int), np.zeros((1, 1)), 0.0)
    assert out[0, 0] == 2.0 ** -13


def test_scale_invariance_exact():
    h_new, h_prev, surv, conf = _case(1)
    a = oracle.esdllm_score(h_new, h_prev, surv, conf, 0.3)
    b = oracle.esdllm_score(2 * h_new, 2 * h_prev, surv, conf, 0.3)
    np.testing.assert_array_equal(a, b)


def test_alpha_limits_and_library_norms():
    h_new, h_prev, surv, conf = _case(2)
    c = np.take_along_axis(conf, surv, 1)
    np.testing.assert_array_equal(oracle.esdllm_score(h_new, h_prev, surv, conf, 1.0), c)
    v = oracle.esdllm_score(h_new, h_prev, surv, conf, 0.0)
    for b in range(2):
        for s in range(surv.shape[1]):
            y = h_prev[b, surv[b, s]]
            want = np.linalg.norm(h_new[b, s] - y, 1) / (math.sqrt(64) * np.linalg.norm(y, 2))
            assert v[b, s] == pytest.approx(want, rel=1e-13)
    mix = oracle.esdllm_score(h_new, h_prev, surv, conf, 0.25)
    np.testing.assert_allclose(mix, 0.25 * c + 0.75 * v, rtol=1e-13)


def test_zero_norm_cases():
    h_prev = np.zeros((1, 2, 8)); h_new = np.zeros((1, 2, 8)); h_new[0, 1, 3] = 1.0
    out = oracle.esdllm_score(h_new, h_prev, np.array([[0, 1]]), np.array([[0.2, 0.4]]), 0.5)
    assert out[0, 0] == 0.1          # 0/0 -> 0
    assert out[0, 1] == math.inf     # x/0 -> inf


def test_skip_layer_survivor_invariants():
    """Two skip layers (r = 0.5 each, as the pages' defaults at 1/8 and 1/4
    depth): S' is a subset of S of size floor(|S| / 2) holding the top
    scores; kept rows are the survivors' rows; the hidden cache changes only
    at survivor positions, to the survivors' new states."""
    r = np.random.default_rng(21)
    batch, prompt, gen, h = 3, 10, 24, 16
    L = prompt + gen
    surv = np.tile(np.arange(prompt, L, dtype=np.int32), (batch, 1))
    conf = r.random((batch, L))
    for layer in range(2):
        cache = r.standard_normal((batch, L, h))
        cur = cache + r.standard_normal((batch, L, h)) * (r.random((batch, L, 1)) < 0.3)
        h_surv = np.stack([cur[b, surv[b]] for b in range(batch)])
        keep = surv.shape[1] // 2
        score, idx, cnt, cu, h_next, s_next, new_cache = oracle.esdllm_skip_layer(
            h_surv, cache, surv, conf, 0.5, keep)
        assert np.all(cnt == keep)
        s_next = s_next.reshape(batch, keep)
        for b in range(batch):
            assert set(s_next[b]) <= set(surv[b]) and np.all(np.diff(s_next[b]) > 0)
            kept_scores = score[b, idx[b]]
            dropped = np.delete(score[b], idx[b])
            assert kept_scores.min() >= dropped.max()
            np.testing.assert_array_equal(h_next[b * keep:(b + 1) * keep], h_surv[b, idx[b]])
            changed = np.flatnonzero(np.any(new_cache[b] != cache[b], axis=1))
            assert set(changed) <= set(surv[b])
            np.testing.assert_array_equal(new_cache[b, surv[b]], h_surv[b])
            other = np.setdiff1d(np.arange(L), surv[b])
            np.testing.assert_array_equal(new_cache[b, other], cache[b, other])
        surv = s_next
    assert surv.shape[1] == gen // 4


GOLD_SCHED = os.path.join(os.path.dirname(__file__), "golden", "esdllm_schedule_example.json")


def test_schedule_hand_worked():
    g = json.load(open(GOLD_SCHED))
    B, keep = g["block_len"], g["keep"]
    one = g["single_sequence"]
    it = np.zeros(1, np.int64)
    rows_last = 0
    for i in range(one["iterations"]):
        s = oracle.esdllm_schedule(it, np.array([100]), B, one["period"], keep)
        assert bool(s["refresh"][0]) == one["refresh"][i]
        assert s["keep"][0, 0] == one["keep_layer0"][i] and s["keep"][1, 0] == one["keep_layer1"][i]
        rows_last += int(s["keep"][1, 0])
        it = s["iter"]
    assert rows_last == one["rows_after_last_skip_total"] and it[0] == one["iterations"]

    bt = g["batch"]
    s = oracle.esdllm_schedule(np.array(bt["iter"]), np.array(bt["block_start"]), B, bt["period"],
                               keep)
    np.testing.assert_array_equal(s["refresh"], bt["refresh"])
    np.testing.assert_array_equal(s["keep"], bt["keep"])
    np.testing.assert_array_equal(s["iter"], bt["iter_next"])
    n = len(bt["iter"])
    np.testing.assert_array_equal(s["count"], np.full(n, B))
    np.testing.assert_array_equal(s["cu"], np.arange(n + 1) * B)
    for b in range(n):                      # every iteration starts from the whole block
        np.testing.assert_array_equal(s["surv_pos"][b], bt["block_start"][b] + np.arange(B))
    for key, period in (("period_zero", 0), ("period_one", 1)):
        c = g[key]
        s = oracle.esdllm_schedule(np.array(c["iter"]), np.zeros(len(c["iter"])), B, period, keep)
        np.testing.assert_array_equal(s["refresh"], c["refresh"])


def _ragged_case(r, counts, L=40, h=32):
    batch = len(counts)
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    cache = r.standard_normal((batch, L, h))
    surv = np.concatenate([np.sort(r.choice(L, size=c, replace=False)) for c in counts]).astype(np.int64)
    h_rows = np.concatenate([cache[b, surv[cu[b]:cu[b + 1]]] for b in range(batch)]) if cu[-1] else \
        np.zeros((0, h))
    h_rows = h_rows + r.standard_normal(h_rows.shape) * (r.random((h_rows.shape[0], 1)) < 0.4)
    return cache, surv, np.array(counts), cu, h_rows, r.random((batch, L))


def test_gather_rows_ragged_matches_index_select():
    r = np.random.default_rng(31)
    counts = np.array([3, 0, 5, 2])
    src_cu = np.concatenate([[0], np.cumsum(counts)])
    src = r.standard_normal((int(src_cu[-1]), 6)).astype(np.float32)
    keep = np.array([2, 0, 3, 1])
    idx = np.full((4, 5), -1, np.int32)
    for b in range(4):
        idx[b, :keep[b]] = np.sort(r.choice(counts[b], size=keep[b], replace=False))
    cu = np.concatenate([[0], np.cumsum(keep)])
    got = oracle.gather_rows_ragged(src, src_cu, idx, keep, cu)
    flat = np.concatenate([src_cu[b] + idx[b, :keep[b]] for b in range(4)])
    ref = torch.from_numpy(src).index_select(0, torch.from_numpy(flat.astype(np.int64))).numpy()
    np.testing.assert_array_equal(got, ref)


def test_skip_layer_ragged_reduces_to_uniform():
    """Full counts and one keep for every sequence: the ragged layer is the uniform one."""
    r = np.random.default_rng(32)
    counts = [8, 8, 8]
    cache, surv, cnt, cu, h_rows, conf = _ragged_case(r, counts)
    got = oracle.esdllm_skip_layer_ragged(h_rows, cache, surv, cnt, cu, conf, 0.5,
                                          np.full(3, 4), 8)
    ref = oracle.esdllm_skip_layer(h_rows.reshape(3, 8, -1), cache, surv.reshape(3, 8), conf, 0.5,
                                   4)
    np.testing.assert_array_equal(got[1][:, :4], ref[1])          # k_max 8 here, 4 there
    assert np.all(got[1][:, 4:] == -1)
    for i in (0, 2, 3, 4, 5, 6):
        np.testing.assert_array_equal(np.asarray(got[i]).reshape(-1), np.asarray(ref[i]).reshape(-1))


def test_skip_layer_ragged_is_per_sequence():
    """Each sequence of a ragged batch gives what the uniform layer gives on it alone."""
    r = np.random.default_rng(33)
    counts, keep, cap = [6, 0, 9, 3], np.array([3, 2, 9, 0]), 9
    cache, surv, cnt, cu, h_rows, conf = _ragged_case(r, counts)
    score, idx, cnt2, cu2, h_next, s_next, new_cache = oracle.esdllm_skip_layer_ragged(
        h_rows, cache, surv, cnt, cu, conf, 0.5, keep, cap)
    assert np.all(np.isneginf(score[1])) and np.isneginf(score[0, 6:]).all()
    for b in range(4):
        n = counts[b]
        if n == 0:
            assert cnt2[b] == 0
            np.testing.assert_array_equal(new_cache[b], cache[b])
            continue
        ref = oracle.esdllm_skip_layer(h_rows[cu[b]:cu[b + 1]][None], cache[b][None],
                                       surv[cu[b]:cu[b + 1]][None], conf[b][None], 0.5,
                                       min(int(keep[b]), n))
        np.testing.assert_array_equal(score[b, :n], ref[0][0])
        assert cnt2[b] == min(int(keep[b]), n)
        np.testing.assert_array_equal(idx[b, :cnt2[b]], ref[1][0, :cnt2[b]])
        np.testing.assert_array_equal(h_next[cu2[b]:cu2[b + 1]], ref[4])
        np.testing.assert_array_equal(s_next[cu2[b]:cu2[b + 1]], ref[5])
        np.testing.assert_array_equal(new_cache[b], ref[6][0])


def test_skip_layer_ragged_refresh_keeps_everyone():
    """keep = |S| (a refresh iteration): every survivor goes on in order, and every
    survivor's cache row takes its new state."""
    r = np.random.default_rng(34)
    counts = [5, 7, 1]
    cache, surv, cnt, cu, h_rows, conf = _ragged_case(r, counts)
    score, idx, cnt2, cu2, h_next, s_next, new_cache = oracle.esdllm_skip_layer_ragged(
        h_rows, cache, surv, cnt, cu, conf, 0.5, cnt, 7)
    np.testing.assert_array_equal(cnt2, cnt)
    np.testing.assert_array_equal(h_next, h_rows)
    np.testing.assert_array_equal(s_next, surv)
    for b in range(3):
        np.testing.assert_array_equal(new_cache[b, surv[cu[b]:cu[b + 1]]], h_rows[cu[b]:cu[b + 1]])


def test_iteration_mixes_refresh_and_skip():
    """Sequences at iterations 0, 1 and 3 with period 3: the first and last refresh and keep
    the whole block through both skip layers, the middle one keeps a half, then a quarter."""
    r = np.random.default_rng(35)
    batch, L, h, blk = 3, 48, 16, 16
    start = np.array([32, 30, 0])
    caches = [r.standard_normal((batch, L, h)) for _ in range(2)]
    cur = [c + r.standard_normal(c.shape) * (r.random((batch, L, 1)) < 0.3) for c in caches]
    conf = r.random((batch, L))

    def states(l, rows, cnt, cu):
        b_of = np.repeat(np.arange(batch), cnt)
        return cur[l][b_of, rows]

    sch, res = oracle.esdllm_iteration(np.array([0, 1, 3]), start, blk, 3, [8, 4], states, caches,
                                       conf, 0.5)
    np.testing.assert_array_equal(sch["refresh"], [True, False, True])
    np.testing.assert_array_equal(res[0][2], [16, 8, 16])
    np.testing.assert_array_equal(res[1][2], [16, 4, 16])
    np.testing.assert_array_equal(res[1][5][:16], start[0] + np.arange(16))     # all kept, in order
    kept = res[1][5][16:20]
    assert set(kept) <= set(res[0][5][16:24]) <= set(start[1] + np.arange(16))
