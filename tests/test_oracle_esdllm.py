"""Pins of the ES-dLLM score oracle (CPU only): closed forms, special cases,
scale invariance and a library cross-check (ES-dLLM notes page, key design 1)."""
import math

import numpy as np
import pytest

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
