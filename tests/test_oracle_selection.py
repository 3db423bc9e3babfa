"""Pins of the top-K oracle (CPU only): exhaustive brute force on tiny inputs
against the dominance definition, a library sort, and invariants (FOCUS
paper Section 4.2: top-K masked tokens by Delta-I)."""
import itertools
import math

import numpy as np
import pytest

import oracle

VALUES = [-math.inf, math.nan, -1.0, -0.0, 0.0, 1.0]


def _beats(s, a, u):
    """a precedes u in the total order: larger score, or equal score and lower index."""
    return s[a] > s[u] or (s[a] == s[u] and a < u)


def _brute(s, k, k_max):
    n = len(s)
    elig = [j for j in range(n) if not math.isnan(s[j]) and s[j] > -math.inf]
    keff = min(max(k, 0), len(elig), k_max)
    found = []
    for sub in itertools.combinations(elig, keff):
        rest = [u for u in elig if u not in sub]
        if all(_beats(s, a, u) for a in sub for u in rest):
            found.append(list(sub))
    assert len(found) == 1          # the result is unique under the total order
    return found[0]


def test_exhaustive_small():
    for n in range(1, 5):
        rows = list(itertools.product(VALUES, repeat=n))
        scores = np.array(rows, dtype=np.float32)
        for k in range(0, n + 2):
            for k_max in (n, max(0, n - 1)):
                kk = np.full(len(rows), k, np.int32)
                idx, count, cu = oracle.topk_select(scores, kk, k_max)
                for r, row in enumerate(rows):
                    want = _brute(row, k, k_max)
                    assert count[r] == len(want)
                    assert idx[r, :count[r]].tolist() == want
                    assert (idx[r, count[r]:] == -1).all()
                np.testing.assert_array_equal(cu[1:], np.cumsum(count))
                assert cu[0] == 0


def test_matches_library_lexsort():
    r = np.random.default_rng(3)
    scores = r.integers(-3, 4, size=(200, 32)).astype(np.float32)   # many exact ties
    scores[r.uniform(size=scores.shape) < 0.3] = -np.inf
    k = r.integers(0, 15, size=200).astype(np.int32)
    idx, count, cu = oracle.topk_select(scores, k, 12)
    for b in range(200):
        elig = np.flatnonzero(np.isfinite(scores[b]))
        order = elig[np.lexsort((elig, -scores[b, elig]))]
        keff = min(k[b], elig.size, 12)
        assert count[b] == keff
        np.testing.assert_array_equal(idx[b, :keff], np.sort(order[:keff]))


def test_invariants_random():
    r = np.random.default_rng(4)
    scores = r.standard_normal((64, 256)).astype(np.float32)
    dec = r.uniform(size=scores.shape) < 0.5
    scores[dec] = -np.inf
    k = np.full(64, 128, np.int32)
    idx, count, cu = oracle.topk_select(scores, k, 128)
    for b in range(64):
        sel = idx[b, :count[b]]
        assert np.all(np.diff(sel) > 0)                       # ascending, distinct
        assert not dec[b, sel].any()                          # decoded never selected
        assert count[b] == min(128, (~dec[b]).sum())
        rest = np.setdiff1d(np.flatnonzero(~dec[b]), sel)
        if sel.size and rest.size:
            assert scores[b, sel].min() >= scores[b, rest].max()


def test_negative_zero_ties_go_to_lower_index():
    s = np.array([[0.0, -0.0, 0.0, -0.0]], np.float32)
    idx, count, _ = oracle.topk_select(s, np.array([2]), 4)
    assert idx[0, :2].tolist() == [0, 1]
    s = np.array([[-0.0, 0.0]], np.float32)
    idx, _, _ = oracle.topk_select(s, np.array([1]), 1)
    assert idx[0, 0] == 0


def test_exhaustive_n6_against_stable_sort():
    """Every row of {-inf, -1, -0.0, +0.0, 1}^6 and every K in [0, 7]: the kept
    set is the first K_eff eligible positions of a stable sort by descending
    score (numpy's stable argsort, ties in index order, -0.0 == +0.0),
    output ascending."""
    vals = [-math.inf, -1.0, -0.0, 0.0, 1.0]
    rows = np.array(list(itertools.product(vals, repeat=6)), dtype=np.float32)
    order = np.argsort(-rows, axis=1, kind="stable")
    elig = rows > -np.inf
    for k in range(0, 8):
        for k_max in (6, 4):
            idx, count, cu = oracle.topk_select(rows, np.full(len(rows), k, np.int32), k_max)
            for r in range(len(rows)):
                ranked = [j for j in order[r] if elig[r, j]]
                want = sorted(ranked[:min(k, len(ranked), k_max)])
                assert count[r] == len(want)
                assert idx[r, :count[r]].tolist() == want
                assert (idx[r, count[r]:] == -1).all()
            assert cu[0] == 0 and np.array_equal(np.diff(cu), count)
