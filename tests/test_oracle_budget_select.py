"""Pins of the FOCUS budget and constrained selection oracles (CPU only).

The budget is pinned by the worked example of the FOCUS notes page
(tests/golden/focus_budget_example.json), the first-step rule (no history
means an average of 1, so alpha > 1 gives K >= 2; FOCUS paper Section 5.3 /
notes page key design 2), the cap at the block size, and a numpy cross-check
of the variance term. The selection is pinned by hand-worked sets and by the
defining properties of each constraint on random inputs."""
import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_budget_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "focus_budget_example.json")))
    delta = np.array(fx["delta"], np.float32)
    k = oracle.focus_budget(delta, fx["token_sum"], fx["total_steps"], fx["alpha"])
    np.testing.assert_array_equal(k, fx["budget"])
    for b in range(2):
        x = delta[b].astype(np.float64)
        assert int((x >= x.std()).sum()) == fx["n_sigma"][b]


def test_budget_first_step_and_cap():
    delta = np.full((3, 32), -np.inf, np.float32)          # nothing masked: N_sigma = 0
    k = oracle.focus_budget(delta, [0, 0, 40], [0, 0, 2], 1.5)
    assert list(k[:2]) == [2, 2]                          # N_bar = 1 before any history
    assert k[2] == 30                                     # ceil(1.5 * 20)
    k = oracle.focus_budget(delta[:1], [100], [1], 1.5)
    assert k[0] == 32                                     # capped at the block size
    k = oracle.focus_budget(delta[:1], [0], [5], 1.5)
    assert k[0] == 0                                      # nothing decoded yet, nothing masked


def test_budget_sigma_term_matches_numpy():
    r = np.random.default_rng(3)
    for trial in range(200):
        B = int(r.integers(1, 65))
        d = r.standard_normal(B).astype(np.float32)
        dec = r.random(B) < r.random()
        d[dec] = -np.inf
        m = d[np.isfinite(d)].astype(np.float64)
        want0 = int((m >= m.std()).sum()) if m.size else 0
        want1 = int((m > m.mean() + m.std()).sum()) if m.size else 0
        # no decoded history (token_sum 0 over one step): the budget is N_sigma
        k0 = oracle.focus_budget(d[None], [0], [1], 1.5, mode=0)[0]
        k1 = oracle.focus_budget(d[None], [0], [1], 1.5, mode=1)[0]
        assert k0 == want0 and k1 == want1, trial


def test_history_update():
    prev = np.array([[1, 0, 0, 1], [0, 0, 0, 0]], bool)
    now = np.array([[1, 1, 0, 1], [1, 1, 1, 0]], bool)
    ts, st = oracle.history_update(prev, now, [5, 0], [2, 0])
    assert list(ts) == [6, 3] and list(st) == [3, 1]


def _sel(delta, k, dec, rp):
    idx, cnt, cu, rpn = oracle.focus_select(np.array([delta], np.float32), [k],
                                            np.array([dec], bool), [rp])
    return sorted(idx[0, :cnt[0]].tolist()), int(rpn[0])


def test_select_hand_examples():
    ninf = -math.inf
    # B = 8, positions 1 and 3 decoded; top-2 candidates are 5 and 2.
    delta = [0.1, ninf, 0.7, ninf, -0.2, 0.9, 0.0, -0.5]
    dec = [0, 1, 0, 1, 0, 0, 0, 0]
    # candidates {2, 5}; predecessors {1, 4}; placeholders masked j in (-1, 5): {0, 2, 4}
    assert _sel(delta, 2, dec, -1) == ([0, 1, 2, 4, 5], 5)
    # positions up to 3 already processed: placeholders only {4}
    assert _sel(delta, 2, dec, 3) == ([1, 2, 4, 5], 5)
    # processed beyond every candidate: no placeholder, rightmost stays
    assert _sel(delta, 2, dec, 6) == ([1, 2, 4, 5], 6)
    # K = 0: no candidate; S falls back to the top-ranked position (5)
    assert _sel(delta, 0, dec, -1) == ([5], 5)
    # candidate at position 0 has no predecessor
    assert _sel([2.0, 0.0, 0.0], 1, [0, 0, 0], -1) == ([0], 0)
    # everything decoded: S = {0} (all -inf tie, lowest index)
    assert _sel([ninf] * 4, 3, [1] * 4, -1) == ([0], 0)


def test_select_properties_random():
    r = np.random.default_rng(4)
    for trial in range(300):
        B = int(r.integers(1, 65))
        dec = r.random(B) < r.random()
        d = r.standard_normal(B).astype(np.float32)
        d[r.random(B) < 0.1] = 0.0                        # ties
        d[dec] = -np.inf
        k = int(r.integers(0, B + 2))
        rp = int(r.integers(-1, B))
        idx, cnt, cu, rpn = oracle.focus_select(d[None], [k], dec[None], [rp])
        S = set(idx[0, :cnt[0]].tolist())
        assert np.all(idx[0, cnt[0]:] == -1) and np.all(np.diff(idx[0, :cnt[0]]) > 0)
        elig = np.flatnonzero(~dec)
        order = elig[np.lexsort((elig, -d[elig].astype(np.float64)))]
        cand = set(order[:min(k, elig.size)].tolist())
        assert cand <= S
        assert all(i - 1 in S for i in cand if i >= 1)
        if cand:
            m = max(cand)
            ph = {j for j in range(rp + 1, m) if not dec[j]}
            assert ph <= S
            assert S == cand | {i - 1 for i in cand if i >= 1} | ph
        else:
            assert len(S) == 1
        assert len(S) >= 1 and cnt[0] == len(S) and cu[1] == cnt[0]
        assert rpn[0] == max(rp, max(S))


def test_commit_mask_truth_table():
    """Every (decoded, cached) state of a 3-position block, against the rule
    written out position by position."""
    import itertools
    for bits in itertools.product([0, 1], repeat=6):
        dec = np.array([bits[:3]], bool)
        cac = np.array([bits[3:]], bool)
        commit, new, done = oracle.commit_mask(dec, cac)
        d, c = dec[0], cac[0]
        want = [not c[0] and d[0] and d[1],
                not c[1] and d[1] and d[2],
                not c[2] and d[2] and d[0] and d[1]]        # last: whole block decoded
        assert commit[0].tolist() == want, bits
        assert new[0].tolist() == [bool(x or y) for x, y in zip(c, want)]
        assert done[0] == int(all(new[0]))


def test_commit_mask_hand_example():
    # decoded 1 1 0 1 1 (right neighbours: 1 0 1 1 -, whole block not decoded)
    commit, new, done = oracle.commit_mask(np.array([[1, 1, 0, 1, 1]], bool),
                                           np.array([[0, 0, 0, 0, 0]], bool))
    assert commit[0].tolist() == [True, False, False, True, False] and done[0] == 0
    commit, new, done = oracle.commit_mask(np.array([[1, 1, 1, 1, 1]], bool), new)
    assert commit[0].tolist() == [False, True, True, False, True] and done[0] == 1


def test_gather_multi_matches_single():
    r = np.random.default_rng(12)
    idx, cnt, cu = oracle.topk_select(r.standard_normal((4, 9)), [3, 0, 9, 5], 9)
    srcs = [r.standard_normal((4, 9, 6)), r.integers(0, 100, (4, 9)).astype(np.int32),
            r.integers(0, 9, (4, 9, 2)).astype(np.int64)]
    outs = oracle.gather_rows_multi(srcs, idx, cnt, cu)
    for s, o in zip(srcs, outs):
        np.testing.assert_array_equal(o, np.concatenate([s[b, idx[b, :cnt[b]]] for b in range(4)]))
