"""Pins of the FOCUS importance-delta oracle (CPU only).

Each test checks the oracle against something other than itself: a
hand-worked example, a closed form, a library routine (torch max_pool1d,
scipy softmax) or an invariant that the definition implies (FOCUS paper,
Section 3.1 Eq. 2, Section 3.2 Eq. 3).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_example_b3():
    g = json.load(open(os.path.join(GOLD, "focus_hand_b3.json")))
    a = {k: np.array(g[k], dtype=np.float64) for k in ("q0", "k0", "q1", "k1")}
    i1 = oracle.importance(a["q1"], a["k1"], 1, 1, g["pool_kernel"])
    np.testing.assert_allclose(i1, g["importance_layer1"], atol=1e-12)
    d = oracle.focus_importance_delta(a["q0"], a["k0"], a["q1"], a["k1"],
                                      np.array(g["decoded"]), 1, 1, g["pool_kernel"])
    np.testing.assert_allclose(d, g["delta"], atol=1e-12)
    idx, count, _ = oracle.topk_select(d.astype(np.float32), np.array([1]), 1)
    assert count[0] == 1 and idx[0, 0] == g["top1_index"]


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "focus_spike.json")))["cases"])
def test_spike_closed_form(case):
    B, hq, D = 32, 4, 64
    s = math.log(2.0)
    p, kp = case["p"], case["pool_kernel"]
    q0 = np.zeros((1, B, hq, D))
    k0 = _rand((1, B, hq, D), 3)
    q1 = np.zeros((1, B, hq, D)); q1[..., 0] = 1.0
    k1 = np.zeros((1, B, hq, D)); k1[0, p, :, 0] = s * math.sqrt(D)
    d = oracle.focus_importance_delta(q0, k0, q1, k1, np.zeros((1, B)), hq, hq, kp)[0]
    r = (kp - 1) // 2
    inw = case["in_window"][0] / case["in_window"][1]
    out = case["outside"][0] / case["outside"][1]
    for j in range(B):
        want = inw if abs(j - p) <= r else out
        assert d[j] == pytest.approx(want, abs=1e-12)


@pytest.mark.parametrize("B,pool_kernel,p,es", [(32, 3, 5, 3.0), (32, 5, 31, 1.5), (32, 9, 1, 7.0),
                                                 (64, 7, 40, 2.0), (64, 1, 63, 3.0), (64, 9, 0, 1.5),
                                                 (48, 13, 33, 2.5), (33, 7, 32, 4.0)])
def test_spike_general(B, pool_kernel, p, es):
    """Same closed form for other windows, edge positions, spike heights e^s > 1 and
    block sizes up to 64 (the FOCUS paper runs blocks of 16, 32 and 64, Section 5.3)."""
    hq, hkv, D = 8, 2, 64
    s = math.log(es)
    q0 = np.zeros((1, B, hq, D))
    q1 = np.zeros((1, B, hq, D)); q1[..., 0] = 1.0
    k1 = np.zeros((1, B, hkv, D)); k1[0, p, :, 0] = s * math.sqrt(D)
    d = oracle.focus_importance_delta(q0, k1, q1, k1, np.zeros((1, B)), hq, hkv, pool_kernel)[0]
    r = (pool_kernel - 1) // 2
    nw = min(B - 1, p + r) - max(0, p - r) + 1
    Z = nw * es + B - nw
    for j in range(B):
        want = hq * (B * es / Z - 1) if abs(j - p) <= r else hq * (B / Z - 1)
        assert d[j] == pytest.approx(want, abs=1e-12)


@pytest.mark.parametrize("B", [32, 64])
@pytest.mark.parametrize("pool_kernel", [1, 3, 5, 7, 9])
def test_maxpool_matches_torch(pool_kernel, B):
    S = _rand((2, 3, 5, B), pool_kernel)
    ref = torch.nn.functional.max_pool1d(torch.from_numpy(S).reshape(-1, 1, B),
                                         pool_kernel, stride=1, padding=pool_kernel // 2)
    np.testing.assert_array_equal(oracle.maxpool_keys(S, pool_kernel),
                                  ref.reshape(S.shape).numpy())


def test_pool1_is_plain_softmax_column_sum():
    q, k = _rand((2, 16, 4, 32), 1), _rand((2, 16, 2, 32), 2)
    S = np.einsum("bihd,bjhd->bhij", q, np.repeat(k, 2, axis=2)) / math.sqrt(32)
    want = scipy.special.softmax(S, axis=-1).sum(axis=(1, 2))
    np.testing.assert_allclose(oracle.importance(q, k, 4, 2, 1), want, rtol=1e-12)


@pytest.mark.parametrize("B,pool_kernel", [(32, 63), (32, 65), (32, 101), (64, 127), (48, 95)])
def test_pool_whole_row_is_uniform(B, pool_kernel):
    """k >= 2B-1: every pooled entry is the row max, softmax uniform, I_j = Hq."""
    q, k = _rand((3, B, 8, 16), 4), _rand((3, B, 2, 16), 5)
    np.testing.assert_allclose(oracle.importance(q, k, 8, 2, pool_kernel), 8.0, rtol=1e-13)


def test_gqa_head_mapping():
    """Query head h reads KV head floor(h / G)."""
    B, hq, hkv, D = 4, 6, 3, 8
    q = np.zeros((1, B, hq, D)); q[..., 0] = 1.0
    k = np.zeros((1, B, hkv, D))
    for g in range(hkv):
        k[0, :, g, 0] = (g + 1) * math.sqrt(D)
    S = oracle.block_scores(q, k, hq, hkv)
    for h in range(hq):
        np.testing.assert_array_equal(S[0, h], h // (hq // hkv) + 1)


def test_block_scores_scale_and_orientation():
    """S[b,h,i,j] uses query i against key j (not transposed), divided by sqrt(D)."""
    B, D = 3, 4
    q = np.zeros((1, B, 1, D)); k = np.zeros((1, B, 1, D))
    q[0, 0, 0, 0] = 2.0                   # only query row 0 nonzero
    k[0, 2, 0, 0] = 3.0                   # only key 2 nonzero
    S = oracle.block_scores(q, k, 1, 1)[0, 0]
    want = np.zeros((B, B)); want[0, 2] = 6.0 / 2.0
    np.testing.assert_array_equal(S, want)


def test_invariants():
    B, hq, hkv = 32, 8, 2
    q0, k0 = _rand((4, B, hq, 64), 6), _rand((4, B, hkv, 64), 7)
    q1, k1 = _rand((4, B, hq, 64), 8), _rand((4, B, hkv, 64), 9)
    for kp in (1, 3, 7):
        A = oracle.softmax_keys(oracle.maxpool_keys(oracle.block_scores(q1, k1, hq, hkv), kp))
        np.testing.assert_allclose(A.sum(-1), 1.0, atol=1e-12)
        i1 = oracle.importance(q1, k1, hq, hkv, kp)
        assert (i1 >= 0).all()
        np.testing.assert_allclose(i1.sum(-1), B * hq, rtol=1e-12)
        d = oracle.focus_importance_delta(q0, k0, q1, k1, np.zeros((4, B)), hq, hkv, kp)
        np.testing.assert_allclose(d.sum(-1), 0.0, atol=1e-9)


def test_permutation_invariance():
    B, hq, hkv = 32, 8, 2
    q, k = _rand((2, B, hq, 32), 10), _rand((2, B, hkv, 32), 11)
    base = oracle.importance(q, k, hq, hkv, 7)
    rows = np.random.default_rng(0).permutation(B)
    np.testing.assert_allclose(oracle.importance(q[:, rows], k, hq, hkv, 7), base, rtol=1e-12)
    heads = np.concatenate([np.arange(4, 8), np.arange(0, 4)])       # swap the two groups
    np.testing.assert_allclose(oracle.importance(q[:, :, heads], k[:, :, ::-1], hq, hkv, 7),
                               base, rtol=1e-12)


def test_decoded_masked_and_identical_layers_zero():
    B, hq = 32, 4
    q, k = _rand((2, B, hq, 16), 12), _rand((2, B, hq, 16), 13)
    dec = (np.random.default_rng(1).uniform(size=(2, B)) < 0.4).astype(np.uint8)
    d = oracle.focus_importance_delta(q, k, q, k, dec, hq, hq, 7)
    assert np.all(np.isneginf(d[dec == 1]))
    assert np.all(d[dec == 0] == 0.0)
