"""FOCUS importance and importance delta, in float64 (oracle; test use only).

Definitions followed (FOCUS: DLLMs Know How to Tame Their Compute Bound,
arXiv 2601.23278):

* Section 3.1, Eq. 2: I_j = sum over query rows i and heads h of
  Softmax(MaxPool1D(S_ij^(h))), with S_ij^(h) = q_i^(h) . k_j^(h) / sqrt(d_k)
  the pre-softmax score of query i on key j in head h (the FOCUS notes page,
  key design 1, gives the same formula and names the pooling SnapKV-style).
* App. E.2.1: the sum runs over the B query rows of the current block and
  the H heads; the kernel there fuses the pooling into the reduction.
* Section 3.2, Eq. 3: Delta-I_j = I_j(layer 1) - I_j(layer 0).
* Section 4.2: only masked (not yet decoded) tokens are candidates.

Readings where the pages leave a step open:
* Pooling runs along the key axis j of each (head, query row), stride 1,
  window `pool_kernel` (odd), "same" output length; the window is cut at
  the block edges, which is what -inf padding gives.
* The softmax runs over the B keys of the block (the metric is block-internal).
* Grouped-query attention: query head h reads key head floor(h / G),
  G = hq / hkv; the sum over heads is over the hq query heads.
* d_k is the head dimension.
* Decoded positions take Delta-I = -inf after the subtraction, so that no
  selection can pick them; they still take part in every softmax.
"""
from __future__ import annotations

import numpy as np


def block_scores(q, k, hq: int, hkv: int) -> np.ndarray:
    """S[b, h, i, j] = q[b, i, h, :] . k[b, j, h // G, :] / sqrt(D).

    q: [batch, B, hq, D], k: [batch, B, hkv, D] (any float dtype, widened
    exactly to float64). Returns [batch, hq, B, B] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    batch, B, nq, D = q.shape
    assert nq == hq and k.shape == (batch, B, hkv, D) and hq % hkv == 0
    G = hq // hkv
    S = np.empty((batch, hq, B, B), dtype=np.float64)
    for h in range(hq):
        g = h // G
        S[:, h] = np.matmul(q[:, :, h, :], np.swapaxes(k[:, :, g, :], 1, 2))
    return S / np.sqrt(D)


def maxpool_keys(S: np.ndarray, pool_kernel: int) -> np.ndarray:
    """P[..., j] = max of S[..., j'] over j' in [j - r, j + r] within the block.

    r = (pool_kernel - 1) / 2; positions outside the block are absent.
    """
    assert pool_kernel >= 1 and pool_kernel % 2 == 1
    r = (pool_kernel - 1) // 2
    B = S.shape[-1]
    P = np.empty_like(S)
    for j in range(B):
        lo, hi = max(0, j - r), min(B, j + r + 1)
        P[..., j] = S[..., lo:hi].max(axis=-1)
    return P


def softmax_keys(P: np.ndarray) -> np.ndarray:
    """Row softmax over the last (key) axis."""
    m = P.max(axis=-1, keepdims=True)
    e = np.exp(P - m)
    return e / e.sum(axis=-1, keepdims=True)


def importance(q, k, hq: int, hkv: int, pool_kernel: int) -> np.ndarray:
    """I[b, j] = sum_h sum_i softmax_j(maxpool_j(S[b, h, i, :]))[j]. [batch, B]."""
    A = softmax_keys(maxpool_keys(block_scores(q, k, hq, hkv), pool_kernel))
    return A.sum(axis=(1, 2))


def focus_importance_delta(q0, k0, q1, k1, decoded, hq: int, hkv: int,
                           pool_kernel: int) -> np.ndarray:
    """Delta-I[b, j] = I1[b, j] - I0[b, j]; -inf where decoded[b, j] != 0."""
    d = importance(q1, k1, hq, hkv, pool_kernel) - importance(q0, k0, hq, hkv, pool_kernel)
    d[np.asarray(decoded) != 0] = -np.inf
    return d
