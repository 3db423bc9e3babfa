"""Reduced-query GQA attention over prefix + block KV, in float64 (oracle; test use only).

Followed: FOCUS paper Section 2 and Section 1 (Block-Diffusion: the block
attends bidirectionally, the preceding sequence is fixed context served from
an exact KV cache; Table 2 "KV Cache Attention"); Section 4.2 (later layers
run only on the kept rows, the evicted tokens serve as fixed reference KV);
App. E.2.4 (attention for non-contiguous, ragged kept queries). ES-dLLM
notes page, key design 2: survivors attend over the full cached KV.

Here, for kept row r of sequence b and query head h, with KV head
g = floor(h / G):
    s_j = scale * q[r, h] . K[seq_start[b] + j, g]   for j < kv_len[b]
    o[r, h] = sum_j softmax(s)_j * V[seq_start[b] + j, g]
No mask: every kept query sees the whole prefix and the whole block.
"""
from __future__ import annotations

import numpy as np


def reduced_attention(q, count, cu, cache_k, cache_v, seq_start, kv_len,
                      hq: int, hkv: int, scale: float, rows=None) -> np.ndarray:
    """q [sum(count), hq, D]; cache_k/v [rows, hkv, D] -> out [sum(count), hq, D] f64.

    `rows`: optional iterable of kept-row ids to compute (others left NaN),
    so that large workloads can be checked on a sample.
    """
    q = np.asarray(q, dtype=np.float64)
    G = hq // hkv
    total = q.shape[0]
    out = np.full(q.shape, np.nan, dtype=np.float64)
    want = None if rows is None else set(int(r) for r in rows)
    for b in range(len(count)):
        lo, n_b = int(cu[b]), int(count[b])
        sel = [r for r in range(lo, lo + n_b) if want is None or r in want]
        if not sel:
            continue
        s0, L = int(seq_start[b]), int(kv_len[b])
        Kb = np.asarray(cache_k[s0:s0 + L], dtype=np.float64)
        Vb = np.asarray(cache_v[s0:s0 + L], dtype=np.float64)
        for h in range(hq):
            g = h // G
            s = float(scale) * (q[sel, h, :] @ Kb[:, g, :].T)     # [len(sel), L]
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[sel, h, :] = p @ Vb[:, g, :]
    assert out.shape[0] == total
    return out
