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
