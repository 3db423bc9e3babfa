"""Work order of the reduced attention (oracle; test use only).

Not part of the method's arithmetic: the GPU library starts the attention of
the longest sequences first (greedy longest-processing-time scheduling), and
this is the order it must produce, by definition: sequence indices sorted by
KV length descending, equal lengths by index ascending; negative lengths
count as 0.
"""
from __future__ import annotations

import numpy as np


def attention_order(kv_len) -> np.ndarray:
    lens = [max(int(v), 0) for v in np.asarray(kv_len).reshape(-1)]
    return np.array(sorted(range(len(lens)), key=lambda i: (-lens[i], i)), dtype=np.int32)
