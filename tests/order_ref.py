"""Reference of the reduced attention's work order (test helper).

A scheduling definition of the library, not part of the method (the pages
define no order), so it lives with the tests rather than in the oracle: the
GPU library starts the attention of the largest work items first (greedy
longest-processing-time scheduling), and this is the order it must produce,
by definition: sequence indices sorted by estimated work descending, equal
work by index ascending. Any order gives the same attention outputs.

Work of sequence i: its KV length (negative counts as 0); with the kept-row
counts given, the length times the number of 64-row query passes over its
keys, ceil(count_i * group / 64) (group = query heads per KV head; a negative
count counts as 0), capped at 2^32 - 1. A key-split attention wave holds 64
query rows, and past 64 rows per KV head the matrix-core work per key tile
doubles.
"""
from __future__ import annotations

import numpy as np

PASS_ROWS = 64
WORK_CAP = 2 ** 32 - 1


def attention_order(kv_len, count=None, group: int = 1) -> np.ndarray:
    lens = [max(int(v), 0) for v in np.asarray(kv_len).reshape(-1)]
    if count is None:
        work = lens
    else:
        cnt = [max(int(v), 0) for v in np.asarray(count).reshape(-1)]
        work = [min(lens[i] * -(-(cnt[i] * group) // PASS_ROWS), WORK_CAP)
                for i in range(len(lens))]
    return np.array(sorted(range(len(work)), key=lambda i: (-work[i], i)), dtype=np.int32)
