"""Neighbour-aware delayed commit of block KV states (oracle; test use only).

Followed: FOCUS paper Section 4.3 (intra-block KV cache: a decoded token's KV
is committed only once it has stabilised, and, by the neighbour-aware
stability criterion, only when both the token and its right neighbour are
decoded); App. E.3.1 (positions are marked cached only when the token and its
right neighbour are unmasked; once the whole block is cached the block state
resets); App. E.3.3 (a token's KV goes to the global cache once its right
neighbour is decoded). FOCUS notes page, key design 4.

Readings: with `decoded` the state entering a step and `cached` the positions
already committed, the positions committed in this step are those not yet
cached whose token and right neighbour are both decoded; the last position of
the block, which has no right neighbour inside it, commits once every
position of the block is decoded. `cached` then includes them; `block_done`
is 1 when every position is cached (the caller resets the block state).
"""
from __future__ import annotations

import numpy as np


def commit_mask(decoded, cached):
    """decoded, cached [batch, B] bool -> (commit [batch, B] bool, cached' [batch, B] bool,
    block_done [batch] int32)."""
    dec = np.asarray(decoded).astype(bool)
    cac = np.asarray(cached).astype(bool)
    batch, B = dec.shape
    commit = np.zeros_like(dec)
    for b in range(batch):
        whole = bool(dec[b].all())
        for i in range(B):
            right = dec[b, i + 1] if i + 1 < B else whole
            commit[b, i] = (not cac[b, i]) and dec[b, i] and right
    new = cac | commit
    return commit, new, new.all(axis=1).astype(np.int32)
