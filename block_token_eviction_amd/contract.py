"""Host-side checks of the device-data contract of libbte (opt-in).

The C entry points validate their host arguments (pointers, sizes, dtypes)
but not the contents of device arrays: indices in range, ascending and
distinct kept positions, counts within k_max, prefix sums consistent with the
counts, cache ranges and page tables inside their buffers. A violation there
is an out-of-bounds access on the GPU. With ``BTE_CHECK=1`` in the
environment, the binding reads those small arrays back before each call and
raises ``ContractError`` instead of launching. It costs a device-to-host copy
and a synchronisation per call, so it is meant for debugging, not for timed
runs.

The functions take numpy arrays (or tensors, copied to the host) and only
compare integers: they compute nothing of the method.
"""
from __future__ import annotations

import os

import numpy as np


class ContractError(ValueError):
    pass


def enabled() -> bool:
    return os.environ.get("BTE_CHECK", "0") == "1"


def _np(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        return a.detach().cpu().numpy()
    return np.asarray(a)


def _fail(msg: str):
    raise ContractError(msg)


def check_rows(idx, count, cu, k_max: int, n: int | None = None, out_rows: int | None = None,
               in_rows: int | None = None):
    """Kept-row lists: 0 <= count[b] <= k_max; idx[b, :count[b]] strictly
    ascending and (if n is given) in [0, n); cu[0] = 0 and cu[b+1] - cu[b] =
    count[b]; the compacted rows cu[-1] fit in out_rows / in_rows."""
    idx, count, cu = _np(idx), _np(count).astype(np.int64), _np(cu).astype(np.int64)
    batch = count.shape[0]
    if cu.shape[0] != batch + 1:
        _fail(f"cu has {cu.shape[0]} entries, want batch + 1 = {batch + 1}")
    if (count < 0).any() or (count > k_max).any():
        b = int(np.flatnonzero((count < 0) | (count > k_max))[0])
        _fail(f"count[{b}] = {count[b]} outside [0, k_max = {k_max}]")
    if cu[0] != 0 or not np.array_equal(np.diff(cu), count):
        _fail("cu is not the exclusive prefix sum of count")
    for b in range(batch):
        row = idx[b, :count[b]].astype(np.int64)
        if row.size and (np.diff(row) <= 0).any():
            _fail(f"idx[{b}] is not strictly ascending: {row.tolist()}")
        if row.size and (row[0] < 0 or (n is not None and row[-1] >= n)):
            _fail(f"idx[{b}] has an entry outside [0, {n})")
    total = int(cu[-1])
    if out_rows is not None and total > out_rows:
        _fail(f"{total} compacted rows do not fit the output's {out_rows}")
    if in_rows is not None and total > in_rows:
        _fail(f"{total} compacted rows exceed the input's {in_rows}")


def _positions(idx, count, pos_map):
    """Per sequence, the kept positions (idx, or pos_map[b, idx])."""
    idx, count = _np(idx), _np(count)
    pm = _np(pos_map)
    out = []
    for b in range(count.shape[0]):
        p = idx[b, :int(count[b])].astype(np.int64)
        out.append(p if pm is None else pm[b, p].astype(np.int64))
    return out


def check_scatter(idx, count, cu, k_max: int, row_base, cache_rows: int, new_rows: int,
                  pos_map=None):
    """Contiguous scatter: row_base[b] + pos inside the cache and distinct over
    the whole call; the kept rows within the new K/V rows."""
    n = None if pos_map is None else _np(pos_map).shape[1]
    check_rows(idx, count, cu, k_max, n=n, in_rows=new_rows)
    rb = _np(row_base).astype(np.int64)
    targets = [rb[b] + p for b, p in enumerate(_positions(idx, count, pos_map))]
    t = np.concatenate(targets) if targets else np.zeros(0, np.int64)
    if t.size and (t.min() < 0 or t.max() >= cache_rows):
        _fail(f"a scatter target row is outside [0, {cache_rows})")
    if np.unique(t).size != t.size:
        _fail("two scattered rows target the same cache row")


def _page_rows(block_table, page_size: int, b: int, pos, pool_rows: int):
    bt = block_table
    page = pos // page_size
    if (pos < 0).any() or (page >= bt.shape[1]).any():
        _fail(f"sequence {b}: a position needs page-table column >= {bt.shape[1]}")
    ent = bt[b, page].astype(np.int64)
    if (ent < 0).any() or ((ent + 1) * page_size > pool_rows).any():
        _fail(f"sequence {b}: a page-table entry is outside the pool of {pool_rows // page_size} pages")
    return ent * page_size + pos % page_size


def check_scatter_paged(idx, count, cu, k_max: int, pos_base, block_table, page_size: int,
                        pool_rows: int, new_rows: int, pos_map=None):
    """Paged scatter: every target position maps through a valid page-table
    entry into the pool, and targets are distinct."""
    n = None if pos_map is None else _np(pos_map).shape[1]
    check_rows(idx, count, cu, k_max, n=n, in_rows=new_rows)
    pb, bt = _np(pos_base).astype(np.int64), _np(block_table)
    rows = [_page_rows(bt, page_size, b, pb[b] + p, pool_rows)
            for b, p in enumerate(_positions(idx, count, pos_map))]
    t = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    if np.unique(t).size != t.size:
        _fail("two scattered rows target the same pool row")


def check_attention(count, cu, kv_len, k_max: int, q_rows: int, seq_start=None,
                    cache_rows: int | None = None, block_table=None, page_size: int = 0,
                    order=None):
    """Reduced attention: counts and prefix sums as for the row lists, kept
    queries within q, kv_len >= 1 for every sequence with kept rows, each
    sequence's KV rows inside the cache (contiguous) or behind valid page-table
    entries (paged), and an order that is a permutation of the sequences."""
    count, cu, kv = _np(count).astype(np.int64), _np(cu).astype(np.int64), _np(kv_len).astype(np.int64)
    batch = count.shape[0]
    if (count < 0).any() or (count > k_max).any():
        _fail(f"a count is outside [0, k_max = {k_max}]")
    if cu.shape[0] != batch + 1 or cu[0] != 0 or not np.array_equal(np.diff(cu), count):
        _fail("cu is not the exclusive prefix sum of count")
    if int(cu[-1]) > q_rows:
        _fail(f"{int(cu[-1])} kept rows exceed the {q_rows} query rows")
    if ((count > 0) & (kv < 1)).any():
        _fail("a sequence with kept rows has kv_len < 1")
    if seq_start is not None:
        ss = _np(seq_start).astype(np.int64)
        live = count > 0
        if ((ss < 0) | (ss + kv > cache_rows))[live].any():
            _fail(f"a sequence's KV rows leave the cache of {cache_rows} rows")
    if block_table is not None:
        bt = _np(block_table)
        for b in np.flatnonzero(count > 0):
            _page_rows(bt, page_size, int(b), np.arange(int(kv[b]), dtype=np.int64), cache_rows)
    if order is not None:
        o = _np(order).astype(np.int64)
        if not np.array_equal(np.sort(o), np.arange(batch)):
            _fail("order is not a permutation of the sequences")


def check_positions(pos, limit: int, name: str):
    """Every entry of pos in [0, limit)."""
    p = _np(pos)
    if p.size and (p.min() < 0 or p.max() >= limit):
        _fail(f"{name} has an entry outside [0, {limit})")


def check_fused_scatter(idx, count, cu, k_max: int, n: int, pos_base, kv_len, new_rows: int,
                        seq_start=None, cache_rows: int | None = None, block_table=None,
                        page_size: int = 0):
    """Scatter fused into the attention: the kept rows' block indices in
    [0, n), each target position pos_base[b] + idx inside [0, kv_len[b]), and
    no written cache row inside another attending sequence's KV rows (that
    sequence would read it during the same launch). Cache rows are
    seq_start[b] + position (contiguous) or pool rows through block_table."""
    check_rows(idx, count, cu, k_max, n=n, in_rows=new_rows)
    pb, kv = _np(pos_base).astype(np.int64), _np(kv_len).astype(np.int64)
    cnt = _np(count).astype(np.int64)
    pos = _positions(idx, count, None)
    for b, p in enumerate(pos):
        q = pb[b] + p
        if q.size and (q.min() < 0 or q.max() >= kv[b]):
            _fail(f"sequence {b}: a scatter target position is outside [0, kv_len = {kv[b]})")
    if seq_start is not None:
        ss = _np(seq_start).astype(np.int64)
        rows = [ss[b] + pb[b] + p for b, p in enumerate(pos)]
        readers = [(ss[b], ss[b] + kv[b]) for b in range(cnt.shape[0])]
    elif block_table is not None:
        bt = _np(block_table)
        rows = [_page_rows(bt, page_size, b, pb[b] + p, cache_rows) for b, p in enumerate(pos)]
        readers = None
    else:
        return
    t = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    owner = np.concatenate([np.full(r.size, b, np.int64) for b, r in enumerate(rows)]) \
        if rows else np.zeros(0, np.int64)
    if np.unique(t).size != t.size:
        _fail("two scattered rows target the same cache row")
    if not t.size:
        return
    order = np.argsort(t)
    t, owner = t[order], owner[order]
    for b in np.flatnonzero(cnt > 0):
        if readers is not None:
            lo, hi = readers[b]
            sel = slice(np.searchsorted(t, lo), np.searchsorted(t, hi))
            hit = owner[sel]
        else:
            read = _page_rows(bt, page_size, int(b), np.arange(int(kv[b]), dtype=np.int64),
                              cache_rows)
            hit = owner[np.isin(t, read)]
        if (hit != b).any():
            _fail(f"sequence {int(b)} reads a cache row that sequence "
                  f"{int(hit[hit != b][0])} writes in the same launch")


def check_survivors(surv_pos, seq_len: int, count=None, cu=None, cap: int | None = None,
                    rows: int | None = None):
    """Skip-layer survivors: per sequence, positions in [0, seq_len) and
    distinct (each survivor's new state is written to its own cache row).
    With count/cu: 0 <= count[b] <= cap, cu the exclusive prefix sum of
    count, and the compacted rows cu[-1] within `rows`."""
    sp = _np(surv_pos)
    if count is None:
        lists = [sp[b] for b in range(sp.shape[0])]
    else:
        cnt, c = _np(count).astype(np.int64), _np(cu).astype(np.int64)
        if c.shape[0] != cnt.shape[0] + 1 or c[0] != 0 or not np.array_equal(np.diff(c), cnt):
            _fail("cu is not the exclusive prefix sum of count")
        if cap is not None and ((cnt < 0) | (cnt > cap)).any():
            _fail(f"a survivor count is outside [0, cap = {cap}]")
        if rows is not None and int(c[-1]) > rows:
            _fail(f"{int(c[-1])} survivor rows exceed the input's {rows}")
        lists = [sp[int(c[b]):int(c[b]) + int(cnt[b])] for b in range(cnt.shape[0])]
    for b, p in enumerate(lists):
        p = np.asarray(p, np.int64)
        if p.size and (p.min() < 0 or p.max() >= seq_len):
            _fail(f"survivor positions of sequence {b} leave [0, {seq_len})")
        if np.unique(p).size != p.size:
            _fail(f"survivor positions of sequence {b} repeat")


def check_ragged_source(src_cu, idx, count, src_rows: int):
    """Gather from compacted sources: every src_cu[b] + idx[b, t], t < count[b],
    inside [0, src_rows)."""
    sc, cnt = _np(src_cu).astype(np.int64), _np(count).astype(np.int64)
    pos = _positions(idx, count, None)
    for b, p in enumerate(pos):
        if p.size and (sc[b] + p.min() < 0 or sc[b] + p.max() >= src_rows):
            _fail(f"sequence {b} gathers a source row outside [0, {src_rows})")
