"""Host-side contract checks of the binding (BTE_CHECK=1): valid inputs pass,
and each kind of device-data violation is caught before a launch. CPU only."""
import importlib.util
import os

import numpy as np
import pytest

_spec = importlib.util.spec_from_file_location(
    "bte_contract", os.path.join(os.path.dirname(__file__), "..", "block_token_eviction_amd",
                                 "contract.py"))
C = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(C)


def _rows(counts, n=32, k_max=12, seed=0):
    r = np.random.default_rng(seed)
    counts = np.asarray(counts, np.int32)
    idx = np.full((counts.size, k_max), -1, np.int32)
    for b, c in enumerate(counts):
        idx[b, :c] = np.sort(r.choice(n, size=c, replace=False))
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return idx, counts, cu


def test_enabled_reads_the_environment(monkeypatch):
    monkeypatch.delenv("BTE_CHECK", raising=False)
    assert not C.enabled()
    monkeypatch.setenv("BTE_CHECK", "1")
    assert C.enabled()


def test_rows_valid_and_each_violation():
    idx, cnt, cu = _rows([3, 0, 12, 5])
    C.check_rows(idx, cnt, cu, 12, n=32, out_rows=20)
    bad = cnt.copy(); bad[1] = 13
    with pytest.raises(C.ContractError, match="count"):
        C.check_rows(idx, bad, np.concatenate([[0], np.cumsum(bad)]), 12)
    with pytest.raises(C.ContractError, match="prefix"):
        C.check_rows(idx, cnt, cu + np.array([0, 0, 1, 1, 1]), 12)
    dup = idx.copy(); dup[0, 1] = dup[0, 0]
    with pytest.raises(C.ContractError, match="ascending"):
        C.check_rows(dup, cnt, cu, 12)
    high = idx.copy(); high[2, 11] = 32
    with pytest.raises(C.ContractError, match="outside"):
        C.check_rows(high, cnt, cu, 12, n=32)
    neg = idx.copy(); neg[3, 0] = -1
    with pytest.raises(C.ContractError, match="outside"):
        C.check_rows(neg, cnt, cu, 12, n=32)
    with pytest.raises(C.ContractError, match="fit"):
        C.check_rows(idx, cnt, cu, 12, out_rows=19)


def _explicit(rows, k_max=12):
    counts = np.array([len(r) for r in rows], np.int32)
    idx = np.full((len(rows), k_max), -1, np.int32)
    for b, r in enumerate(rows):
        idx[b, :len(r)] = r
    return idx, counts, np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def test_scatter_targets():
    idx, cnt, cu = _explicit([[1, 30], [0, 5, 31]])
    row_base = np.array([0, 40], np.int64)
    C.check_scatter(idx, cnt, cu, 12, row_base, cache_rows=80, new_rows=5)
    with pytest.raises(C.ContractError, match="outside"):        # 60 + 31 >= 80
        C.check_scatter(idx, cnt, cu, 12, np.array([0, 60], np.int64), cache_rows=80, new_rows=5)
    with pytest.raises(C.ContractError, match="same cache row"):  # both sequences write row 30
        C.check_scatter(idx, cnt, cu, 12, np.array([0, 25], np.int64), cache_rows=80, new_rows=5)
    with pytest.raises(C.ContractError, match="exceed"):
        C.check_scatter(idx, cnt, cu, 12, row_base, cache_rows=80, new_rows=4)
    # through a position map: positions repeated within a sequence collide
    pm = np.tile(np.arange(32, dtype=np.int32), (2, 1))
    C.check_scatter(idx, cnt, cu, 12, row_base, 80, 5, pos_map=pm)
    pm[1, :] = 7
    with pytest.raises(C.ContractError, match="same cache row"):
        C.check_scatter(idx, cnt, cu, 12, row_base, 80, 5, pos_map=pm)


def test_scatter_paged_targets():
    idx, cnt, cu = _explicit([[2, 9], [1, 8, 15]])                # pages 0 and 1 of each
    bt = np.array([[3, 1, -1], [0, 2, -1]], np.int32)          # pages of 8 rows, pool of 4 pages
    pos_base = np.array([0, 0], np.int32)
    C.check_scatter_paged(idx, cnt, cu, 12, pos_base, bt, 8, pool_rows=32, new_rows=5)
    with pytest.raises(C.ContractError, match="page-table entry"):   # 8 + 8 -> column 2 holds -1
        C.check_scatter_paged(idx, cnt, cu, 12, np.array([0, 8], np.int32), bt, 8, 32, 5)
    with pytest.raises(C.ContractError, match="column"):             # column 3 does not exist
        C.check_scatter_paged(idx, cnt, cu, 12, np.array([0, 24], np.int32), bt, 8, 32, 5)
    with pytest.raises(C.ContractError, match="outside the pool"):   # page 3 of a 3-page pool
        C.check_scatter_paged(idx, cnt, cu, 12, pos_base, bt, 8, pool_rows=24, new_rows=5)


def test_fused_scatter_targets():
    idx, cnt, cu = _explicit([[1, 30], [0, 5, 31]])
    kv = np.array([40, 50], np.int32)
    ss = np.array([0, 40], np.int64)
    pb = np.array([8, 18], np.int32)                           # blocks end at 40 and 50
    C.check_fused_scatter(idx, cnt, cu, 12, 32, pb, kv, 5, seq_start=ss, cache_rows=90)
    with pytest.raises(C.ContractError, match="kv_len"):          # 10 + 30 >= 40
        C.check_fused_scatter(idx, cnt, cu, 12, 32, np.array([10, 18], np.int32), kv, 5,
                              seq_start=ss, cache_rows=90)
    with pytest.raises(C.ContractError, match=r"outside \[0, 31\)"):   # block index 31, n = 31
        C.check_fused_scatter(idx, cnt, cu, 12, 31, pb, kv, 5, seq_start=ss, cache_rows=90)
    # sequence 0's KV rows overlap sequence 1's: sequence 1 writes rows sequence 0 reads
    with pytest.raises(C.ContractError, match="reads a cache row"):
        C.check_fused_scatter(idx, cnt, cu, 12, 32, pb, kv, 5, seq_start=np.array([0, 5]),
                              cache_rows=90)
    # paged: sequence 1's block lands on a page that sequence 0 also maps
    bt = np.array([[0, 1, 2, 3, 4], [5, 6, 7, 8, 9], ], np.int32)
    C.check_fused_scatter(idx, cnt, cu, 12, 32, pb, kv, 5, cache_rows=100, block_table=bt,
                          page_size=10)
    shared = bt.copy()
    shared[1, 2] = 1                                           # positions 20..29 of seq 1 -> page 1
    with pytest.raises(C.ContractError, match="reads a cache row"):
        C.check_fused_scatter(idx, cnt, cu, 12, 32, pb, kv, 5, cache_rows=100,
                              block_table=shared, page_size=10)


def test_attention_contract():
    cnt = np.array([2, 0, 3], np.int32)
    cu = np.array([0, 2, 2, 5], np.int32)
    kv = np.array([10, 0, 7], np.int32)
    ss = np.array([0, 10, 10], np.int64)
    C.check_attention(cnt, cu, kv, 4, q_rows=5, seq_start=ss, cache_rows=17,
                      order=np.array([2, 0, 1]))
    with pytest.raises(C.ContractError, match="kv_len"):
        C.check_attention(cnt, cu, np.array([0, 0, 7]), 4, 5, seq_start=ss, cache_rows=17)
    with pytest.raises(C.ContractError, match="leave the cache"):
        C.check_attention(cnt, cu, kv, 4, 5, seq_start=ss, cache_rows=16)
    with pytest.raises(C.ContractError, match="query rows"):
        C.check_attention(cnt, cu, kv, 4, 4, seq_start=ss, cache_rows=17)
    with pytest.raises(C.ContractError, match="permutation"):
        C.check_attention(cnt, cu, kv, 4, 5, seq_start=ss, cache_rows=17, order=np.array([0, 0, 1]))
    bt = np.array([[0, 1], [-1, -1], [2, -1]], np.int32)
    C.check_attention(cnt, cu, kv, 4, 5, cache_rows=24, block_table=bt, page_size=8)
    with pytest.raises(C.ContractError, match="page-table entry"):
        C.check_attention(cnt, cu, kv, 4, 5, cache_rows=24,
                          block_table=np.array([[0, -1], [-1, -1], [2, -1]], np.int32), page_size=8)


def test_positions():
    C.check_positions(np.array([[0, 5, 767]]), 768, "surv_pos")
    with pytest.raises(C.ContractError, match="surv_pos"):
        C.check_positions(np.array([[0, 768]]), 768, "surv_pos")


def test_survivors():
    """Skip-layer survivor sets: positions in range and distinct per sequence (each
    survivor's new state is written to its own cache row); with count/cu the counts
    within cap, cu their prefix sum and the rows inside the input."""
    sp = np.array([[5, 6, 7], [0, 1, 9]], np.int32)
    C.check_survivors(sp, 10)
    with pytest.raises(C.ContractError, match="leave"):
        C.check_survivors(np.array([[5, 6, 10]], np.int32), 10)
    with pytest.raises(C.ContractError, match="repeat"):
        C.check_survivors(np.array([[5, 6, 5]], np.int32), 10)
    rows = np.array([3, 4, 8, 1, 2], np.int32)
    cnt, cu = np.array([3, 0, 2], np.int32), np.array([0, 3, 3, 5], np.int32)
    C.check_survivors(rows, 10, cnt, cu, cap=3, rows=5)
    with pytest.raises(C.ContractError, match="prefix"):
        C.check_survivors(rows, 10, cnt, np.array([0, 3, 4, 5], np.int32), cap=3, rows=5)
    with pytest.raises(C.ContractError, match="cap"):
        C.check_survivors(rows, 10, cnt, cu, cap=2, rows=5)
    with pytest.raises(C.ContractError, match="exceed"):
        C.check_survivors(rows, 10, cnt, cu, cap=3, rows=4)
    with pytest.raises(C.ContractError, match="repeat"):
        C.check_survivors(np.array([3, 4, 3, 1, 2], np.int32), 10, cnt, cu, cap=3, rows=5)


def test_ragged_source():
    idx, cnt, cu = _rows([2, 0, 3], n=4, k_max=4)
    src_cu = np.array([0, 4, 4], np.int32)
    C.check_ragged_source(src_cu, idx, cnt, 8)
    with pytest.raises(C.ContractError, match="source row"):
        C.check_ragged_source(src_cu, idx, cnt, 6)
