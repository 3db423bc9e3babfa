"""Pins of the gather, scatter and attention oracles (CPU only): torch
index_select / index_copy_ and scaled_dot_product_attention as library
routines, closed forms and invariants."""
import numpy as np
import pytest
import torch

import oracle
import order_ref


def _sel(batch, n, k_max, seed):
    r = np.random.default_rng(seed)
    count = r.integers(0, k_max + 1, size=batch).astype(np.int32)
    idx = np.full((batch, k_max), -1, np.int32)
    for b in range(batch):
        idx[b, :count[b]] = np.sort(r.choice(n, count[b], replace=False))
    cu = np.zeros(batch + 1, np.int32); cu[1:] = np.cumsum(count)
    return idx, count, cu


@pytest.mark.parametrize("dtype", [np.float32, np.uint16, np.float64])
def test_gather_matches_index_select(dtype):
    batch, n, h = 5, 32, 24
    src = (np.random.default_rng(0).standard_normal((batch, n, h)) * 100).astype(dtype)
    idx, count, cu = _sel(batch, n, 12, 1)
    flat = np.concatenate([b * n + idx[b, :count[b]] for b in range(batch)]).astype(np.int64)
    want = torch.index_select(torch.from_numpy(src.reshape(batch * n, h)), 0, torch.from_numpy(flat))
    got = oracle.gather_rows(src, idx, count, cu)
    assert got.dtype == src.dtype
    np.testing.assert_array_equal(got, want.numpy())


@pytest.mark.parametrize("use_map", [False, True])
def test_scatter_matches_index_copy(use_map):
    batch, n, hkv, D = 4, 32, 2, 8
    r = np.random.default_rng(2)
    L = r.integers(40, 80, size=batch)
    seq_start = np.concatenate([[0], np.cumsum(L)[:-1]])
    rows = int(L.sum())
    cache_k = r.standard_normal((rows, hkv, D)).astype(np.float32)
    cache_v = r.standard_normal((rows, hkv, D)).astype(np.float32)
    idx, count, cu = _sel(batch, n, 10, 3)
    new_k = r.standard_normal((int(cu[-1]), hkv, D)).astype(np.float32)
    new_v = r.standard_normal((int(cu[-1]), hkv, D)).astype(np.float32)
    pos_map = np.stack([r.permutation(n) + 5 for _ in range(batch)]) if use_map else None
    row_base = seq_start + (L - n - 5 if use_map else L - n)
    ok, ov = oracle.kv_scatter(new_k, new_v, idx, count, cu, row_base, cache_k, cache_v, pos_map)
    dest = []
    for b in range(batch):
        for t in range(count[b]):
            j = idx[b, t]
            dest.append(row_base[b] + (pos_map[b, j] if use_map else j))
    dest = torch.tensor(dest, dtype=torch.int64)
    for new, cache, got in ((new_k, cache_k, ok), (new_v, cache_v, ov)):
        want = torch.from_numpy(cache.copy()).index_copy_(0, dest, torch.from_numpy(new))
        np.testing.assert_array_equal(got, want.numpy())
        untouched = np.setdiff1d(np.arange(rows), dest.numpy())
        np.testing.assert_array_equal(got[untouched], cache[untouched])   # bit-identical


def _attn_case(seed, batch=3, hq=8, hkv=2, D=16):
    r = np.random.default_rng(seed)
    L = r.integers(1, 70, size=batch).astype(np.int32)
    seq_start = np.concatenate([[0], np.cumsum(L)[:-1]]).astype(np.int64)
    rows = int(L.sum())
    count = r.integers(0, 6, size=batch).astype(np.int32)
    cu = np.zeros(batch + 1, np.int32); cu[1:] = np.cumsum(count)
    q = r.standard_normal((int(cu[-1]), hq, D))
    ck = r.standard_normal((rows, hkv, D)); cv = r.standard_normal((rows, hkv, D))
    return q, count, cu, ck, cv, seq_start, L


def test_attention_matches_torch_sdpa():
    hq, hkv, D = 8, 2, 16
    q, count, cu, ck, cv, ss, L = _attn_case(5, hq=hq, hkv=hkv, D=D)
    scale = 1.0 / np.sqrt(D)
    got = oracle.reduced_attention(q, count, cu, ck, cv, ss, L, hq, hkv, scale)
    for b in range(len(count)):
        if count[b] == 0:
            continue
        qq = torch.from_numpy(q[cu[b]:cu[b + 1]]).transpose(0, 1)            # [hq, n, D]
        kk = torch.from_numpy(ck[ss[b]:ss[b] + L[b]]).transpose(0, 1)
        vv = torch.from_numpy(cv[ss[b]:ss[b] + L[b]]).transpose(0, 1)
        kk = kk.repeat_interleave(hq // hkv, 0); vv = vv.repeat_interleave(hq // hkv, 0)
        want = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
        np.testing.assert_allclose(got[cu[b]:cu[b + 1]], want.transpose(0, 1).numpy(),
                                   rtol=1e-10, atol=1e-12)


def test_attention_closed_forms():
    hq, hkv, D = 4, 1, 8
    r = np.random.default_rng(6)
    q = r.standard_normal((3, hq, D))
    count = np.array([1, 1, 1], np.int32); cu = np.array([0, 1, 2, 3], np.int32)
    ck = r.standard_normal((1 + 5 + 4, hkv, D)); cv = r.standard_normal(ck.shape)
    ck[1:6] = ck[1]                                    # seq 1: five identical keys
    ck[6:10] = 0.0; ck[6 + 2] = 50.0 * q[2, 0] / np.linalg.norm(q[2, 0]) ** 2 * np.sqrt(D)
    ss = np.array([0, 1, 6], np.int64); L = np.array([1, 5, 4], np.int32)
    out = oracle.reduced_attention(q, count, cu, ck, cv, ss, L, hq, hkv, 1 / np.sqrt(D))
    np.testing.assert_array_equal(out[0], np.broadcast_to(cv[0, 0], (hq, D)))   # kv_len 1 -> V0
    np.testing.assert_allclose(out[1], np.broadcast_to(cv[1:6, 0].mean(0), (hq, D)), rtol=1e-12)
    np.testing.assert_allclose(out[2, 0], cv[8, 0], atol=1e-15)               # logit 50 dominates


def test_attention_key_permutation_invariance():
    hq, hkv, D = 8, 2, 16
    q, count, cu, ck, cv, ss, L = _attn_case(7, hq=hq, hkv=hkv, D=D)
    base = oracle.reduced_attention(q, count, cu, ck, cv, ss, L, hq, hkv, 0.25)
    perm = np.arange(ck.shape[0])
    for b in range(len(L)):
        perm[ss[b]:ss[b] + L[b]] = ss[b] + np.random.default_rng(b).permutation(L[b])
    got = oracle.reduced_attention(q, count, cu, ck[perm], cv[perm], ss, L, hq, hkv, 0.25)
    np.testing.assert_allclose(got, base, rtol=1e-11, atol=1e-13)


def test_attention_order_brute_force():
    """The order is the unique permutation with non-increasing lengths whose
    equal-length runs are in ascending index order: found here by enumerating
    every permutation of small inputs (ties, zeros and a negative length)."""
    import itertools
    cases = [[3], [1, 1, 1], [2, 5, 5, 0], [-4, 0, 7, 7, 1], [9, 2, 9, 2, 9, 4]]
    for lens in cases:
        eff = [max(v, 0) for v in lens]
        valid = [p for p in itertools.permutations(range(len(lens)))
                 if all(eff[p[i]] > eff[p[i + 1]] or (eff[p[i]] == eff[p[i + 1]] and p[i] < p[i + 1])
                        for i in range(len(p) - 1))]
        assert len(valid) == 1
        np.testing.assert_array_equal(order_ref.attention_order(np.array(lens, np.int32)), valid[0])


def test_attention_order_invariants():
    lens = np.random.default_rng(8).integers(1, 50, 3000).astype(np.int32)
    o = order_ref.attention_order(lens)
    assert sorted(o.tolist()) == list(range(lens.size))
    d = lens[o]
    assert np.all(d[:-1] >= d[1:])
    tie = d[:-1] == d[1:]
    assert np.all(o[:-1][tie] < o[1:][tie])


def test_attention_order_by_work_hand_example():
    """Worked by hand, group 4 (64 query rows per pass): counts 17, 3, 20, 0, 16 give
    68, 12, 80, 0, 64 rows per KV head, so 2, 1, 2, 0, 1 passes; with lengths 100, 100,
    60, 50, 130 the work is 200, 100, 120, 0, 130."""
    got = order_ref.attention_order(np.array([100, 100, 60, 50, 130], np.int32),
                                 count=np.array([17, 3, 20, 0, 16], np.int32), group=4)
    np.testing.assert_array_equal(got, [0, 4, 2, 1, 3])


def test_attention_order_by_work_special_cases():
    r = np.random.default_rng(12)
    lens = r.integers(-2, 400, 500).astype(np.int32)
    # one pass for every sequence that keeps rows: the length order, empty sequences last
    cnt = r.integers(1, 17, 500).astype(np.int32)
    np.testing.assert_array_equal(order_ref.attention_order(lens, count=cnt, group=4),
                                  order_ref.attention_order(lens))
    lens = np.maximum(lens, 1)             # zero work only from the counts below
    cnt[::7] = 0
    o = order_ref.attention_order(lens, count=cnt, group=4)
    tail = o[-int((cnt == 0).sum()):]
    assert set(tail.tolist()) == set(np.flatnonzero(cnt == 0).tolist())
    assert np.all(np.diff(tail) > 0)
    # work saturates at 2^32 - 1: the two largest tie and keep index order
    big = order_ref.attention_order(np.array([2 ** 30, 2 ** 30 - 5, 7], np.int32),
                                 count=np.array([64 * 8, 64 * 9, 1], np.int32), group=1)
    np.testing.assert_array_equal(big, [0, 1, 2])


def _paged_layout(r, kv_len, page_size, extra_pages=3):
    """A random page table over a pool with spare pages, and the pool filled so
    that every sequence reads the contiguous rows it stands for."""
    need = [(int(L) + page_size - 1) // page_size for L in kv_len]
    max_pages = max(need)
    n_pages = sum(need) + extra_pages
    perm = r.permutation(n_pages)
    bt = np.full((len(kv_len), max_pages), -1, np.int32)
    at = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[at:at + n]
        at += n
    return bt, n_pages


def test_paged_attention_equals_contiguous():
    """Through a shuffled page table, paged attention is the contiguous one
    bit for bit (same rows, same order, same float64 steps)."""
    hq, hkv, D = 8, 2, 16
    q, count, cu, ck, cv, ss, L = _attn_case(9, hq=hq, hkv=hkv, D=D)
    r = np.random.default_rng(10)
    for P in (1, 2, 4, 16):
        bt, n_pages = _paged_layout(r, L, P)
        pk = r.standard_normal((n_pages * P, hkv, D))      # garbage in unused rows
        pv = r.standard_normal((n_pages * P, hkv, D))
        for b in range(len(L)):
            for p in range(int(L[b])):
                row = oracle.physical_row(bt, b, p, P)
                pk[row], pv[row] = ck[ss[b] + p], cv[ss[b] + p]
        want = oracle.reduced_attention(q, count, cu, ck, cv, ss, L, hq, hkv, 0.25)
        got = oracle.reduced_attention_paged(q, count, cu, pk, pv, bt, P, L, hq, hkv, 0.25)
        np.testing.assert_array_equal(got, want)


def test_paged_scatter_hand_example():
    # page size 2, sequence 0 owns pages [3, 0], sequence 1 owns page [1]; pool of 4 pages
    bt = np.array([[3, 0], [1, -1]], np.int32)
    cache = np.arange(8 * 2, dtype=np.int32).reshape(8, 2)
    new = np.array([[100, 101], [102, 103], [104, 105]], np.int32)
    idx = np.array([[0, 2], [1, -1]], np.int32)
    count = np.array([2, 1], np.int32)
    cu = np.array([0, 2, 3], np.int32)
    pos_base = np.array([1, 0], np.int32)
    # seq 0: logical 1 -> page 3 row 1 = 7; logical 3 -> page 0 row 1 = 1
    # seq 1: logical 1 -> page 1 row 1 = 3
    k2, _ = oracle.kv_scatter_paged(new, new, idx, count, cu, pos_base, bt, 2, cache, cache)
    want = cache.copy()
    want[7], want[1], want[3] = new[0], new[1], new[2]
    np.testing.assert_array_equal(k2, want)


def test_zero_kept_rows():
    """A sequence that keeps nothing (every position decoded): the gather writes no rows
    and the scatter leaves the cache as it was, also when its new-row slice is empty."""
    src = np.arange(2 * 4 * 3, dtype=np.float32).reshape(2, 4, 3)
    idx = np.array([[-1, -1], [1, 3]], np.int32)
    count = np.array([0, 2], np.int32)
    cu = np.array([0, 0, 2], np.int32)
    got = oracle.gather_rows(src, idx, count, cu)
    np.testing.assert_array_equal(got, src[1, [1, 3]])
    one0 = np.array([0], np.int32)
    empty = oracle.gather_rows(src[:1], idx[:1], one0, np.array([0, 0], np.int32))
    assert empty.shape == (0, 3)
    cache = np.arange(6 * 3, dtype=np.float32).reshape(6, 3)
    ck, cv = oracle.kv_scatter(np.zeros((0, 3), np.float32), np.zeros((0, 3), np.float32),
                               idx[:1], one0, np.array([0, 0], np.int32), np.array([2]), cache,
                               cache)
    np.testing.assert_array_equal(ck, cache)
    np.testing.assert_array_equal(cv, cache)
