"""Shared comparison helpers for the GPU parity tests."""
import sys

import numpy as np
import torch

ABS_TOL, REL_TOL = 1e-3, 2e-2      # |gpu - ref| <= max(1e-3, 2e-2 |ref|) for float results


def say(msg: str):
    """Name the case before GPU work, so a crash log points at it."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(d: dict, device="cuda"):
    return {k: (v.to(device) if torch.is_tensor(v) else v) for k, v in d.items()}


def host(t) -> np.ndarray:
    return t.detach().to("cpu").numpy() if t.dtype != torch.bfloat16 else t.detach().to("cpu", torch.float32).numpy()


def assert_close(got, ref, name=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{name}: -inf positions differ"
    assert np.array_equal(np.isposinf(got), np.isposinf(ref)), f"{name}: +inf positions differ"
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(got[fin])), f"{name}: non-finite values where the oracle is finite"
    err = np.abs(got[fin] - ref[fin])
    tol = np.maximum(ABS_TOL, REL_TOL * np.abs(ref[fin]))
    bad = err > tol
    if bad.any():
        i = np.flatnonzero(bad)[0]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} out of tolerance; first: got "
                             f"{got[fin][i]!r} ref {ref[fin][i]!r} (max err {err.max():.3g})")


def selection_valid(g_idx, g_cnt, ref_delta, k, k_max, tol_abs=ABS_TOL, tol_rel=REL_TOL):
    """GPU selection from fp32 scores vs float64 reference scores: same count, only
    eligible positions, and every kept score >= every dropped eligible score up to
    the score tolerance. Returns the rows whose index sets differ from the
    reference's own top-K (near-ties)."""
    batch = ref_delta.shape[0]
    differ = []
    for b in range(batch):
        elig = np.flatnonzero(np.isfinite(ref_delta[b]))
        keff = min(max(int(k[b]), 0), elig.size, k_max)
        assert g_cnt[b] == keff, (b, g_cnt[b], keff)
        sel = g_idx[b, :keff]
        assert np.all(np.diff(sel) > 0) and np.all(g_idx[b, keff:] == -1)
        assert np.all(np.isfinite(ref_delta[b, sel])), "a decoded position was selected"
        rest = np.setdiff1d(elig, sel)
        if sel.size and rest.size:
            lo = ref_delta[b, sel].min()
            hi = ref_delta[b, rest].max()
            tol = max(tol_abs, tol_rel * max(abs(lo), abs(hi)))
            assert lo >= hi - 2 * tol, (b, lo, hi)
        order = elig[np.lexsort((elig, -ref_delta[b, elig]))]
        if not np.array_equal(np.sort(order[:keff]), sel):
            differ.append(b)
    return differ


def page_table(kv_len, page_size, seed, spare=5):
    """Shuffled pages: block_table [batch, max_pages] (-1 past a sequence's
    pages) and, for every pool row, the contiguous cache row it holds (-1 if
    none)."""
    r = np.random.default_rng(seed)
    kv_len = np.asarray(kv_len, np.int64)
    need = (kv_len + page_size - 1) // page_size
    n_pages = int(need.sum()) + spare
    perm = r.permutation(n_pages).astype(np.int32)
    bt = np.full((len(kv_len), int(need.max())), -1, np.int32)
    src = np.full(n_pages * page_size, -1, np.int64)
    seq_start = np.concatenate([[0], np.cumsum(kv_len)[:-1]])
    at = 0
    for b in range(len(kv_len)):
        pages = perm[at:at + need[b]]
        at += need[b]
        bt[b, :need[b]] = pages
        p = np.arange(kv_len[b])
        src[pages[p // page_size].astype(np.int64) * page_size + p % page_size] = seq_start[b] + p
    return bt, src, n_pages


def pool(cache, src, n_pages, page_size):
    pool = torch.randn((n_pages * page_size,) + tuple(cache.shape[1:]), device=cache.device).to(cache.dtype)
    have = torch.from_numpy(np.flatnonzero(src >= 0)).to(cache.device)
    pool[have] = cache[torch.from_numpy(src[src >= 0]).to(cache.device)]
    return pool
