"""Python binding of libbte, the MI355X (gfx950) block token-eviction library.

Argument marshalling only: every function checks tensor shapes, dtypes and
devices on the host, passes raw device pointers and the current HIP stream
to the C ABI declared in ``include/bte.h``, and raises on a nonzero status.
All arithmetic runs in the library's HIP kernels. There is no fallback: if
``libbte.so`` is missing or fails to load, importing this package raises.

Names follow the C ABI: ``focus_importance_delta``, ``esdllm_score``,
``topk_select``, ``gather_rows``, ``kv_scatter``, ``reduced_attention``.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

from . import contract

__all__ = ["lib", "LIB_PATH", "BteError", "status_string", "focus_importance_delta",
           "esdllm_score", "topk_select", "gather_rows", "kv_scatter", "reduced_attention",
           "attention_order", "reduced_attention_paged", "kv_scatter_paged", "focus_budget",
           "focus_history_update", "focus_select", "focus_commit_mask", "gather_rows_multi",
           "kv_scatter_attention", "kv_scatter_attention_paged", "BTE_F32", "BTE_BF16", "contract"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbte.so")
BTE_F32, BTE_BF16 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python block_token_eviction_amd/build.py` (hipcc, gfx950)")
lib = ctypes.CDLL(LIB_PATH)

_p, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIG = {
    "bte_status_string": ([_i], ctypes.c_char_p),
    "bte_version": ([], _i),
    "bte_focus_importance_delta": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p], _i),
    "bte_esdllm_score": ([_p, _p, _p, _p, _f, _p, _i, _i, _i, _i, _i, _p], _i),
    "bte_topk_select": ([_p, _p, _p, _p, _p, _i, _i, _i, _p], _i),
    "bte_gather_rows": ([_p, _p, _p, _p, _p, _i, _i, _i, _sz, _p], _i),
    "bte_kv_scatter": ([_p, _p, _p, _p, _p, _p, _i, _p, _p, _p, _i, _i, _sz, _p], _i),
    "bte_reduced_attention": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p], _i),
    "bte_attention_order": ([_p, _p, _i, _i, _p, _p], _i),
    "bte_reduced_attention_paged": ([_p, _p, _p, _p, _p, _p, _i, _i, _p, _p, _p, _i, _i, _i, _i, _i,
                                     _f, _i, _p], _i),
    "bte_kv_scatter_paged": ([_p, _p, _p, _p, _p, _p, _i, _p, _p, _i, _i, _p, _p, _i, _i, _sz, _p],
                             _i),
    "bte_focus_budget": ([_p, _p, _p, _f, _i, _p, _i, _i, _p], _i),
    "bte_focus_history_update": ([_p, _p, _p, _p, _i, _i, _p], _i),
    "bte_focus_select": ([_p, _p, _p, _p, _p, _p, _p, _i, _i, _p], _i),
    "bte_focus_commit_mask": ([_p, _p, _p, _p, _i, _i, _p], _i),
    "bte_gather_rows_multi": ([_p, _i, _p, _p, _p, _i, _i, _i, _p], _i),
    "bte_kv_scatter_attention": ([_p, _p, _p, _p, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i,
                                  _i, _i, _i, _f, _i, _p], _i),
    "bte_kv_scatter_attention_paged": ([_p, _p, _p, _p, _i, _p, _p, _p, _p, _p, _p, _i, _i, _p, _p,
                                        _p, _i, _i, _i, _i, _i, _f, _i, _p], _i),
}
for _name, (_args, _res) in _SIG.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class BteError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def status_string(status: int) -> str:
    return lib.bte_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise BteError(fn, status)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libbte works on device tensors only")
            if not t.is_contiguous():
                raise ValueError("libbte needs contiguous tensors")


def _dtype(t) -> int:
    if t.dtype == torch.bfloat16:
        return BTE_BF16
    if t.dtype == torch.float32:
        return BTE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _want(t, dtype, name):
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def focus_importance_delta(q0, k0, q1, k1, decoded, pool_kernel: int, out=None):
    """q* [batch, B, hq, D], k* [batch, B, hkv, D], decoded uint8 [batch, B] -> delta f32 [batch, B]."""
    _dev(q0, k0, q1, k1, decoded, out)
    batch, block, hq, d = q0.shape
    hkv = k0.shape[2]
    for t in (q1,):
        assert t.shape == q0.shape and t.dtype == q0.dtype
    for t in (k0, k1):
        assert t.shape == (batch, block, hkv, d) and t.dtype == q0.dtype
    _want(decoded, torch.uint8, "decoded")
    assert decoded.shape == (batch, block)
    if out is None:
        out = torch.empty((batch, block), dtype=torch.float32, device=q0.device)
    _want(out, torch.float32, "out")
    _check("bte_focus_importance_delta", lib.bte_focus_importance_delta(
        _ptr(q0), _ptr(k0), _ptr(q1), _ptr(k1), _ptr(decoded), _ptr(out), batch, block, hq, hkv,
        d, pool_kernel, _dtype(q0), _stream()))
    return out


def esdllm_score(h_new, h_prev, surv_pos, conf, alpha: float, out=None):
    """h_new [batch, n_surv, h], h_prev [batch, L, h], surv_pos int32, conf f32 [batch, L]."""
    _dev(h_new, h_prev, surv_pos, conf, out)
    batch, n_surv, hidden = h_new.shape
    seq_len = h_prev.shape[1]
    assert h_prev.shape == (batch, seq_len, hidden) and h_prev.dtype == h_new.dtype
    _want(surv_pos, torch.int32, "surv_pos")
    _want(conf, torch.float32, "conf")
    assert surv_pos.shape == (batch, n_surv) and conf.shape == (batch, seq_len)
    if out is None:
        out = torch.empty((batch, n_surv), dtype=torch.float32, device=h_new.device)
    if contract.enabled():
        contract.check_positions(surv_pos, h_prev.shape[1], "surv_pos")
    _check("bte_esdllm_score", lib.bte_esdllm_score(
        _ptr(h_new), _ptr(h_prev), _ptr(surv_pos), _ptr(conf), float(alpha), _ptr(out), batch,
        n_surv, seq_len, hidden, _dtype(h_new), _stream()))
    return out


def topk_select(scores, k, k_max: int, idx=None, count=None, cu=None):
    """scores f32 [batch, n], k int32 [batch] -> (idx [batch, k_max], count [batch], cu [batch+1])."""
    _dev(scores, k, idx, count, cu)
    _want(scores, torch.float32, "scores")
    _want(k, torch.int32, "k")
    batch, n = scores.shape
    dev = scores.device
    if idx is None:
        idx = torch.empty((batch, max(k_max, 0)), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((batch,), dtype=torch.int32, device=dev)
    if cu is None:
        cu = torch.empty((batch + 1,), dtype=torch.int32, device=dev)
    _check("bte_topk_select", lib.bte_topk_select(
        _ptr(scores), _ptr(k), _ptr(idx) if k_max > 0 else None, _ptr(count), _ptr(cu), batch, n,
        k_max, _stream()))
    return idx, count, cu


def gather_rows(src, idx, count, cu, out=None):
    """src [batch, n, ...] -> out [capacity, ...]; rows cu[b]+t for t < count[b] are written.

    Without `out`, the capacity is batch * k_max rows (the device-side total is
    not read back)."""
    _dev(src, idx, count, cu, out)
    batch, n = src.shape[:2]
    k_max = idx.shape[1]
    row_bytes = src[0, 0].numel() * src.element_size()
    if out is None:
        out = torch.empty((batch * k_max,) + tuple(src.shape[2:]), dtype=src.dtype, device=src.device)
    assert out.dtype == src.dtype and out[0].numel() * out.element_size() == row_bytes
    if contract.enabled():
        contract.check_rows(idx, count, cu, k_max, n=n, out_rows=out.shape[0])
    _check("bte_gather_rows", lib.bte_gather_rows(
        _ptr(src), _ptr(idx), _ptr(count), _ptr(cu), _ptr(out), batch, n, k_max, row_bytes,
        _stream()))
    return out


def kv_scatter(new_k, new_v, idx, count, cu, row_base, cache_k, cache_v, pos_map=None):
    """Write new_k/new_v rows cu[b]+t into cache rows row_base[b] + pos (in place)."""
    _dev(new_k, new_v, idx, count, cu, row_base, cache_k, cache_v, pos_map)
    _want(row_base, torch.int64, "row_base")
    batch, k_max = idx.shape
    row_bytes = cache_k[0].numel() * cache_k.element_size()
    assert new_k[0].numel() * new_k.element_size() == row_bytes
    n = 0 if pos_map is None else pos_map.shape[1]
    if contract.enabled():
        contract.check_scatter(idx, count, cu, k_max, row_base, cache_k.shape[0], new_k.shape[0],
                               pos_map)
    _check("bte_kv_scatter", lib.bte_kv_scatter(
        _ptr(new_k), _ptr(new_v), _ptr(idx), _ptr(count), _ptr(cu), _ptr(pos_map), n,
        _ptr(row_base), _ptr(cache_k), _ptr(cache_v), batch, k_max, row_bytes, _stream()))
    return cache_k, cache_v


def reduced_attention(q, count, cu, cache_k, cache_v, seq_start, kv_len, k_max: int,
                      scale: float | None = None, out=None, order=None):
    """q [capacity, hq, D], cache [rows, hkv, D] -> out [capacity, hq, D] (rows cu[b]+t written).

    `order` (int32 [batch], e.g. from attention_order) only schedules the work."""
    _dev(q, count, cu, cache_k, cache_v, seq_start, kv_len, out, order)
    _want(seq_start, torch.int64, "seq_start")
    _want(kv_len, torch.int32, "kv_len")
    hq, d = q.shape[1], q.shape[2]
    hkv = cache_k.shape[1]
    batch = count.shape[0]
    assert cache_v.shape == cache_k.shape and cache_k.dtype == q.dtype
    if order is not None:
        _want(order, torch.int32, "order")
        assert order.shape == (batch,)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if contract.enabled():
        contract.check_attention(count, cu, kv_len, k_max, min(q.shape[0], out.shape[0]),
                                 seq_start=seq_start, cache_rows=cache_k.shape[0], order=order)
    _check("bte_reduced_attention", lib.bte_reduced_attention(
        _ptr(q), _ptr(count), _ptr(cu), _ptr(cache_k), _ptr(cache_v), _ptr(seq_start),
        _ptr(kv_len), _ptr(order), _ptr(out), batch, k_max, hq, hkv, d, float(scale), _dtype(q),
        _stream()))
    return out


def kv_scatter_attention(q, count, cu, idx, n: int, pos_base, new_k, new_v, cache_k, cache_v,
                         seq_start, kv_len, k_max: int, scale: float | None = None, out=None,
                         order=None):
    """kv_scatter into rows seq_start[b] + pos_base[b] + idx, then reduced_attention, in one launch.

    idx int32 [batch, k_max] block indices in [0, n); pos_base int32 [batch]. The cache is
    updated in place and out [capacity, hq, D] (rows cu[b]+t) is the attention over it."""
    _dev(q, count, cu, idx, pos_base, new_k, new_v, cache_k, cache_v, seq_start, kv_len, out, order)
    _want(seq_start, torch.int64, "seq_start")
    _want(kv_len, torch.int32, "kv_len")
    _want(pos_base, torch.int32, "pos_base")
    _want(idx, torch.int32, "idx")
    hq, d = q.shape[1], q.shape[2]
    hkv = cache_k.shape[1]
    batch = count.shape[0]
    assert idx.shape == (batch, k_max) and pos_base.shape == (batch,)
    assert cache_v.shape == cache_k.shape and cache_k.dtype == q.dtype
    assert new_k.shape[1:] == cache_k.shape[1:] and new_v.shape == new_k.shape
    assert new_k.dtype == q.dtype and new_v.dtype == q.dtype
    if order is not None:
        _want(order, torch.int32, "order")
        assert order.shape == (batch,)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if contract.enabled():
        contract.check_attention(count, cu, kv_len, k_max, min(q.shape[0], out.shape[0]),
                                 seq_start=seq_start, cache_rows=cache_k.shape[0], order=order)
        contract.check_fused_scatter(idx, count, cu, k_max, n, pos_base, kv_len, new_k.shape[0],
                                     seq_start=seq_start, cache_rows=cache_k.shape[0])
    _check("bte_kv_scatter_attention", lib.bte_kv_scatter_attention(
        _ptr(q), _ptr(count), _ptr(cu), _ptr(idx), n, _ptr(pos_base), _ptr(new_k), _ptr(new_v),
        _ptr(cache_k), _ptr(cache_v), _ptr(seq_start), _ptr(kv_len), _ptr(order), _ptr(out), batch,
        k_max, hq, hkv, d, float(scale), _dtype(q), _stream()))
    return out


def attention_order(kv_len, out=None, count=None, group: int = 1):
    """kv_len int32 [batch] -> order int32 [batch]: sequences by work descending, index
    ascending. Work is the length, or with the kept counts (int32 [batch]) and group =
    hq / hkv the length times ceil(count * group / 64) query passes."""
    _dev(kv_len, out, count)
    _want(kv_len, torch.int32, "kv_len")
    batch = kv_len.shape[0]
    if count is not None:
        _want(count, torch.int32, "count")
        assert count.shape == (batch,)
    if out is None:
        out = torch.empty((batch,), dtype=torch.int32, device=kv_len.device)
    _want(out, torch.int32, "out")
    _check("bte_attention_order", lib.bte_attention_order(_ptr(kv_len), _ptr(count), int(group),
                                                          batch, _ptr(out), _stream()))
    return out


def focus_budget(delta, token_sum, total_steps, alpha: float, threshold_mode: int = 0, out=None):
    """delta f32 [batch, B], token_sum/total_steps int32 [batch] -> K int32 [batch]."""
    _dev(delta, token_sum, total_steps, out)
    _want(delta, torch.float32, "delta")
    _want(token_sum, torch.int32, "token_sum")
    _want(total_steps, torch.int32, "total_steps")
    batch, block = delta.shape
    assert token_sum.shape == (batch,) and total_steps.shape == (batch,)
    if out is None:
        out = torch.empty((batch,), dtype=torch.int32, device=delta.device)
    _want(out, torch.int32, "out")
    _check("bte_focus_budget", lib.bte_focus_budget(
        _ptr(delta), _ptr(token_sum), _ptr(total_steps), float(alpha), int(threshold_mode),
        _ptr(out), batch, block, _stream()))
    return out


def focus_history_update(decoded_prev, decoded_now, token_sum, total_steps):
    """In place: token_sum += newly decoded positions, total_steps += 1."""
    _dev(decoded_prev, decoded_now, token_sum, total_steps)
    _want(decoded_prev, torch.uint8, "decoded_prev")
    _want(decoded_now, torch.uint8, "decoded_now")
    _want(token_sum, torch.int32, "token_sum")
    _want(total_steps, torch.int32, "total_steps")
    batch, block = decoded_now.shape
    assert decoded_prev.shape == (batch, block)
    _check("bte_focus_history_update", lib.bte_focus_history_update(
        _ptr(decoded_prev), _ptr(decoded_now), _ptr(token_sum), _ptr(total_steps), batch, block,
        _stream()))
    return token_sum, total_steps


def focus_select(delta, k, decoded, rightmost_processed, idx=None, count=None, cu=None):
    """Top-K + AR-context + placeholder integrity + |S| >= 1.
    -> (idx int32 [batch, B], count [batch], cu [batch + 1]); rightmost_processed updated in place."""
    _dev(delta, k, decoded, rightmost_processed, idx, count, cu)
    _want(delta, torch.float32, "delta")
    _want(k, torch.int32, "k")
    _want(decoded, torch.uint8, "decoded")
    _want(rightmost_processed, torch.int32, "rightmost_processed")
    batch, block = delta.shape
    dev = delta.device
    if idx is None:
        idx = torch.empty((batch, block), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((batch,), dtype=torch.int32, device=dev)
    if cu is None:
        cu = torch.empty((batch + 1,), dtype=torch.int32, device=dev)
    _check("bte_focus_select", lib.bte_focus_select(
        _ptr(delta), _ptr(k), _ptr(decoded), _ptr(rightmost_processed), _ptr(idx), _ptr(count),
        _ptr(cu), batch, block, _stream()))
    return idx, count, cu


def reduced_attention_paged(q, count, cu, cache_k, cache_v, block_table, page_size: int, kv_len,
                            k_max: int, scale: float | None = None, out=None, order=None):
    """q [capacity, hq, D]; page pool cache [n_pages * page_size, hkv, D];
    block_table int32 [batch, max_pages] -> out [capacity, hq, D]."""
    _dev(q, count, cu, cache_k, cache_v, block_table, kv_len, out, order)
    _want(block_table, torch.int32, "block_table")
    _want(kv_len, torch.int32, "kv_len")
    hq, d = q.shape[1], q.shape[2]
    hkv = cache_k.shape[1]
    batch = count.shape[0]
    assert cache_v.shape == cache_k.shape and cache_k.dtype == q.dtype
    assert block_table.shape[0] == batch
    if order is not None:
        _want(order, torch.int32, "order")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if contract.enabled():
        contract.check_attention(count, cu, kv_len, k_max, min(q.shape[0], out.shape[0]),
                                 cache_rows=cache_k.shape[0], block_table=block_table,
                                 page_size=page_size, order=order)
    _check("bte_reduced_attention_paged", lib.bte_reduced_attention_paged(
        _ptr(q), _ptr(count), _ptr(cu), _ptr(cache_k), _ptr(cache_v), _ptr(block_table),
        block_table.shape[1], page_size, _ptr(kv_len), _ptr(order), _ptr(out), batch, k_max, hq,
        hkv, d, float(scale), _dtype(q), _stream()))
    return out


def kv_scatter_attention_paged(q, count, cu, idx, n: int, pos_base, new_k, new_v, cache_k, cache_v,
                               block_table, page_size: int, kv_len, k_max: int,
                               scale: float | None = None, out=None, order=None):
    """kv_scatter_paged (logical positions pos_base[b] + idx) then reduced_attention_paged,
    in one launch over the same page pool and table."""
    _dev(q, count, cu, idx, pos_base, new_k, new_v, cache_k, cache_v, block_table, kv_len, out,
         order)
    _want(block_table, torch.int32, "block_table")
    _want(kv_len, torch.int32, "kv_len")
    _want(pos_base, torch.int32, "pos_base")
    _want(idx, torch.int32, "idx")
    hq, d = q.shape[1], q.shape[2]
    hkv = cache_k.shape[1]
    batch = count.shape[0]
    assert idx.shape == (batch, k_max) and pos_base.shape == (batch,)
    assert cache_v.shape == cache_k.shape and cache_k.dtype == q.dtype
    assert new_k.shape[1:] == cache_k.shape[1:] and new_v.shape == new_k.shape
    assert new_k.dtype == q.dtype and new_v.dtype == q.dtype
    assert block_table.shape[0] == batch
    if order is not None:
        _want(order, torch.int32, "order")
        assert order.shape == (batch,)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if contract.enabled():
        contract.check_attention(count, cu, kv_len, k_max, min(q.shape[0], out.shape[0]),
                                 cache_rows=cache_k.shape[0], block_table=block_table,
                                 page_size=page_size, order=order)
        contract.check_fused_scatter(idx, count, cu, k_max, n, pos_base, kv_len, new_k.shape[0],
                                     cache_rows=cache_k.shape[0], block_table=block_table,
                                     page_size=page_size)
    _check("bte_kv_scatter_attention_paged", lib.bte_kv_scatter_attention_paged(
        _ptr(q), _ptr(count), _ptr(cu), _ptr(idx), n, _ptr(pos_base), _ptr(new_k), _ptr(new_v),
        _ptr(cache_k), _ptr(cache_v), _ptr(block_table), block_table.shape[1], page_size,
        _ptr(kv_len), _ptr(order), _ptr(out), batch, k_max, hq, hkv, d, float(scale), _dtype(q),
        _stream()))
    return out


def kv_scatter_paged(new_k, new_v, idx, count, cu, pos_base, block_table, page_size: int,
                     cache_k, cache_v, pos_map=None):
    """Write new_k/new_v rows cu[b]+t to the pool rows of logical positions pos_base[b] + pos."""
    _dev(new_k, new_v, idx, count, cu, pos_base, block_table, cache_k, cache_v, pos_map)
    _want(pos_base, torch.int32, "pos_base")
    _want(block_table, torch.int32, "block_table")
    batch, k_max = idx.shape
    row_bytes = cache_k[0].numel() * cache_k.element_size()
    assert new_k[0].numel() * new_k.element_size() == row_bytes
    n = 0 if pos_map is None else pos_map.shape[1]
    if contract.enabled():
        contract.check_scatter_paged(idx, count, cu, k_max, pos_base, block_table, page_size,
                                     cache_k.shape[0], new_k.shape[0], pos_map)
    _check("bte_kv_scatter_paged", lib.bte_kv_scatter_paged(
        _ptr(new_k), _ptr(new_v), _ptr(idx), _ptr(count), _ptr(cu), _ptr(pos_map), n,
        _ptr(pos_base), _ptr(block_table), block_table.shape[1], page_size, _ptr(cache_k),
        _ptr(cache_v), batch, k_max, row_bytes, _stream()))
    return cache_k, cache_v


def focus_commit_mask(decoded, cached, commit=None, block_done=None):
    """decoded uint8 [batch, B], cached uint8 [batch, B] (updated in place)
    -> (commit uint8 [batch, B], block_done int32 [batch])."""
    _dev(decoded, cached, commit, block_done)
    _want(decoded, torch.uint8, "decoded")
    _want(cached, torch.uint8, "cached")
    batch, block = decoded.shape
    assert cached.shape == (batch, block)
    if commit is None:
        commit = torch.empty_like(decoded)
    if block_done is None:
        block_done = torch.empty((batch,), dtype=torch.int32, device=decoded.device)
    _check("bte_focus_commit_mask", lib.bte_focus_commit_mask(
        _ptr(decoded), _ptr(cached), _ptr(commit), _ptr(block_done), batch, block, _stream()))
    return commit, block_done


class _RowsTensor(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("row_bytes", ctypes.c_size_t)]


def gather_rows_multi(srcs, idx, count, cu, outs=None):
    """Each src [batch, n, ...] compacted with the same index set in one launch;
    returns the outputs [batch * k_max, ...] (rows cu[b]+t written)."""
    _dev(idx, count, cu, *srcs)
    batch, k_max = idx.shape
    n = srcs[0].shape[1]
    if outs is None:
        outs = [torch.empty((batch * k_max,) + tuple(s.shape[2:]), dtype=s.dtype, device=s.device)
                for s in srcs]
    _dev(*outs)
    descs = []
    for s_, o in zip(srcs, outs):
        assert s_.shape[:2] == (batch, n) and o.dtype == s_.dtype
        rb = s_[0, 0].numel() * s_.element_size()
        assert o[0].numel() * o.element_size() == rb
        descs.append(_RowsTensor(s_.data_ptr(), o.data_ptr(), rb))
    if contract.enabled():
        contract.check_rows(idx, count, cu, k_max, n=n, out_rows=min(o.shape[0] for o in outs))
    arr = (_RowsTensor * len(descs))(*descs)
    _check("bte_gather_rows_multi", lib.bte_gather_rows_multi(
        ctypes.cast(arr, ctypes.c_void_p), len(descs), _ptr(idx), _ptr(count), _ptr(cu), batch, n,
        k_max, _stream()))
    return outs
