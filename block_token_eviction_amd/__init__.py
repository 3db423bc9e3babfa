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
           "kv_scatter_attention", "kv_scatter_attention_paged", "esdllm_score_update",
           "esdllm_schedule", "gather_rows_multi_ragged", "BTE_F32", "BTE_BF16", "contract"]

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
    "bte_esdllm_score_update": ([_p, _p, _p, _p, _p, _p, _f, _p, _i, _i, _i, _i, _i, _p], _i),
    "bte_esdllm_schedule": ([_p, _p, _i, _i, _p, _i, _p, _p, _p, _p, _p, _i, _p], _i),
    "bte_gather_rows_multi_ragged": ([_p, _i, _p, _p, _p, _p, _i, _i, _p], _i),
}
ES_MAX_SKIP_LAYERS = 8
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


def _need(cond: bool, msg: str):
    """Host-side argument check that survives ``python -O`` (unlike assert)."""
    if not cond:
        raise ValueError(msg)


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _i32(t, name, shape=None):
    """An int32 index tensor (a wider integer would be read as pairs of int32)."""
    if t is None:
        return
    _want(t, torch.int32, name)
    if shape is not None:
        _shape(t, shape, name)


def _kept_lists(idx, count, cu, batch=None):
    """idx int32 [batch, k_max], count int32 [batch], cu int32 [batch + 1] -> (batch, k_max)."""
    _need(idx.dim() == 2, f"idx must be [batch, k_max], got {tuple(idx.shape)}")
    b, k_max = idx.shape
    if batch is not None:
        _need(b == batch, f"idx has {b} rows for a batch of {batch}")
    _i32(idx, "idx")
    _i32(count, "count", (b,))
    _i32(cu, "cu", (b + 1,))
    return b, k_max


def _row_bytes(t) -> int:
    return t[0].numel() * t.element_size() if t.shape[0] else 0


def focus_importance_delta(q0, k0, q1, k1, decoded, pool_kernel: int, out=None):
    """q* [batch, B, hq, D], k* [batch, B, hkv, D], decoded uint8 [batch, B] -> delta f32 [batch, B]."""
    _dev(q0, k0, q1, k1, decoded, out)
    _need(q0.dim() == 4 and k0.dim() == 4, "q* must be [batch, B, hq, D] and k* [batch, B, hkv, D]")
    batch, block, hq, d = q0.shape
    hkv = k0.shape[2]
    _shape(q1, q0.shape, "q1")
    _need(q1.dtype == q0.dtype, "q0 and q1 must share a dtype")
    for name, t in (("k0", k0), ("k1", k1)):
        _shape(t, (batch, block, hkv, d), name)
        _need(t.dtype == q0.dtype, f"{name} must have the dtype of q0")
    _want(decoded, torch.uint8, "decoded")
    _shape(decoded, (batch, block), "decoded")
    if out is None:
        out = torch.empty((batch, block), dtype=torch.float32, device=q0.device)
    _want(out, torch.float32, "out")
    _shape(out, (batch, block), "out")
    _check("bte_focus_importance_delta", lib.bte_focus_importance_delta(
        _ptr(q0), _ptr(k0), _ptr(q1), _ptr(k1), _ptr(decoded), _ptr(out), batch, block, hq, hkv,
        d, pool_kernel, _dtype(q0), _stream()))
    return out


def esdllm_score(h_new, h_prev, surv_pos, conf, alpha: float, out=None):
    """h_new [batch, n_surv, h], h_prev [batch, L, h], surv_pos int32, conf f32 [batch, L]."""
    _dev(h_new, h_prev, surv_pos, conf, out)
    _need(h_new.dim() == 3 and h_prev.dim() == 3, "h_new and h_prev must be [batch, rows, hidden]")
    batch, n_surv, hidden = h_new.shape
    seq_len = h_prev.shape[1]
    _shape(h_prev, (batch, seq_len, hidden), "h_prev")
    _need(h_prev.dtype == h_new.dtype, "h_new and h_prev must share a dtype")
    _i32(surv_pos, "surv_pos", (batch, n_surv))
    _want(conf, torch.float32, "conf")
    _shape(conf, (batch, seq_len), "conf")
    if out is None:
        out = torch.empty((batch, n_surv), dtype=torch.float32, device=h_new.device)
    _want(out, torch.float32, "out")
    _shape(out, (batch, n_surv), "out")
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
    _need(scores.dim() == 2, "scores must be [batch, n]")
    batch, n = scores.shape
    _i32(k, "k", (batch,))
    dev = scores.device
    if idx is None:
        idx = torch.empty((batch, max(k_max, 0)), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((batch,), dtype=torch.int32, device=dev)
    if cu is None:
        cu = torch.empty((batch + 1,), dtype=torch.int32, device=dev)
    _i32(idx, "idx", (batch, max(k_max, 0)))
    _i32(count, "count", (batch,))
    _i32(cu, "cu", (batch + 1,))
    _check("bte_topk_select", lib.bte_topk_select(
        _ptr(scores), _ptr(k), _ptr(idx) if k_max > 0 else None, _ptr(count), _ptr(cu), batch, n,
        k_max, _stream()))
    return idx, count, cu


def gather_rows(src, idx, count, cu, out=None):
    """src [batch, n, ...] -> out [capacity, ...]; rows cu[b]+t for t < count[b] are written.

    Without `out`, the capacity is batch * k_max rows (the device-side total is
    not read back)."""
    _dev(src, idx, count, cu, out)
    _need(src.dim() >= 3, "src must be [batch, n, ...]")
    batch, n = src.shape[:2]
    _, k_max = _kept_lists(idx, count, cu, batch)
    row_bytes = src[0, 0].numel() * src.element_size()
    if out is None:
        out = torch.empty((batch * k_max,) + tuple(src.shape[2:]), dtype=src.dtype, device=src.device)
    _need(out.dtype == src.dtype, "out must have the dtype of src")
    _need(_row_bytes(out) == row_bytes, "out rows must be the size of src rows")
    if contract.enabled():
        contract.check_rows(idx, count, cu, k_max, n=n, out_rows=out.shape[0])
    _check("bte_gather_rows", lib.bte_gather_rows(
        _ptr(src), _ptr(idx), _ptr(count), _ptr(cu), _ptr(out), batch, n, k_max, row_bytes,
        _stream()))
    return out


def kv_scatter(new_k, new_v, idx, count, cu, row_base, cache_k, cache_v, pos_map=None):
    """Write new_k/new_v rows cu[b]+t into cache rows row_base[b] + pos (in place)."""
    _dev(new_k, new_v, idx, count, cu, row_base, cache_k, cache_v, pos_map)
    batch, k_max = _kept_lists(idx, count, cu)
    _want(row_base, torch.int64, "row_base")
    _shape(row_base, (batch,), "row_base")
    row_bytes = _row_bytes(cache_k)
    _need(_row_bytes(new_k) == row_bytes, "new_k rows must be the size of cache_k rows")
    _need(new_k.dtype == cache_k.dtype, "new_k must have the dtype of cache_k")
    _need((new_v is None) == (cache_v is None), "give new_v and cache_v together")
    if new_v is not None:
        _shape(new_v, new_k.shape, "new_v")
        _shape(cache_v, cache_k.shape, "cache_v")
        _need(new_v.dtype == new_k.dtype and cache_v.dtype == cache_k.dtype,
              "K and V tensors must share a dtype")
    if pos_map is not None:
        _i32(pos_map, "pos_map")
        _need(pos_map.dim() == 2 and pos_map.shape[0] == batch, "pos_map must be [batch, n]")
    n = 0 if pos_map is None else pos_map.shape[1]
    if contract.enabled():
        contract.check_scatter(idx, count, cu, k_max, row_base, cache_k.shape[0], new_k.shape[0],
                               pos_map)
    _check("bte_kv_scatter", lib.bte_kv_scatter(
        _ptr(new_k), _ptr(new_v), _ptr(idx), _ptr(count), _ptr(cu), _ptr(pos_map), n,
        _ptr(row_base), _ptr(cache_k), _ptr(cache_v), batch, k_max, row_bytes, _stream()))
    return cache_k, cache_v


def _attn_shapes(q, count, cu, cache_k, cache_v):
    """q [rows, hq, D], count int32 [batch], cu int32 [batch + 1], cache K/V [rows, hkv, D]
    of q's dtype -> (hq, D, hkv, batch)."""
    _need(q.dim() == 3 and cache_k.dim() == 3, "q must be [rows, hq, D] and the cache [rows, hkv, D]")
    _need(count.dim() == 1, "count must be [batch]")
    batch = count.shape[0]
    _i32(count, "count")
    _i32(cu, "cu", (batch + 1,))
    hq, d = q.shape[1], q.shape[2]
    hkv = cache_k.shape[1]
    _need(cache_k.shape[2] == d, "the cache's head dim must equal q's")
    _shape(cache_v, cache_k.shape, "cache_v")
    _need(cache_k.dtype == q.dtype and cache_v.dtype == q.dtype, "the cache must have q's dtype")
    return hq, d, hkv, batch


def _attn_out(q, out):
    if out is None:
        return torch.empty_like(q)
    _need(out.dtype == q.dtype and out.dim() == 3 and out.shape[1:] == q.shape[1:],
          "out must be [rows, hq, D] with q's dtype")
    return out


def _fused_rows(idx, pos_base, new_k, new_v, q, cache_k, batch, k_max):
    _i32(idx, "idx", (batch, k_max))
    _i32(pos_base, "pos_base", (batch,))
    _need(new_k.dim() == 3 and new_k.shape[1:] == cache_k.shape[1:],
          "new_k must be [rows, hkv, D] like the cache")
    _shape(new_v, new_k.shape, "new_v")
    _need(new_k.dtype == q.dtype and new_v.dtype == q.dtype, "new_k/new_v must have q's dtype")


def _page_table(block_table, batch):
    _want(block_table, torch.int32, "block_table")
    _need(block_table.dim() == 2 and block_table.shape[0] == batch,
          "block_table must be [batch, max_pages]")


def reduced_attention(q, count, cu, cache_k, cache_v, seq_start, kv_len, k_max: int,
                      scale: float | None = None, out=None, order=None):
    """q [capacity, hq, D], cache [rows, hkv, D] -> out [capacity, hq, D] (rows cu[b]+t written).

    `order` (int32 [batch], e.g. from attention_order) only schedules the work."""
    _dev(q, count, cu, cache_k, cache_v, seq_start, kv_len, out, order)
    hq, d, hkv, batch = _attn_shapes(q, count, cu, cache_k, cache_v)
    _want(seq_start, torch.int64, "seq_start")
    _shape(seq_start, (batch,), "seq_start")
    _i32(kv_len, "kv_len", (batch,))
    _i32(order, "order", (batch,))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _attn_out(q, out)
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
    hq, d, hkv, batch = _attn_shapes(q, count, cu, cache_k, cache_v)
    _want(seq_start, torch.int64, "seq_start")
    _shape(seq_start, (batch,), "seq_start")
    _i32(kv_len, "kv_len", (batch,))
    _i32(order, "order", (batch,))
    _fused_rows(idx, pos_base, new_k, new_v, q, cache_k, batch, k_max)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _attn_out(q, out)
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
    _need(kv_len.dim() == 1, "kv_len must be [batch]")
    batch = kv_len.shape[0]
    _i32(kv_len, "kv_len")
    _i32(count, "count", (batch,))
    if out is None:
        out = torch.empty((batch,), dtype=torch.int32, device=kv_len.device)
    _i32(out, "out", (batch,))
    _check("bte_attention_order", lib.bte_attention_order(_ptr(kv_len), _ptr(count), int(group),
                                                          batch, _ptr(out), _stream()))
    return out


def focus_budget(delta, token_sum, total_steps, alpha: float, threshold_mode: int = 0, out=None):
    """delta f32 [batch, B], token_sum/total_steps int32 [batch] -> K int32 [batch]."""
    _dev(delta, token_sum, total_steps, out)
    _want(delta, torch.float32, "delta")
    _need(delta.dim() == 2, "delta must be [batch, B]")
    batch, block = delta.shape
    _i32(token_sum, "token_sum", (batch,))
    _i32(total_steps, "total_steps", (batch,))
    if out is None:
        out = torch.empty((batch,), dtype=torch.int32, device=delta.device)
    _i32(out, "out", (batch,))
    _check("bte_focus_budget", lib.bte_focus_budget(
        _ptr(delta), _ptr(token_sum), _ptr(total_steps), float(alpha), int(threshold_mode),
        _ptr(out), batch, block, _stream()))
    return out


def focus_history_update(decoded_prev, decoded_now, token_sum, total_steps):
    """In place: token_sum += newly decoded positions, total_steps += 1."""
    _dev(decoded_prev, decoded_now, token_sum, total_steps)
    _want(decoded_prev, torch.uint8, "decoded_prev")
    _want(decoded_now, torch.uint8, "decoded_now")
    _need(decoded_now.dim() == 2, "decoded_now must be [batch, B]")
    batch, block = decoded_now.shape
    _shape(decoded_prev, (batch, block), "decoded_prev")
    _i32(token_sum, "token_sum", (batch,))
    _i32(total_steps, "total_steps", (batch,))
    _check("bte_focus_history_update", lib.bte_focus_history_update(
        _ptr(decoded_prev), _ptr(decoded_now), _ptr(token_sum), _ptr(total_steps), batch, block,
        _stream()))
    return token_sum, total_steps


def focus_select(delta, k, decoded, rightmost_processed, idx=None, count=None, cu=None):
    """Top-K + AR-context + placeholder integrity + |S| >= 1.
    -> (idx int32 [batch, B], count [batch], cu [batch + 1]); rightmost_processed updated in place."""
    _dev(delta, k, decoded, rightmost_processed, idx, count, cu)
    _want(delta, torch.float32, "delta")
    _need(delta.dim() == 2, "delta must be [batch, B]")
    batch, block = delta.shape
    _i32(k, "k", (batch,))
    _want(decoded, torch.uint8, "decoded")
    _shape(decoded, (batch, block), "decoded")
    _i32(rightmost_processed, "rightmost_processed", (batch,))
    dev = delta.device
    if idx is None:
        idx = torch.empty((batch, block), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((batch,), dtype=torch.int32, device=dev)
    if cu is None:
        cu = torch.empty((batch + 1,), dtype=torch.int32, device=dev)
    _i32(idx, "idx", (batch, block))
    _i32(count, "count", (batch,))
    _i32(cu, "cu", (batch + 1,))
    _check("bte_focus_select", lib.bte_focus_select(
        _ptr(delta), _ptr(k), _ptr(decoded), _ptr(rightmost_processed), _ptr(idx), _ptr(count),
        _ptr(cu), batch, block, _stream()))
    return idx, count, cu


def reduced_attention_paged(q, count, cu, cache_k, cache_v, block_table, page_size: int, kv_len,
                            k_max: int, scale: float | None = None, out=None, order=None):
    """q [capacity, hq, D]; page pool cache [n_pages * page_size, hkv, D];
    block_table int32 [batch, max_pages] -> out [capacity, hq, D]."""
    _dev(q, count, cu, cache_k, cache_v, block_table, kv_len, out, order)
    hq, d, hkv, batch = _attn_shapes(q, count, cu, cache_k, cache_v)
    _page_table(block_table, batch)
    _i32(kv_len, "kv_len", (batch,))
    _i32(order, "order", (batch,))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _attn_out(q, out)
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
    hq, d, hkv, batch = _attn_shapes(q, count, cu, cache_k, cache_v)
    _page_table(block_table, batch)
    _i32(kv_len, "kv_len", (batch,))
    _i32(order, "order", (batch,))
    _fused_rows(idx, pos_base, new_k, new_v, q, cache_k, batch, k_max)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _attn_out(q, out)
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
    batch, k_max = _kept_lists(idx, count, cu)
    _i32(pos_base, "pos_base", (batch,))
    _page_table(block_table, batch)
    row_bytes = _row_bytes(cache_k)
    _need(_row_bytes(new_k) == row_bytes, "new_k rows must be the size of cache_k rows")
    _need(new_k.dtype == cache_k.dtype, "new_k must have the dtype of cache_k")
    _need((new_v is None) == (cache_v is None), "give new_v and cache_v together")
    if new_v is not None:
        _shape(new_v, new_k.shape, "new_v")
        _shape(cache_v, cache_k.shape, "cache_v")
        _need(new_v.dtype == new_k.dtype and cache_v.dtype == cache_k.dtype,
              "K and V tensors must share a dtype")
    if pos_map is not None:
        _i32(pos_map, "pos_map")
        _need(pos_map.dim() == 2 and pos_map.shape[0] == batch, "pos_map must be [batch, n]")
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
    _need(decoded.dim() == 2, "decoded must be [batch, B]")
    batch, block = decoded.shape
    _shape(cached, (batch, block), "cached")
    if commit is None:
        commit = torch.empty_like(decoded)
    if block_done is None:
        block_done = torch.empty((batch,), dtype=torch.int32, device=decoded.device)
    _want(commit, torch.uint8, "commit")
    _shape(commit, (batch, block), "commit")
    _i32(block_done, "block_done", (batch,))
    _check("bte_focus_commit_mask", lib.bte_focus_commit_mask(
        _ptr(decoded), _ptr(cached), _ptr(commit), _ptr(block_done), batch, block, _stream()))
    return commit, block_done


class _RowsTensor(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("row_bytes", ctypes.c_size_t)]


def gather_rows_multi(srcs, idx, count, cu, outs=None):
    """Each src [batch, n, ...] compacted with the same index set in one launch;
    returns the outputs [batch * k_max, ...] (rows cu[b]+t written)."""
    _dev(idx, count, cu, *srcs)
    batch, k_max = _kept_lists(idx, count, cu)
    _need(len(srcs) >= 1 and srcs[0].dim() >= 2, "give at least one src [batch, n, ...]")
    n = srcs[0].shape[1]
    if outs is None:
        outs = [torch.empty((batch * k_max,) + tuple(s.shape[2:]), dtype=s.dtype, device=s.device)
                for s in srcs]
    _need(len(outs) == len(srcs), "give one output per source")
    _dev(*outs)
    descs = []
    for i, (s_, o) in enumerate(zip(srcs, outs)):
        _need(s_.dim() >= 2 and tuple(s_.shape[:2]) == (batch, n), f"src {i} must be [batch, n, ...]")
        _need(o.dtype == s_.dtype, f"output {i} must have the dtype of its source")
        rb = s_[0, 0].numel() * s_.element_size()
        _need(_row_bytes(o) == rb, f"output {i} rows must be the size of its source rows")
        descs.append(_RowsTensor(s_.data_ptr(), o.data_ptr(), rb))
    if contract.enabled():
        contract.check_rows(idx, count, cu, k_max, n=n, out_rows=min(o.shape[0] for o in outs))
    arr = (_RowsTensor * len(descs))(*descs)
    _check("bte_gather_rows_multi", lib.bte_gather_rows_multi(
        ctypes.cast(arr, ctypes.c_void_p), len(descs), _ptr(idx), _ptr(count), _ptr(cu), batch, n,
        k_max, _stream()))
    return outs


def esdllm_score_update(h_new, h_cache, surv_pos, conf, alpha: float, count=None, cu=None,
                        cap: int | None = None, out=None):
    """Score the survivors against h_cache [batch, L, h] and write their new states into it.

    Without count/cu: h_new [batch, cap, h] and surv_pos int32 [batch, cap] (every slot a
    survivor). With count (int32 [batch]) and cu (int32 [batch + 1]): h_new [rows, h] and
    surv_pos int32 [rows], sequence b's survivors at rows cu[b] .. cu[b] + count[b] - 1, and
    `cap` slots per sequence in the output. -> score f32 [batch, cap] (-inf past count)."""
    _dev(h_new, h_cache, surv_pos, conf, count, cu, out)
    _need(h_cache.dim() == 3, "h_cache must be [batch, seq_len, hidden]")
    batch, seq_len, hidden = h_cache.shape
    _need(h_new.dtype == h_cache.dtype, "h_new and h_cache must share a dtype")
    _need(h_new.data_ptr() != h_cache.data_ptr(), "h_new must not be h_cache")
    _want(conf, torch.float32, "conf")
    _shape(conf, (batch, seq_len), "conf")
    _need((count is None) == (cu is None), "give count and cu together")
    if count is None:
        _need(h_new.dim() == 3 and tuple(h_new.shape[::2]) == (batch, hidden),
              "h_new must be [batch, cap, hidden]")
        cap = h_new.shape[1]
        _i32(surv_pos, "surv_pos", (batch, cap))
    else:
        _need(cap is not None and cap > 0, "give cap (survivor slots per sequence) with count")
        _i32(count, "count", (batch,))
        _i32(cu, "cu", (batch + 1,))
        _need(h_new.dim() == 2 and h_new.shape[1] == hidden, "h_new must be [rows, hidden]")
        _i32(surv_pos, "surv_pos")
        _need(surv_pos.dim() == 1 and surv_pos.shape[0] == h_new.shape[0],
              "surv_pos must be [rows] like h_new")
    if out is None:
        out = torch.empty((batch, cap), dtype=torch.float32, device=h_new.device)
    _want(out, torch.float32, "out")
    _shape(out, (batch, cap), "out")
    if contract.enabled():
        contract.check_survivors(surv_pos, seq_len, count, cu, cap, rows=h_new.shape[0])
    _check("bte_esdllm_score_update", lib.bte_esdllm_score_update(
        _ptr(h_new), _ptr(h_cache), _ptr(surv_pos), _ptr(count), _ptr(cu), _ptr(conf),
        float(alpha), _ptr(out), batch, cap, seq_len, hidden, _dtype(h_new), _stream()))
    return out


def esdllm_schedule(iter_, block_start, block_len: int, period: int, keep, surv_pos=None,
                    count=None, cu=None, keep_out=None, refresh=None):
    """One iteration's bookkeeping: iter_ int32 [batch] (advanced in place), block_start int32
    [batch], keep = the skip layers' keep counts (host ints) -> (surv_pos [batch, block_len],
    count [batch], cu [batch + 1], keep_out [n_layers, batch] int32, refresh uint8 [batch])."""
    _dev(iter_, block_start, surv_pos, count, cu, keep_out, refresh)
    _need(iter_.dim() == 1, "iter must be [batch]")
    batch = iter_.shape[0]
    _i32(iter_, "iter")
    _i32(block_start, "block_start", (batch,))
    keep = [int(v) for v in keep]
    n_layers = len(keep)
    _need(n_layers <= ES_MAX_SKIP_LAYERS, f"at most {ES_MAX_SKIP_LAYERS} skip layers")
    dev, i32 = iter_.device, torch.int32
    if surv_pos is None:
        surv_pos = torch.empty((batch, block_len), dtype=i32, device=dev)
    if count is None:
        count = torch.empty((batch,), dtype=i32, device=dev)
    if cu is None:
        cu = torch.empty((batch + 1,), dtype=i32, device=dev)
    if keep_out is None:
        keep_out = torch.empty((max(n_layers, 1), batch), dtype=i32, device=dev)
    if refresh is None:
        refresh = torch.empty((batch,), dtype=torch.uint8, device=dev)
    _i32(surv_pos, "surv_pos", (batch, block_len))
    _i32(count, "count", (batch,))
    _i32(cu, "cu", (batch + 1,))
    _i32(keep_out, "keep_out")
    _need(keep_out.dim() == 2 and keep_out.shape[1] == batch and keep_out.shape[0] >= n_layers,
          "keep_out must be [n_layers, batch]")
    _want(refresh, torch.uint8, "refresh")
    _shape(refresh, (batch,), "refresh")
    karr = (ctypes.c_int32 * max(n_layers, 1))(*keep) if n_layers else None
    _check("bte_esdllm_schedule", lib.bte_esdllm_schedule(
        _ptr(iter_), _ptr(block_start), int(block_len), int(period),
        ctypes.cast(karr, ctypes.c_void_p) if karr is not None else None, n_layers, _ptr(surv_pos),
        _ptr(count), _ptr(cu), _ptr(keep_out), _ptr(refresh), batch, _stream()))
    return surv_pos, count, cu, keep_out, refresh


def gather_rows_multi_ragged(srcs, src_cu, idx, count, cu, outs=None):
    """Each src [rows, ...], compacted by sequence (sequence b's rows start at src_cu[b]),
    gathered with one index set in one launch: out[cu[b] + t] = src[src_cu[b] + idx[b, t]].
    Returns the outputs [batch * k_max, ...]."""
    _dev(src_cu, idx, count, cu, *srcs)
    batch, k_max = _kept_lists(idx, count, cu)
    _i32(src_cu, "src_cu")
    _need(src_cu.dim() == 1 and src_cu.shape[0] >= batch, "src_cu must be [batch] (or [batch + 1])")
    _need(len(srcs) >= 1, "give at least one source")
    if outs is None:
        outs = [torch.empty((batch * k_max,) + tuple(s.shape[1:]), dtype=s.dtype, device=s.device)
                for s in srcs]
    _need(len(outs) == len(srcs), "give one output per source")
    _dev(*outs)
    descs = []
    for i, (s_, o) in enumerate(zip(srcs, outs)):
        _need(s_.dim() >= 1 and o.dtype == s_.dtype, f"output {i} must have the dtype of its source")
        rb = _row_bytes(s_)
        _need(_row_bytes(o) == rb, f"output {i} rows must be the size of its source rows")
        descs.append(_RowsTensor(s_.data_ptr(), o.data_ptr(), rb))
    if contract.enabled():
        contract.check_rows(idx, count, cu, k_max, out_rows=min(o.shape[0] for o in outs))
        contract.check_ragged_source(src_cu, idx, count, min(s_.shape[0] for s_ in srcs))
    arr = (_RowsTensor * len(descs))(*descs)
    _check("bte_gather_rows_multi_ragged", lib.bte_gather_rows_multi_ragged(
        ctypes.cast(arr, ctypes.c_void_p), len(descs), _ptr(src_cu), _ptr(idx), _ptr(count),
        _ptr(cu), batch, k_max, _stream()))
    return outs
