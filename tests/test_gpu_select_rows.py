"""GPU parity: top-K selection, gather and KV scatter (bit-exact vs the oracle)."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import dev, say

pytestmark = pytest.mark.gpu


def _bte():
    import block_token_eviction_amd as bte
    return bte


def _topk(scores: np.ndarray, k: np.ndarray, k_max: int):
    bte = _bte()
    say(f"topk batch={scores.shape[0]} n={scores.shape[1]} k_max={k_max}")
    idx, cnt, cu = bte.topk_select(torch.from_numpy(scores).cuda(),
                                   torch.from_numpy(k.astype(np.int32)).cuda(), k_max)
    torch.cuda.synchronize()
    r = oracle.topk_select(scores, k, k_max)
    np.testing.assert_array_equal(cnt.cpu().numpy(), r[1])
    np.testing.assert_array_equal(cu.cpu().numpy(), r[2])
    if k_max:
        np.testing.assert_array_equal(idx.cpu().numpy(), r[0])


def test_topk_exhaustive_special_values():
    vals = [-math.inf, math.nan, -1.0, -0.0, 0.0, 1.0, math.inf]
    rows = np.array(list(itertools.product(vals, repeat=4)), dtype=np.float32)
    for kk in range(0, 6):
        for k_max in (0, 2, 4, 6):
            _topk(rows, np.full(len(rows), kk), k_max)


@pytest.mark.parametrize("n", [32, 64, 65, 256, 1000, 1024])
def test_topk_random_with_ties(n):
    r = np.random.default_rng(n)
    batch = 300
    s = r.integers(-4, 5, size=(batch, n)).astype(np.float32) * 0.25      # many exact ties
    s[r.uniform(size=s.shape) < 0.3] = -np.inf
    s[r.uniform(size=s.shape) < 0.01] = np.nan
    k = r.integers(-2, n + 3, size=batch)
    _topk(s, k, min(n, 40))


@pytest.mark.parametrize("n", [1, 7, 32, 64, 65, 200, 256, 257, 1024])
@pytest.mark.parametrize("batch", [1, 2, 3, 8, 9, 32, 33])
def test_topk_small_batches(n, batch):
    """Small and odd batch sizes across the kernel's row-width classes (n <= 64, <= 256,
    <= 1024): ties, -inf, NaN, K <= 0 and K > n; counts and cu also with k_max = 0."""
    r = np.random.default_rng(1000 * n + batch)
    s = r.integers(-3, 4, size=(batch, n)).astype(np.float32) * 0.5
    s[r.uniform(size=s.shape) < 0.25] = -np.inf
    s[r.uniform(size=s.shape) < 0.02] = np.nan
    k = r.integers(-1, n + 2, size=batch)
    _topk(s, k, min(n, 40))
    _topk(s, k, 0)                                          # counts and cu only


def test_topk_config_shapes_and_long_scan():
    r = np.random.default_rng(5)
    s = r.standard_normal((5000, 32)).astype(np.float32)                 # > 1024 rows: scan loops
    s[r.uniform(size=s.shape) < 0.45] = -np.inf
    _topk(s, r.integers(4, 13, size=5000), 12)
    s = r.standard_normal((8, 256)).astype(np.float32)                   # ES-dLLM: 128 of 256
    _topk(s, np.full(8, 128), 128)


def test_gather_focus_b256_full_size():
    bte = _bte()
    cfg = W.FOCUS_B256
    fi = W.focus_inputs(cfg)
    r = np.random.default_rng(7)
    scores = r.standard_normal((cfg.batch, cfg.block)).astype(np.float32)
    scores[fi["decoded"].numpy() != 0] = -np.inf
    idx, cnt, cu = oracle.topk_select(scores, fi["k"].numpy(), cfg.k_hi)
    src = fi["hidden"]
    say("gather b256 h4096 bf16")
    out = bte.gather_rows(src.cuda(), torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                          torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    ref = oracle.gather_rows(src.view(torch.int16).numpy(), idx, cnt, cu)
    np.testing.assert_array_equal(out[: int(cu[-1])].cpu().view(torch.int16).numpy(), ref)


@pytest.mark.parametrize("row_bytes", [16, 48, 4096 * 2 + 16 * 3])
def test_gather_ragged_row_sizes(row_bytes):
    bte = _bte()
    r = np.random.default_rng(row_bytes)
    batch, n = 9, 40
    src = torch.from_numpy(r.integers(0, 255, size=(batch, n, row_bytes), dtype=np.uint8))
    scores = r.standard_normal((batch, n)).astype(np.float32)
    idx, cnt, cu = oracle.topk_select(scores, r.integers(0, 9, size=batch), 8)
    say(f"gather row_bytes={row_bytes}")
    out = bte.gather_rows(src.cuda(), torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                          torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out[: int(cu[-1])].cpu().numpy(), oracle.gather_rows(src.numpy(), idx, cnt, cu))


def _scatter_check(ai, idx, cnt, cu, pos_map=None, single=False):
    bte = _bte()
    g = dev(ai)
    ck, cv = g["cache_k"].clone(), g["cache_v"].clone()
    ti, tc, tu = (torch.from_numpy(x).cuda() for x in (idx, cnt, cu))
    pm = None if pos_map is None else torch.from_numpy(pos_map).cuda()
    say(f"scatter rows={ck.shape[0]} single={single} map={pos_map is not None}")
    if single:
        bte.kv_scatter(g["new_k"], None, ti, tc, tu, g["row_base"], ck, None, pos_map=pm)
    else:
        bte.kv_scatter(g["new_k"], g["new_v"], ti, tc, tu, g["row_base"], ck, cv, pos_map=pm)
    torch.cuda.synchronize()
    as_i = lambda t: t.cpu().view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
    rk, rv = oracle.kv_scatter(as_i(ai["new_k"]), as_i(ai["new_v"]), idx, cnt, cu,
                               ai["row_base"].numpy(), as_i(ai["cache_k"]), as_i(ai["cache_v"]), pos_map)
    np.testing.assert_array_equal(as_i(ck), rk)
    np.testing.assert_array_equal(as_i(cv), as_i(ai["cache_v"]) if single else rv)


def test_scatter_attn_b256_full_size():
    ai = W.attention_inputs(W.ATTN_B256)
    _scatter_check(ai, ai["idx"].numpy(), ai["count"].numpy(), ai["cu"].numpy())


def test_scatter_esdllm_pos_map_and_single_tensor():
    cfg = W.ES_B8
    ei = W.esdllm_inputs(cfg)
    r = np.random.default_rng(3)
    scores = r.standard_normal((cfg.batch, cfg.generated)).astype(np.float32)
    idx, cnt, cu = oracle.topk_select(scores, ei["k"].numpy(), cfg.keep)
    ai = dict(new_k=ei["new_k"], new_v=ei["new_v"], cache_k=ei["cache_k"], cache_v=ei["cache_v"],
              row_base=ei["row_base"])
    _scatter_check(ai, idx, cnt, cu, pos_map=ei["surv_pos"].numpy())
    _scatter_check(ai, idx, cnt, cu, pos_map=ei["surv_pos"].numpy(), single=True)
