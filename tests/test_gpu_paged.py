"""GPU parity of the paged KV scatter and paged reduced attention: bitwise
equal to the contiguous kernels on the rows a shuffled page table maps to,
and within tolerance of the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import assert_close, dev, page_table as _page_table, pool as _pool, say

pytestmark = pytest.mark.gpu


def _bte():
    import block_token_eviction_amd as bte
    return bte


CFGS = [
    (W.ATTN_B256, 64),
    (W.ATTN_B256, 16),
    (W.AttnCfg("paged_small", seed=71, batch=9, kept=None, k_lo=0, k_hi=12, hq=32, hkv=8,
               head_dim=128, prefix_lo=1, prefix_hi=300), 8),
    (W.AttnCfg("paged_d64", seed=72, batch=600, kept=None, k_lo=1, k_hi=16, hq=32, hkv=8,
               head_dim=64, prefix_lo=30, prefix_hi=200), 256),
    (W.AttnCfg("paged_f32", seed=73, batch=5, kept=4, hq=8, hkv=2, head_dim=128, dtype=W.F32,
               prefix_lo=40, prefix_hi=150), 32),
    # fp32 head dim 64 through pages smaller than a key tile (one lookup per copy)
    (W.AttnCfg("paged_f32_d64", seed=76, batch=7, kept=None, k_lo=1, k_hi=8, hq=16, hkv=4,
               head_dim=64, dtype=W.F32, prefix_lo=1, prefix_hi=120), 8),
    # head dim 64 with up to 96 query rows per KV head (query split) through the table
    (W.AttnCfg("paged_d64_qsplit", seed=77, batch=40, kept=None, k_lo=8, k_hi=24, hq=32, hkv=8,
               head_dim=64, prefix_lo=5, prefix_hi=300), 16),
    # up to 128 query rows per KV head: query-split workgroups through the table
    (W.AttnCfg("paged_qsplit", seed=75, batch=150, kept=None, k_lo=4, k_hi=32, hq=32, hkv=8,
               head_dim=128, prefix_lo=10, prefix_hi=400), 16),
    # more than 2048 pages per sequence: page entries are read from memory
    (W.AttnCfg("paged_long_table", seed=74, batch=3, kept=5, hq=8, hkv=2, head_dim=128,
               prefix_lo=16600, prefix_hi=17000), 8),
]


@pytest.mark.parametrize("cfg,page", CFGS, ids=[f"{c.name}-p{p}" for c, p in CFGS])
@pytest.mark.parametrize("ordered", [False, True], ids=["index_order", "longest_first"])
def test_paged_attention(cfg, page, ordered):
    bte = _bte()
    ai = W.attention_inputs(cfg)
    g = dev(ai)
    bt, src, n_pages = _page_table(ai["kv_len"].numpy(), page, seed=cfg.seed)
    say(f"paged attention {cfg.name} page={page} ordered={ordered}")
    pk, pv = _pool(g["cache_k"], src, n_pages, page), _pool(g["cache_v"], src, n_pages, page)
    order = bte.attention_order(g["kv_len"]) if ordered else None
    out_p = bte.reduced_attention_paged(g["q"], g["count"], g["cu"], pk, pv,
                                        torch.from_numpy(bt).cuda(), page, g["kv_len"],
                                        ai["k_max"], order=order)
    out_c = bte.reduced_attention(g["q"], g["count"], g["cu"], g["cache_k"], g["cache_v"],
                                  g["seq_start"], g["kv_len"], ai["k_max"], order=order)
    n = int(ai["cu"][-1])
    assert torch.equal(out_p[:n], out_c[:n])
    if ai["rows"] > 200_000:
        return        # the contiguous kernel is checked against the oracle at this size
    ref = oracle.reduced_attention_paged(W.to_f64(ai["q"]), ai["count"].numpy(), ai["cu"].numpy(),
                                         W.to_f64(pk), W.to_f64(pv), bt, page,
                                         ai["kv_len"].numpy(), cfg.hq, cfg.hkv,
                                         1.0 / math.sqrt(cfg.head_dim))
    assert_close(out_p[:n].cpu().double().numpy(), ref[:n], cfg.name)


@pytest.mark.parametrize("page", [1, 16, 64])
def test_paged_scatter(page):
    bte = _bte()
    cfg = W.ATTN_B256
    ai = W.attention_inputs(cfg)
    g = dev(ai)
    bt, src, n_pages = _page_table(ai["kv_len"].numpy(), page, seed=page)
    say(f"paged scatter page={page}")
    pk, pv = _pool(g["cache_k"], src, n_pages, page), _pool(g["cache_v"], src, n_pages, page)
    pk0, pv0 = pk.clone(), pv.clone()
    pos_base = ai["prefix"].to(torch.int32).cuda()
    bte.kv_scatter_paged(g["new_k"], g["new_v"], g["idx"], g["count"], g["cu"], pos_base,
                         torch.from_numpy(bt).cuda(), page, pk, pv)
    # the oracle on the same pool
    bits = lambda t: t.cpu().view(torch.int16).numpy()
    rk, rv = oracle.kv_scatter_paged(bits(ai["new_k"]), bits(ai["new_v"]), ai["idx"].numpy(),
                                     ai["count"].numpy(), ai["cu"].numpy(), ai["prefix"].numpy(),
                                     bt, page, bits(pk0), bits(pv0))
    np.testing.assert_array_equal(pk.cpu().view(torch.int16).numpy(), rk)
    np.testing.assert_array_equal(pv.cpu().view(torch.int16).numpy(), rv)
    # and the contiguous scatter lands the same bytes on the rows the table maps to
    ck, cv = g["cache_k"].clone(), g["cache_v"].clone()
    bte.kv_scatter(g["new_k"], g["new_v"], g["idx"], g["count"], g["cu"], g["row_base"], ck, cv)
    have = torch.from_numpy(np.flatnonzero(src >= 0)).cuda()
    back = torch.from_numpy(src[src >= 0]).cuda()
    assert torch.equal(pk[have], ck[back]) and torch.equal(pv[have], cv[back])
