"""GPU parity of the KV scatter fused into the reduced attention
(bte_kv_scatter_attention and its paged form): bitwise equal to
bte_kv_scatter followed by bte_reduced_attention (outputs and every cache
row), and within tolerance of the oracle's scatter followed by its attention."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import assert_close, dev, page_table, pool, say

pytestmark = pytest.mark.gpu


def _bte():
    import block_token_eviction_amd as bte
    return bte


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _pos_base(ai, cfg, anywhere: bool):
    """The block at the end of each sequence (position P_b), or anywhere a
    block fits inside it."""
    prefix = ai["prefix"].numpy()
    if not anywhere:
        return prefix.astype(np.int32)
    r = np.random.default_rng(cfg.seed + 1000)
    return r.integers(0, prefix + 1).astype(np.int32)


def _oracle(ai, cfg, pos_base, rows=None):
    """Oracle scatter into rows seq_start + pos_base + idx, then the oracle attention."""
    raw = lambda t: t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()
    row_base = ai["seq_start"].numpy() + pos_base.astype(np.int64)
    rk, rv = oracle.kv_scatter(raw(ai["new_k"]), raw(ai["new_v"]), ai["idx"].numpy(),
                               ai["count"].numpy(), ai["cu"].numpy(), row_base,
                               raw(ai["cache_k"]), raw(ai["cache_v"]))
    back = lambda a: W.to_f64(torch.from_numpy(a).view(cfg.dtype))
    return oracle.reduced_attention(W.to_f64(ai["q"]), ai["count"].numpy(), ai["cu"].numpy(),
                                    back(rk), back(rv), ai["seq_start"].numpy(),
                                    ai["kv_len"].numpy(), cfg.hq, cfg.hkv,
                                    1.0 / math.sqrt(cfg.head_dim), rows=rows)


def _fused(cfg, ordered, anywhere=False, sample=None):
    bte = _bte()
    ai = W.attention_inputs(cfg)
    g = dev(ai)
    pb_np = _pos_base(ai, cfg, anywhere)
    pb = torch.from_numpy(pb_np).cuda()
    say(f"fused scatter+attention {cfg.name} batch={cfg.batch} k_max={ai['k_max']} "
        f"D={cfg.head_dim} ordered={ordered} anywhere={anywhere}")
    order = bte.attention_order(g["kv_len"]) if ordered else None
    ck_u, cv_u = g["cache_k"].clone(), g["cache_v"].clone()
    bte.kv_scatter(g["new_k"], g["new_v"], g["idx"], g["count"], g["cu"],
                   g["seq_start"] + pb.to(torch.int64), ck_u, cv_u)
    out_u = bte.reduced_attention(g["q"], g["count"], g["cu"], ck_u, cv_u, g["seq_start"],
                                  g["kv_len"], ai["k_max"], order=order)
    ck_f, cv_f = g["cache_k"].clone(), g["cache_v"].clone()
    out_f = bte.kv_scatter_attention(g["q"], g["count"], g["cu"], g["idx"], cfg.block, pb,
                                     g["new_k"], g["new_v"], ck_f, cv_f, g["seq_start"],
                                     g["kv_len"], ai["k_max"], order=order)
    torch.cuda.synchronize()
    n = int(ai["cu"][-1])
    assert torch.equal(_bits(out_f[:n]), _bits(out_u[:n])), "output differs from scatter + attention"
    assert torch.equal(_bits(ck_f), _bits(ck_u)) and torch.equal(_bits(cv_f), _bits(cv_u)), \
        "cache differs from the separate scatter"
    rows = None
    if sample is not None and n > sample:
        rows = np.random.default_rng(cfg.seed).choice(n, size=sample, replace=False)
    ref = _oracle(ai, cfg, pb_np, rows=rows)
    got = out_f[:n].cpu().to(torch.float64).numpy()
    sel = np.arange(n) if rows is None else np.asarray(rows)
    assert_close(got[sel], ref[:n][sel], cfg.name)


CASES = [
    W.AttnCfg("len1", seed=131, batch=3, kept=1, hq=8, hkv=2, head_dim=128, prefix_lo=0,
              prefix_hi=0, block=1),
    W.AttnCfg("block_across_tiles", seed=132, batch=6, kept=5, hq=8, hkv=2, head_dim=128,
              prefix_lo=1, prefix_hi=70),
    W.AttnCfg("some_empty", seed=133, batch=7, kept=None, k_lo=0, k_hi=12, hq=32, hkv=8,
              head_dim=128, prefix_lo=90, prefix_hi=500),
    W.AttnCfg("no_gqa", seed=134, batch=4, kept=6, hq=8, hkv=8, head_dim=128, prefix_lo=100,
              prefix_hi=300),
    W.AttnCfg("d64", seed=135, batch=4, kept=7, hq=16, hkv=4, head_dim=64, prefix_lo=33,
              prefix_hi=400),
    W.AttnCfg("f32_d128", seed=136, batch=3, kept=4, hq=8, hkv=2, head_dim=128, dtype=W.F32,
              prefix_lo=60, prefix_hi=200),
    W.AttnCfg("f32_d64", seed=137, batch=3, kept=5, hq=8, hkv=2, head_dim=64, dtype=W.F32,
              prefix_lo=1, prefix_hi=90),
    W.AttnCfg("qsplit", seed=138, batch=40, kept=None, k_lo=0, k_hi=32, hq=32, hkv=8,
              head_dim=128, prefix_lo=1, prefix_hi=300),
    W.AttnCfg("qsplit_d64", seed=139, batch=30, kept=None, k_lo=10, k_hi=32, hq=32, hkv=8,
              head_dim=64, prefix_lo=1, prefix_hi=150),
    W.AttnCfg("many_items", seed=140, batch=600, kept=None, k_lo=0, k_hi=12, hq=32, hkv=8,
              head_dim=128, prefix_lo=1, prefix_hi=200),
    W.AttnCfg("block64", seed=141, batch=5, kept=None, k_lo=1, k_hi=20, hq=16, hkv=4,
              head_dim=128, prefix_lo=1, prefix_hi=100, block=64),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
@pytest.mark.parametrize("ordered", [False, True], ids=["index_order", "longest_first"])
def test_fused_edge_cases(cfg, ordered):
    _fused(cfg, ordered)


@pytest.mark.parametrize("cfg", [CASES[1], CASES[2], CASES[7]], ids=["across_tiles", "some_empty",
                                                                    "qsplit"])
def test_fused_block_anywhere_in_sequence(cfg):
    """The written block starts at any position of the sequence, not only after the prefix."""
    _fused(cfg, True, anywhere=True)


def test_fused_b256_full_size():
    """Batch 256, 8 kept rows, prefixes 256..2048 + 32: every cache row bitwise, 512 sampled
    output rows against the oracle."""
    _fused(W.ATTN_B256, True, sample=512)


PAGED = [
    (W.ATTN_B256, 64),
    (W.AttnCfg("paged_small", seed=151, batch=9, kept=None, k_lo=0, k_hi=12, hq=32, hkv=8,
               head_dim=128, prefix_lo=1, prefix_hi=300), 8),
    (W.AttnCfg("paged_qsplit", seed=152, batch=60, kept=None, k_lo=4, k_hi=32, hq=32, hkv=8,
               head_dim=128, prefix_lo=10, prefix_hi=400), 16),
    (W.AttnCfg("paged_f32_d64", seed=153, batch=7, kept=None, k_lo=1, k_hi=8, hq=16, hkv=4,
               head_dim=64, dtype=W.F32, prefix_lo=1, prefix_hi=120), 8),
    (W.AttnCfg("paged_long_table", seed=154, batch=3, kept=5, hq=8, hkv=2, head_dim=128,
               prefix_lo=16600, prefix_hi=17000), 8),
]


@pytest.mark.parametrize("cfg,page", PAGED, ids=[f"{c.name}-p{p}" for c, p in PAGED])
def test_fused_paged(cfg, page):
    """Paged fused call vs paged scatter + paged attention over a shuffled pool, bitwise."""
    bte = _bte()
    ai = W.attention_inputs(cfg)
    g = dev(ai)
    bt_np, src, n_pages = page_table(ai["kv_len"].numpy(), page, seed=cfg.seed)
    bt = torch.from_numpy(bt_np).cuda()
    say(f"fused paged {cfg.name} page={page}")
    pk, pv = pool(g["cache_k"], src, n_pages, page), pool(g["cache_v"], src, n_pages, page)
    pb = ai["prefix"].to(torch.int32).cuda()
    order = bte.attention_order(g["kv_len"])
    pk_u, pv_u = pk.clone(), pv.clone()
    bte.kv_scatter_paged(g["new_k"], g["new_v"], g["idx"], g["count"], g["cu"], pb, bt, page,
                         pk_u, pv_u)
    out_u = bte.reduced_attention_paged(g["q"], g["count"], g["cu"], pk_u, pv_u, bt, page,
                                        g["kv_len"], ai["k_max"], order=order)
    pk_f, pv_f = pk.clone(), pv.clone()
    out_f = bte.kv_scatter_attention_paged(g["q"], g["count"], g["cu"], g["idx"], cfg.block, pb,
                                           g["new_k"], g["new_v"], pk_f, pv_f, bt, page,
                                           g["kv_len"], ai["k_max"], order=order)
    torch.cuda.synchronize()
    n = int(ai["cu"][-1])
    assert torch.equal(_bits(out_f[:n]), _bits(out_u[:n]))
    assert torch.equal(_bits(pk_f), _bits(pk_u)) and torch.equal(_bits(pv_f), _bits(pv_u))
