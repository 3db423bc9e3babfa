"""GPU parity: reduced-query attention and the ES-dLLM score vs the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import order_ref
import workloads as W
from helpers import assert_close, dev, say

pytestmark = pytest.mark.gpu


def _bte():
    import block_token_eviction_amd as bte
    return bte


def _attn(cfg, ai=None, rows=None, ordered=False):
    bte = _bte()
    ai = ai if ai is not None else W.attention_inputs(cfg)
    g = dev(ai)
    say(f"attention {cfg.name} batch={cfg.batch} hq={cfg.hq} hkv={cfg.hkv} D={cfg.head_dim} "
        f"k_max={ai['k_max']} ordered={ordered}")
    order = bte.attention_order(g["kv_len"]) if ordered else None
    out = bte.reduced_attention(g["q"], g["count"], g["cu"], g["cache_k"], g["cache_v"],
                                g["seq_start"], g["kv_len"], ai["k_max"], order=order)
    torch.cuda.synchronize()
    f64 = W.to_f64
    ref = oracle.reduced_attention(f64(ai["q"]), ai["count"].numpy(), ai["cu"].numpy(),
                                   f64(ai["cache_k"]), f64(ai["cache_v"]), ai["seq_start"].numpy(),
                                   ai["kv_len"].numpy(), cfg.hq, cfg.hkv,
                                   1.0 / math.sqrt(cfg.head_dim), rows=rows)
    n = int(ai["cu"][-1])
    got = out[:n].cpu().to(torch.float64).numpy()
    sel = np.arange(n) if rows is None else np.asarray(rows)
    assert_close(got[sel], ref[:n][sel], cfg.name)


def test_tiny_fp32():
    _attn(W.TINY_ATTN)


def test_attn_b256_full_size():
    """Batch 256, 8 kept rows, prefixes 256..2048 + 32: every output row."""
    _attn(W.ATTN_B256)


CASES = [
    W.AttnCfg("len1", seed=31, batch=3, kept=1, hq=8, hkv=2, head_dim=128, prefix_lo=0, prefix_hi=0, block=1),
    W.AttnCfg("partial_tiles", seed=32, batch=6, kept=5, hq=8, hkv=2, head_dim=128, prefix_lo=1, prefix_hi=70),
    W.AttnCfg("two_row_tiles", seed=33, batch=7, kept=None, k_lo=0, k_hi=12, hq=32, hkv=8,
              head_dim=128, prefix_lo=90, prefix_hi=500),
    W.AttnCfg("no_gqa", seed=34, batch=4, kept=6, hq=8, hkv=8, head_dim=128, prefix_lo=100, prefix_hi=300),
    W.AttnCfg("d64", seed=35, batch=4, kept=7, hq=16, hkv=4, head_dim=64, prefix_lo=33, prefix_hi=400),
    W.AttnCfg("f32_d128", seed=36, batch=3, kept=4, hq=8, hkv=2, head_dim=128, dtype=W.F32,
              prefix_lo=60, prefix_hi=200),
    W.AttnCfg("rows_beyond_64", seed=37, batch=3, kept=20, hq=16, hkv=4, head_dim=128,
              prefix_lo=40, prefix_hi=130),
    # fp32 takes 32-row groups: 80 rows per KV head are three of them
    W.AttnCfg("f32_rows_beyond_64", seed=40, batch=3, kept=20, hq=16, hkv=4, head_dim=128,
              dtype=W.F32, prefix_lo=40, prefix_hi=130),
    W.AttnCfg("long", seed=38, batch=2, kept=3, hq=8, hkv=2, head_dim=128, prefix_lo=8000, prefix_hi=9000),
    # sequences of about 131K positions: over 4,000 key tiles per item
    W.AttnCfg("very_long", seed=39, batch=2, kept=2, hq=8, hkv=2, head_dim=128, prefix_lo=130000,
              prefix_hi=131040),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
@pytest.mark.parametrize("ordered", [False, True], ids=["index_order", "longest_first"])
def test_attention_edge_cases(cfg, ordered):
    _attn(cfg, ordered=ordered)


# Enough (sequence, KV head) items that the launch takes two waves per item
# (the smaller cases above take four); budgets up to 12 or 16 kept rows give
# workgroups of one and of two 32-row query tiles. Short prefixes keep the
# float64 oracle fast.
MANY = [
    W.AttnCfg("many_items", seed=61, batch=600, kept=None, k_lo=0, k_hi=12, hq=32, hkv=8,
              head_dim=128, prefix_lo=1, prefix_hi=200),
    W.AttnCfg("many_items_d64", seed=62, batch=520, kept=None, k_lo=1, k_hi=16, hq=32, hkv=8,
              head_dim=64, prefix_lo=30, prefix_hi=90),
]


@pytest.mark.parametrize("cfg", MANY, ids=[c.name for c in MANY])
@pytest.mark.parametrize("ordered", [False, True], ids=["index_order", "longest_first"])
def test_attention_many_items(cfg, ordered):
    _attn(cfg, ordered=ordered)


# More than 64 query rows per KV head (k_max * G > 64): four-wave workgroups over
# 128-row groups, whose waves take 32 rows each and share one LDS ring of key
# tiles; waves past a group's last row only copy. Budgets 0..32 give groups with
# one to four busy waves in one launch; with G = 8 a sequence has up to 256
# rows (a second row group). Sequences of one to three key tiles are shorter
# than the ring's lead (the prologue repeats the last tile).
QSPLIT = [
    W.AttnCfg("qsplit_mixed", seed=64, batch=300, kept=None, k_lo=0, k_hi=32, hq=32, hkv=8,
              head_dim=128, prefix_lo=1, prefix_hi=300),
    W.AttnCfg("qsplit_g8", seed=65, batch=120, kept=None, k_lo=1, k_hi=32, hq=32, hkv=4,
              head_dim=128, prefix_lo=20, prefix_hi=260),
    W.AttnCfg("qsplit_d64", seed=66, batch=200, kept=None, k_lo=10, k_hi=32, hq=32, hkv=8,
              head_dim=64, prefix_lo=1, prefix_hi=150),
    W.AttnCfg("qsplit_short", seed=67, batch=60, kept=None, k_lo=17, k_hi=32, hq=32, hkv=8,
              head_dim=128, prefix_lo=0, prefix_hi=64),
    # fewer than four KV heads: the row group is the slowest grid dimension
    W.AttnCfg("qsplit_hkv2", seed=68, batch=50, kept=None, k_lo=9, k_hi=32, hq=16, hkv=2,
              head_dim=128, prefix_lo=10, prefix_hi=200),
    W.AttnCfg("qsplit_hkv1", seed=69, batch=40, kept=None, k_lo=0, k_hi=32, hq=8, hkv=1,
              head_dim=64, prefix_lo=10, prefix_hi=200),
    # more than eight KV heads (a sequence's workgroups span two rounds of the XCDs)
    W.AttnCfg("qsplit_hkv16", seed=70, batch=30, kept=None, k_lo=12, k_hi=32, hq=64, hkv=16,
              head_dim=128, prefix_lo=10, prefix_hi=300),
    # many short items: 3,000 sequences over 24,000 query-split workgroups
    W.AttnCfg("qsplit_many", seed=71, batch=3000, kept=None, k_lo=10, k_hi=24, hq=32, hkv=8,
              head_dim=128, prefix_lo=1, prefix_hi=40),
]


@pytest.mark.parametrize("cfg", QSPLIT, ids=[c.name for c in QSPLIT])
@pytest.mark.parametrize("ordered", [False, True], ids=["index_order", "longest_first"])
def test_attention_query_split(cfg, ordered):
    _attn(cfg, ordered=ordered)


@pytest.mark.parametrize("batch", [1, 7, 64, 65, 1000, 1024, 2000, 3000, 5000, 16384])
def test_attention_order_matches_oracle(batch):
    bte = _bte()
    lens = np.random.default_rng(batch).integers(-3, 300, batch).astype(np.int32)   # ties, negatives
    say(f"attention_order batch={batch}")
    got = bte.attention_order(torch.from_numpy(lens).cuda()).cpu().numpy()
    np.testing.assert_array_equal(got, order_ref.attention_order(lens))


@pytest.mark.parametrize("batch", [1, 65, 1024, 5000, 16384])
def test_attention_order_by_work_matches_oracle(batch):
    """Kept counts 0..32 with group 4: up to two 64-row query passes; ties, zero counts,
    negative lengths."""
    bte = _bte()
    r = np.random.default_rng(batch + 7)
    lens = r.integers(-3, 300, batch).astype(np.int32)
    cnt = r.integers(0, 33, batch).astype(np.int32)
    say(f"attention_order by work batch={batch}")
    got = bte.attention_order(torch.from_numpy(lens).cuda(), count=torch.from_numpy(cnt).cuda(),
                              group=4).cpu().numpy()
    np.testing.assert_array_equal(got, order_ref.attention_order(lens, count=cnt, group=4))


@pytest.mark.parametrize("lens,cnt,group", [
    ([5, 0, 7, 2 ** 31 - 1], [2 ** 31 - 1, 2 ** 31 - 1, 1, 3], 2 ** 31 - 1),   # > 2^32 passes
    ([2 ** 31 - 1, 2 ** 30, 9], [32, 64, 1], 2 ** 20),                         # product capped
])
def test_attention_order_by_work_saturates(lens, cnt, group):
    bte = _bte()
    lens, cnt = np.array(lens, np.int32), np.array(cnt, np.int32)
    say(f"attention_order saturation lens={lens.tolist()} cnt={cnt.tolist()} group={group}")
    got = bte.attention_order(torch.from_numpy(lens).cuda(), count=torch.from_numpy(cnt).cuda(),
                              group=group).cpu().numpy()
    np.testing.assert_array_equal(got, order_ref.attention_order(lens, count=cnt, group=group))


def test_attention_order_only_schedules():
    """Two different orders (same launch shape) give bit-identical outputs."""
    bte = _bte()
    cfg = W.AttnCfg("perm", seed=63, batch=300, kept=None, k_lo=2, k_hi=12, prefix_lo=10,
                    prefix_hi=400)
    ai = W.attention_inputs(cfg)
    g = dev(ai)
    say("attention order invariance")
    lpt = bte.attention_order(g["kv_len"])
    perm = torch.from_numpy(np.random.default_rng(5).permutation(cfg.batch).astype(np.int32)).cuda()
    outs = [bte.reduced_attention(g["q"], g["count"], g["cu"], g["cache_k"], g["cache_v"],
                                  g["seq_start"], g["kv_len"], ai["k_max"], order=o)
            for o in (lpt, perm)]
    n = int(ai["cu"][-1])
    assert torch.equal(outs[0][:n], outs[1][:n])


def test_attention_kv_len_one_is_v0_exactly():
    bte = _bte()
    ai = W.attention_inputs(W.AttnCfg("one", seed=39, batch=4, kept=1, hq=8, hkv=2, head_dim=128,
                                      prefix_lo=0, prefix_hi=0, block=1))
    # every sequence holds one key: out must equal that V row bit for bit (bf16)
    g = dev(ai)
    say("attention kv_len=1")
    out = bte.reduced_attention(g["q"], g["count"], g["cu"], g["cache_k"], g["cache_v"],
                                g["seq_start"], g["kv_len"], 1).cpu()
    for b in range(4):
        v = ai["cache_v"][int(ai["seq_start"][b])]                       # [hkv, D]
        want = v.repeat_interleave(4, dim=0)
        assert torch.equal(out[b], want)


def _es(cfg, ei=None):
    bte = _bte()
    ei = ei if ei is not None else W.esdllm_inputs(cfg)
    g = dev(ei)
    say(f"esdllm {cfg.name}")
    out = bte.esdllm_score(g["h_new"], g["h_prev"], g["surv_pos"], g["conf"], ei["alpha"])
    torch.cuda.synchronize()
    ref = oracle.esdllm_score(W.to_f64(ei["h_new"]), W.to_f64(ei["h_prev"]), ei["surv_pos"].numpy(),
                              ei["conf"].numpy(), ei["alpha"])
    return out.cpu().numpy(), ref, ei


def test_esdllm_b8_full_size_and_exact_copy_rows():
    got, ref, ei = _es(W.ES_B8)
    assert_close(got, ref, "esdllm_b8")
    same = ~ei["perturbed"].numpy()
    c = np.take_along_axis(ei["conf"].numpy(), ei["surv_pos"].numpy(), 1)
    assert np.array_equal(got[same], (np.float32(0.5) * c[same]).astype(np.float32))


def test_esdllm_closed_form_and_scale_invariance():
    bte = _bte()
    h = 4096
    h_prev = torch.ones((1, 3, h), dtype=torch.bfloat16)
    h_new = torch.ones((1, 1, h), dtype=torch.bfloat16); h_new[0, 0, 123] = 1.5
    pos = torch.tensor([[2]], dtype=torch.int32)
    conf = torch.zeros((1, 3))
    say("esdllm closed form")
    s = bte.esdllm_score(h_new.cuda(), h_prev.cuda(), pos.cuda(), conf.cuda(), 0.0).cpu()
    assert s.item() == 2.0 ** -13
    cfg = W.EsCfg("scale", seed=41, batch=2, prompt=8, generated=64, hidden=512, keep=32)
    ei = W.esdllm_inputs(cfg)
    g = dev(ei)
    a = bte.esdllm_score(g["h_new"], g["h_prev"], g["surv_pos"], g["conf"], 0.3)
    b = bte.esdllm_score(g["h_new"] * 2, g["h_prev"] * 2, g["surv_pos"], g["conf"], 0.3)
    assert torch.equal(a, b)


def test_esdllm_fp32_and_odd_sizes():
    cfg = W.EsCfg("f32", seed=42, batch=3, prompt=5, generated=37, hidden=200, dtype=W.F32, keep=10)
    got, ref, _ = _es(cfg)
    assert_close(got, ref, "esdllm f32")


def test_esdllm_two_skip_layers():
    """ES-dLLM skip layers at 1/8 and 1/4 depth (r = 0.5 each) on the batch-8
    workload: 256 -> 128 -> 64 survivors. Per layer: scores within tolerance of
    the oracle; the selection equal to the oracle's top-K of the same fp32
    scores; kept rows, survivor positions and the updated hidden cache bit
    for bit."""
    from block_token_eviction_amd.chain import EsSkipLayer
    bte = _bte()
    cfg = W.ES_B8
    x = W.es_pipeline_inputs(cfg, layers=2, device="cuda")
    L = cfg.prompt + cfg.generated
    bits = lambda t: t.detach().cpu().view(torch.int16).numpy()
    surv = x["surv_pos"]
    n = surv.shape[1]
    # this layer's survivor states, standing in for the model's layers before it
    one = torch.arange(cfg.batch + 1, dtype=torch.int32, device="cuda")
    for layer in range(2):
        keep = n // 2
        h_surv = bte.gather_rows(x["h_cur"][layer], surv, torch.full((cfg.batch,), n, dtype=torch.int32,
                                 device="cuda"), one * n).view(cfg.batch, n, -1)
        cache0 = bits(x["h_cache"][layer])                 # before the in-place update
        cache0_f64 = W.to_f64(x["h_cache"][layer])
        say(f"es skip layer {layer}: {n} -> {keep}")
        step = EsSkipLayer(cfg.batch, n, keep, L, cfg.hidden, cfg.dtype, "cuda")
        h_next, s_next = step.run(h_surv, x["h_cache"][layer], surv, x["conf"], x["alpha"])
        torch.cuda.synchronize()
        ref_score = oracle.esdllm_score(W.to_f64(h_surv), cache0_f64, surv.cpu().numpy(),
                                        x["conf"].cpu().numpy(), x["alpha"])
        assert_close(step.score.cpu().numpy(), ref_score, f"es score layer {layer}")
        g_score = step.score.cpu().numpy()
        r_idx, r_cnt, r_cu = oracle.topk_select(g_score, np.full(cfg.batch, keep), keep)
        np.testing.assert_array_equal(step.idx.cpu().numpy(), r_idx)
        np.testing.assert_array_equal(bits(h_next).reshape(cfg.batch * keep, -1),
                                      oracle.gather_rows(bits(h_surv), r_idx, r_cnt, r_cu))
        want_s = np.take_along_axis(surv.cpu().numpy(), r_idx, axis=1)
        np.testing.assert_array_equal(s_next.cpu().numpy(), want_s)
        rows = bits(h_surv).reshape(cfg.batch * n, -1)
        ident = np.tile(np.arange(n, dtype=np.int32), (cfg.batch, 1))
        want_cache, _ = oracle.kv_scatter(rows, rows, ident, np.full(cfg.batch, n, np.int32),
                                          np.arange(cfg.batch + 1, dtype=np.int32) * n,
                                          np.arange(cfg.batch) * L, cache0.reshape(cfg.batch * L, -1),
                                          cache0.reshape(cfg.batch * L, -1), pos_map=surv.cpu().numpy())
        np.testing.assert_array_equal(bits(x["h_cache"][layer]).reshape(cfg.batch * L, -1), want_cache)
        surv, n = s_next.contiguous(), keep
    assert n == cfg.generated // 4


def test_es_step_graph_replays_match_eager():
    """The ES-dLLM step (score, top-K, gather, scatter at the batch-8 workload) captured in
    a HIP graph and replayed three times, with the cache restored eagerly in between:
    every replay equals the eager step bit for bit."""
    from block_token_eviction_amd.chain import EsStep
    cfg = W.ES_B8
    ei = dev(W.esdllm_inputs(cfg))
    say("ES-dLLM step under graph capture")
    step = EsStep(cfg.batch, cfg.generated, cfg.hidden, cfg.keep, cfg.dtype, "cuda")
    args = dict(h_new=ei["h_new"], h_prev=ei["h_prev"], surv_pos=ei["surv_pos"], conf=ei["conf"],
                alpha=ei["alpha"], k=ei["k"], new_k=ei["new_k"], new_v=ei["new_v"],
                row_base=ei["row_base"], cache_k=ei["cache_k"], cache_v=ei["cache_v"])
    cache0 = (ei["cache_k"].clone(), ei["cache_v"].clone())
    step.run(**args)
    torch.cuda.synchronize()
    n = int(step.cu[-1])
    outs = lambda: [step.score, step.idx, step.count, step.cu, step.gathered[:n], ei["cache_k"],
                    ei["cache_v"]]
    want = [t.clone() for t in outs()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run(**args)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run(**args)
    for rep in range(3):
        ei["cache_k"].copy_(cache0[0])
        ei["cache_v"].copy_(cache0[1])
        step.gathered.zero_()
        step.score.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), want):
            assert torch.equal(a, b), f"replay {rep}"
