"""With BTE_CHECK=1 the binding validates the device-data contract on the host:
valid calls give the same results as without it, and a violating call raises
ContractError before anything is launched (the bad input never reaches a
kernel)."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import dev, say

pytestmark = pytest.mark.gpu


def _bte():
    import block_token_eviction_amd as bte
    return bte


def test_checked_calls_match_and_violations_raise(monkeypatch):
    bte = _bte()
    cfg = W.AttnCfg("contract", seed=91, batch=12, kept=None, k_lo=0, k_hi=12, prefix_lo=5,
                    prefix_hi=200)
    ai = W.attention_inputs(cfg)
    g = dev(ai)
    say("contract checks through the binding")
    src = torch.randn(cfg.batch, cfg.block, 256, device="cuda").to(torch.bfloat16)
    plain = bte.gather_rows(src, g["idx"], g["count"], g["cu"])
    att = bte.reduced_attention(g["q"], g["count"], g["cu"], g["cache_k"], g["cache_v"],
                                g["seq_start"], g["kv_len"], ai["k_max"])
    monkeypatch.setenv("BTE_CHECK", "1")
    n = int(ai["cu"][-1])
    assert torch.equal(bte.gather_rows(src, g["idx"], g["count"], g["cu"])[:n], plain[:n])
    att2 = bte.reduced_attention(g["q"], g["count"], g["cu"], g["cache_k"], g["cache_v"],
                                 g["seq_start"], g["kv_len"], ai["k_max"])
    assert torch.equal(att2[:n], att[:n])

    # an index past the block: caught on the host
    bad = ai["idx"].clone()
    b = int(np.flatnonzero(ai["count"].numpy() > 0)[0])
    bad[b, int(ai["count"][b]) - 1] = cfg.block
    with pytest.raises(bte.contract.ContractError):
        bte.gather_rows(src, bad.cuda(), g["count"], g["cu"])
    # a sequence whose KV rows run past the cache
    ss = ai["seq_start"].clone()
    ss[b] = ai["rows"]
    with pytest.raises(bte.contract.ContractError):
        bte.reduced_attention(g["q"], g["count"], g["cu"], g["cache_k"], g["cache_v"], ss.cuda(),
                              g["kv_len"], ai["k_max"])
    # kept rows scattered past the end of the cache
    rb = ai["row_base"].clone()
    rb[b] = ai["rows"]
    with pytest.raises(bte.contract.ContractError):
        bte.kv_scatter(g["new_k"], g["new_v"], g["idx"], g["count"], g["cu"], rb.cuda(),
                       g["cache_k"].clone(), g["cache_v"].clone())


def test_checked_fused_scatter_attention(monkeypatch):
    """The fused scatter + attention under BTE_CHECK=1: a valid call equals the unchecked
    one (output and caches); a block position past kv_len and an index outside the block
    raise before launching, leaving the caches untouched."""
    bte = _bte()
    cfg = W.AttnCfg("contract_fused", seed=92, batch=12, kept=None, k_lo=0, k_hi=12,
                    prefix_lo=5, prefix_hi=200)
    ai = W.attention_inputs(cfg)
    g = dev(ai)
    say("contract checks of the fused scatter + attention")
    pb = ai["prefix"].to(torch.int32).cuda()
    ck, cv = g["cache_k"].clone(), g["cache_v"].clone()
    out = bte.kv_scatter_attention(g["q"], g["count"], g["cu"], g["idx"], cfg.block, pb,
                                   g["new_k"], g["new_v"], ck, cv, g["seq_start"], g["kv_len"],
                                   ai["k_max"])
    monkeypatch.setenv("BTE_CHECK", "1")
    ck2, cv2 = g["cache_k"].clone(), g["cache_v"].clone()
    out2 = bte.kv_scatter_attention(g["q"], g["count"], g["cu"], g["idx"], cfg.block, pb,
                                    g["new_k"], g["new_v"], ck2, cv2, g["seq_start"], g["kv_len"],
                                    ai["k_max"])
    n = int(ai["cu"][-1])
    assert torch.equal(out2[:n], out[:n]) and torch.equal(ck2, ck) and torch.equal(cv2, cv)
    b = int(np.flatnonzero(ai["count"].numpy() > 0)[0])
    ck3, cv3 = g["cache_k"].clone(), g["cache_v"].clone()
    late = pb.clone()
    late[b] = int(ai["kv_len"][b])                         # every kept position at or past kv_len
    bad_idx = ai["idx"].clone()
    bad_idx[b, int(ai["count"][b]) - 1] = cfg.block        # outside [0, n)
    for kw in (dict(pos_base=late, idx=g["idx"]), dict(pos_base=pb, idx=bad_idx.cuda())):
        with pytest.raises(bte.contract.ContractError):
            bte.kv_scatter_attention(g["q"], g["count"], g["cu"], kw["idx"], cfg.block,
                                     kw["pos_base"], g["new_k"], g["new_v"], ck3, cv3,
                                     g["seq_start"], g["kv_len"], ai["k_max"])
    torch.cuda.synchronize()
    assert torch.equal(ck3, g["cache_k"]) and torch.equal(cv3, g["cache_v"])


def test_binding_rejects_wrong_index_dtypes_and_shapes():
    """Index tensors must be int32 (an int64 tensor would be read as pairs of int32) and
    caller-supplied outputs must have the documented shapes: ValueError before any launch."""
    import block_token_eviction_amd as bte
    say("binding argument checks")
    dev = "cuda"
    scores = torch.randn((4, 32), device=dev)
    k = torch.full((4,), 3, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        bte.topk_select(scores, k.long(), 8)
    with pytest.raises(ValueError):
        bte.topk_select(scores, k, 8, idx=torch.empty((4, 4), dtype=torch.int32, device=dev))
    with pytest.raises(ValueError):
        bte.topk_select(scores, k, 8, cu=torch.empty((4,), dtype=torch.int32, device=dev))
    idx, count, cu = bte.topk_select(scores, k, 8)
    src = torch.randn((4, 32, 64), device=dev)
    with pytest.raises(ValueError):
        bte.gather_rows(src, idx.long(), count, cu)
    with pytest.raises(ValueError):
        bte.gather_rows(src, idx, count.long(), cu)
    with pytest.raises(ValueError):
        bte.gather_rows(src, idx, count, cu, out=torch.empty((32, 32), device=dev))
    cache = torch.randn((200, 2, 64), device=dev)
    new = torch.randn((32, 2, 64), device=dev)
    rb = torch.arange(4, dtype=torch.int64, device=dev) * 40
    with pytest.raises(ValueError):
        bte.kv_scatter(new, new, idx, count, cu, rb.int(), cache, cache.clone())
    with pytest.raises(ValueError):
        bte.kv_scatter(new, new, idx, count, cu.long(), rb, cache, cache.clone())
    q = torch.randn((32, 4, 64), device=dev)
    kv_len = torch.full((4,), 40, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        bte.reduced_attention(q, count, cu, cache, cache, rb, kv_len.long(), 8)
    with pytest.raises(ValueError):
        bte.reduced_attention(q, count, cu, cache, cache, rb, kv_len, 8,
                              out=torch.empty((32, 4, 32), device=dev))
    torch.cuda.synchronize()


def test_checked_es_calls_match_and_violations_raise(monkeypatch):
    """With BTE_CHECK=1 the fused ES score/update and the ragged gather give what the
    unchecked calls give, and repeated survivor positions or out-of-range source rows
    raise before launching (the caches stay untouched)."""
    import block_token_eviction_amd as bte
    say("checked ES calls")
    r = np.random.default_rng(71)
    batch, L, h, cap = 3, 40, 64, 8
    cache = torch.randn((batch, L, h), device="cuda")
    counts = np.array([5, 0, 8], np.int32)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    surv = torch.from_numpy(np.concatenate([np.sort(r.choice(L, size=c, replace=False))
                                            for c in counts]).astype(np.int32)).cuda()
    rows = torch.randn((int(counts.sum()), h), device="cuda")
    conf = torch.rand((batch, L), device="cuda")
    cnt = torch.from_numpy(counts).cuda()
    c1, c2 = cache.clone(), cache.clone()
    plain = bte.esdllm_score_update(rows, c1, surv, conf, 0.5, count=cnt, cu=cu, cap=cap)
    monkeypatch.setenv("BTE_CHECK", "1")
    checked = bte.esdllm_score_update(rows, c2, surv, conf, 0.5, count=cnt, cu=cu, cap=cap)
    torch.cuda.synchronize()
    assert torch.equal(plain, checked) and torch.equal(c1, c2)
    dup = surv.clone()
    dup[1] = dup[0]
    c3 = cache.clone()
    with pytest.raises(bte.contract.ContractError):
        bte.esdllm_score_update(rows, c3, dup, conf, 0.5, count=cnt, cu=cu, cap=cap)
    assert torch.equal(c3, cache)
    k = torch.tensor([2, 0, 3], dtype=torch.int32, device="cuda")
    idx, kc, kcu = bte.topk_select(plain, k, cap)
    outs = bte.gather_rows_multi_ragged([rows, surv], cu, idx, kc, kcu)
    torch.cuda.synchronize()
    with pytest.raises(bte.contract.ContractError):
        bte.gather_rows_multi_ragged([rows[:4], surv[:4]], cu, idx, kc, kcu)
    assert outs[0].shape[0] == batch * cap
