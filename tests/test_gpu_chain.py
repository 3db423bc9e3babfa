"""GPU parity of the whole FOCUS step at the batch-1024 workload, in the launch
configuration bench.py times (FocusStep on one stream), checked against the
oracle on every sequence: the delta, the selection, the gather, the KV cache
and the attention outputs. Also a small chain.""" 
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.chain as oc
import workloads as W
from helpers import assert_close, say, selection_valid

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _check_chain(fc, ac, attn_sample, device="cuda", fused=False):
    """Every sequence: delta to tolerance, a valid selection, and, where the kept set equals
    the oracle's own, the gathered rows and the scattered block rows bit for bit; the rest
    of both caches unchanged (compared on the device against a copy taken before the step).
    attn_sample: the sequences whose attention output is checked against the oracle."""
    from block_token_eviction_amd.chain import FocusStep
    say(f"chain {fc.name} batch={fc.batch} attention sample={len(attn_sample)} fused={fused}")
    x = W.chain_inputs(fc, ac, device=device)
    seq_start = x["seq_start"].cpu().numpy()
    kv_len = x["kv_len"].cpu().numpy()
    block_rows = torch.from_numpy((x["row_base"].cpu().numpy()[:, None]
                                   + np.arange(fc.block)[None, :]).reshape(-1)).to(device)
    pre_k, pre_v = x["cache_k"].clone(), x["cache_v"].clone()
    blk_k0 = _bits(x["cache_k"][block_rows]).reshape(fc.batch, fc.block, -1)
    blk_v0 = _bits(x["cache_v"][block_rows]).reshape(fc.batch, fc.block, -1)
    step = FocusStep(fc.batch, fc.block, fc.hidden, fc.hq, fc.head_dim, fc.k_hi, fc.dtype, device,
                     hkv=fc.hkv)
    step.run(q0=x["q0"], k0=x["k0"], q1=x["q1"], k1=x["k1"], decoded=x["decoded"], k=x["k"],
             hidden_rows=x["hidden_rows"], pool_kernel=fc.pool_kernel, new_k=x["new_k"],
             new_v=x["new_v"], q_kept=x["q_kept"], cache_k=x["cache_k"], cache_v=x["cache_v"],
             seq_start=x["seq_start"], kv_len=x["kv_len"], row_base=x["row_base"],
             pos_base=x["prefix"].to(torch.int32), fused=fused)
    torch.cuda.synchronize()
    # rows outside every block are untouched (on the device: the caches are GBs)
    outside = torch.ones(x["cache_k"].shape[0], dtype=torch.bool, device=device)
    outside[block_rows] = False
    assert torch.equal(x["cache_k"][outside], pre_k[outside])
    assert torch.equal(x["cache_v"][outside], pre_v[outside])
    del pre_k, pre_v, outside
    g_delta = step.delta.cpu().numpy()
    g_idx, g_cnt, g_cu = step.idx.cpu().numpy(), step.count.cpu().numpy(), step.cu.cpu().numpy()
    assert g_cu[0] == 0 and np.array_equal(np.diff(g_cu), g_cnt)
    ref_delta = oracle.focus_importance_delta(_f64(x["q0"]), _f64(x["k0"]), _f64(x["q1"]),
                                              _f64(x["k1"]), x["decoded"].cpu().numpy(), fc.hq,
                                              fc.hkv, fc.pool_kernel)
    assert_close(g_delta, ref_delta, "delta")
    k_host = x["k"].cpu().numpy()
    differ = selection_valid(g_idx, g_cnt, ref_delta, k_host, fc.k_hi)
    assert len(differ) <= max(2, fc.batch // 50), f"near-tie selections on {len(differ)} rows"
    # Downstream of the selection: sequences whose kept set equals the oracle's own.
    r_idx, r_cnt, _ = oracle.topk_select(ref_delta, k_host, fc.k_hi)
    hid = _bits(x["hidden_rows"])
    gathered = _bits(step.gathered)
    blk_k, blk_v = (_bits(x[c][block_rows]).reshape(fc.batch, fc.block, -1)
                    for c in ("cache_k", "cache_v"))
    new_k, new_v = _bits(x["new_k"]), _bits(x["new_v"])
    zero = np.zeros(1, np.int64)
    checked = 0
    for b in range(fc.batch):
        if b in differ:
            continue
        n_b, cub = int(r_cnt[b]), int(g_cu[b])
        one = np.array([n_b], np.int32)
        ocu = np.array([0, n_b], np.int32)
        ridx = r_idx[b:b + 1]
        np.testing.assert_array_equal(gathered[cub:cub + n_b],
                                      oracle.gather_rows(hid[b:b + 1], ridx, one, ocu))
        rk, rv = oracle.kv_scatter(new_k[cub:cub + n_b], new_v[cub:cub + n_b], ridx, one, ocu,
                                   zero, blk_k0[b], blk_v0[b])
        np.testing.assert_array_equal(blk_k[b], rk)
        np.testing.assert_array_equal(blk_v[b], rv)
        checked += 1
    assert checked == fc.batch - len(differ)
    for b in attn_sample:
        if b in differ:
            continue
        n_b, cub = int(r_cnt[b]), int(g_cu[b])
        r0, r1 = int(seq_start[b]), int(seq_start[b] + kv_len[b])
        ck, cv = _bits(x["cache_k"][r0:r1]), _bits(x["cache_v"][r0:r1])
        ref_o = oracle.reduced_attention(oc.bf16_bits_to_f64(_bits(x["q_kept"][cub:cub + n_b])),
                                         np.array([n_b]), np.array([0, n_b]),
                                         oc.bf16_bits_to_f64(ck), oc.bf16_bits_to_f64(cv),
                                         np.array([0]), np.array([kv_len[b]]), fc.hq, fc.hkv,
                                         1.0 / math.sqrt(fc.head_dim))
        assert_close(_f64(step.out[cub:cub + n_b]), ref_o, f"attention seq {b}")
    return differ


FUSED = pytest.mark.parametrize("fused", [False, True], ids=["scatter_then_attention",
                                                              "fused_scatter_attention"])


@FUSED
def test_chain_small_every_sequence(fused):
    fc = W.FocusCfg("chain_small", seed=51, batch=48)
    ac = W.AttnCfg("chain_small", seed=51, batch=48, kept=None, prefix_lo=40, prefix_hi=700)
    _check_chain(fc, ac, list(range(48)), fused=fused)


@FUSED
def test_chain_b1024_full_size(fused):
    """The benchmarked workload itself (batch 1024, prefixes 1024..4096): every sequence's
    delta, selection, gathered rows, cache rows and attention outputs."""
    _check_chain(W.CHAIN_FOCUS_B1024, W.CHAIN_ATTN_B1024, list(range(1024)), fused=fused)


@FUSED
def test_chain_b1024_block64_full_size(fused):
    """The whole step at blocks of 64 as bench.py's chain_b1024_block64 leg runs it (batch
    1024, K ~ U{8..24}, prefixes 1024..4096 + 64): every sequence's delta, selection,
    gathered rows and cache rows; the attention of every 8th sequence, about 40 % of which
    have more than 64 query rows per KV head (query-split workgroups)."""
    fc = W.FocusCfg("chain_b1024_block64", seed=8, batch=1024, block=64, k_lo=8, k_hi=24)
    ac = W.AttnCfg("chain_b1024_block64", seed=8, batch=1024, kept=None, k_lo=8, k_hi=24,
                   block=64, prefix_lo=1024, prefix_hi=4096)
    _check_chain(fc, ac, list(range(0, 1024, 8)), fused=fused)


@FUSED
@pytest.mark.parametrize("block", [32, 64], ids=["block32", "block64_query_split"])
def test_focus_step_graph_replays_match_eager(fused, block):
    """A FOCUS step captured in a HIP graph and replayed three times, with eager
    work and synchronisations in between: every replay equals the eager step
    bit for bit (the kernels allocate nothing and record no memset nodes). At
    blocks of 64 (budgets 8..24) the delta takes its 64-key kernel and the
    attention its query-split workgroups."""
    from block_token_eviction_amd.chain import FocusStep
    k_lo, k_hi = (4, 12) if block == 32 else (8, 24)
    fc = W.FocusCfg("graph", seed=81, batch=64, block=block, k_lo=k_lo, k_hi=k_hi)
    ac = W.AttnCfg("graph", seed=81, batch=64, kept=None, k_lo=k_lo, k_hi=k_hi, block=block,
                   prefix_lo=100, prefix_hi=600)
    say(f"focus step under graph capture fused={fused} block={block}")
    x = W.chain_inputs(fc, ac, device="cuda")
    step = FocusStep(fc.batch, fc.block, fc.hidden, fc.hq, fc.head_dim, fc.k_hi, fc.dtype, "cuda",
                     hkv=fc.hkv)
    args = {k: x[k] for k in ("q0", "k0", "q1", "k1", "decoded", "k", "hidden_rows", "pool_kernel",
                              "new_k", "new_v", "q_kept", "cache_k", "cache_v", "seq_start",
                              "kv_len", "row_base")}
    args.update(pos_base=x["prefix"].to(torch.int32), fused=fused)
    cache0 = (x["cache_k"].clone(), x["cache_v"].clone())
    step.run(**args)
    torch.cuda.synchronize()
    n = int(step.cu[-1])                                   # rows the step writes
    want = [t.clone() for t in (step.delta, step.idx, step.count, step.cu, step.gathered[:n],
                                step.out[:n], x["cache_k"], x["cache_v"])]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                              # warm-up on the capture stream
        step.run(**args)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run(**args)
    for rep in range(3):
        x["cache_k"].copy_(cache0[0])                      # eager work between replays
        x["cache_v"].copy_(cache0[1])
        step.out.zero_()
        step.gathered.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (step.delta, step.idx, step.count, step.cu, step.gathered[:n], step.out[:n],
               x["cache_k"], x["cache_v"])
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep}"
