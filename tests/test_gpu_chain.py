"""GPU parity of the whole FOCUS step at the batch-1024 workload, in the launch
configuration bench.py times (FocusStep on one stream), checked on a sample of
sequences against the oracle's own chain. Also a small full-check chain."""
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


def _check_chain(fc, ac, sample, device="cuda", fused=False):
    from block_token_eviction_amd.chain import FocusStep
    say(f"chain {fc.name} batch={fc.batch} sample={len(sample)} fused={fused}")
    x = W.chain_inputs(fc, ac, device=device)
    cache_k0 = {int(b): None for b in sample}
    seq_start = x["seq_start"].cpu().numpy()
    kv_len = x["kv_len"].cpu().numpy()
    for b in sample:                         # pre-images of the sampled sequences' caches
        r0, r1 = int(seq_start[b]), int(seq_start[b] + kv_len[b])
        cache_k0[int(b)] = (_bits(x["cache_k"][r0:r1]), _bits(x["cache_v"][r0:r1]))
    step = FocusStep(fc.batch, fc.block, fc.hidden, fc.hq, fc.head_dim, fc.k_hi, fc.dtype, device,
                     hkv=fc.hkv)
    step.run(q0=x["q0"], k0=x["k0"], q1=x["q1"], k1=x["k1"], decoded=x["decoded"], k=x["k"],
             hidden_rows=x["hidden_rows"], pool_kernel=fc.pool_kernel, new_k=x["new_k"],
             new_v=x["new_v"], q_kept=x["q_kept"], cache_k=x["cache_k"], cache_v=x["cache_v"],
             seq_start=x["seq_start"], kv_len=x["kv_len"], row_base=x["row_base"],
             pos_base=x["prefix"].to(torch.int32), fused=fused)
    torch.cuda.synchronize()
    g_delta = step.delta.cpu().numpy()
    g_idx, g_cnt, g_cu = step.idx.cpu().numpy(), step.count.cpu().numpy(), step.cu.cpu().numpy()
    assert g_cu[0] == 0 and np.array_equal(np.diff(g_cu), g_cnt)
    sample = np.asarray(sample)
    ref_delta = oracle.focus_importance_delta(_f64(x["q0"][sample]), _f64(x["k0"][sample]),
                                              _f64(x["q1"][sample]), _f64(x["k1"][sample]),
                                              x["decoded"][sample].cpu().numpy(), fc.hq, fc.hkv,
                                              fc.pool_kernel)
    assert_close(g_delta[sample], ref_delta, "delta")
    k_host = x["k"].cpu().numpy()
    differ = selection_valid(g_idx[sample], g_cnt[sample], ref_delta, k_host[sample], fc.k_hi)
    assert len(differ) <= max(2, len(sample) // 50), f"near-tie selections on {len(differ)} rows"
    # Downstream of the selection: sequences whose kept set equals the oracle's own.
    r_idx, r_cnt, _ = oracle.topk_select(ref_delta, k_host[sample], fc.k_hi)
    hid = _bits(x["hidden_rows"][sample])
    checked = 0
    for si, b in enumerate(sample):
        if si in differ:
            continue
        n_b, cub = int(r_cnt[si]), int(g_cu[b])
        one = np.array([n_b], np.int32)
        ocu = np.array([0, n_b], np.int32)
        ridx = r_idx[si:si + 1]
        # gather
        ref_rows = oracle.gather_rows(hid[si:si + 1], ridx, one, ocu)
        np.testing.assert_array_equal(_bits(step.gathered[cub:cub + n_b]), ref_rows)
        # scatter (this sequence's slice of the cache)
        ck0, cv0 = cache_k0[int(b)]
        nk, nv = _bits(x["new_k"][cub:cub + n_b]), _bits(x["new_v"][cub:cub + n_b])
        pre = int(kv_len[b]) - fc.block
        rk, rv = oracle.kv_scatter(nk, nv, ridx, one, ocu, np.array([pre]), ck0, cv0)
        r0, r1 = int(seq_start[b]), int(seq_start[b] + kv_len[b])
        np.testing.assert_array_equal(_bits(x["cache_k"][r0:r1]), rk)
        np.testing.assert_array_equal(_bits(x["cache_v"][r0:r1]), rv)
        # attention of this sequence's kept rows
        ref_o = oracle.reduced_attention(oc.bf16_bits_to_f64(_bits(x["q_kept"][cub:cub + n_b])),
                                         one, ocu, oc.bf16_bits_to_f64(rk), oc.bf16_bits_to_f64(rv),
                                         np.array([0]), np.array([kv_len[b]]), fc.hq, fc.hkv,
                                         1.0 / math.sqrt(fc.head_dim))
        assert_close(_f64(step.out[cub:cub + n_b]), ref_o, f"attention seq {b}")
        checked += 1
    assert checked >= len(sample) - len(differ)
    return differ


FUSED = pytest.mark.parametrize("fused", [False, True], ids=["scatter_then_attention",
                                                              "fused_scatter_attention"])


@FUSED
def test_chain_small_every_sequence(fused):
    fc = W.FocusCfg("chain_small", seed=51, batch=48)
    ac = W.AttnCfg("chain_small", seed=51, batch=48, kept=None, prefix_lo=40, prefix_hi=700)
    _check_chain(fc, ac, list(range(48)), fused=fused)


@FUSED
def test_chain_b1024_full_size_sampled(fused):
    """The benchmarked workload itself (batch 1024, prefixes 1024..4096)."""
    sample = sorted(np.random.default_rng(9).choice(1024, size=48, replace=False).tolist())
    _check_chain(W.CHAIN_FOCUS_B1024, W.CHAIN_ATTN_B1024, sample, fused=fused)


@FUSED
def test_focus_step_graph_replays_match_eager(fused):
    """A FOCUS step captured in a HIP graph and replayed three times, with eager
    work and synchronisations in between: every replay equals the eager step
    bit for bit (the kernels allocate nothing and record no memset nodes)."""
    from block_token_eviction_amd.chain import FocusStep
    fc = W.FocusCfg("graph", seed=81, batch=64)
    ac = W.AttnCfg("graph", seed=81, batch=64, kept=None, prefix_lo=100, prefix_hi=600)
    say(f"focus step under graph capture fused={fused}")
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
