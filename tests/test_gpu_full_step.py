"""GPU parity of the extended FOCUS step (FocusFullStep: delta -> device budget
-> constrained selection -> one-launch compaction of four per-token tensors
-> paged KV scatter -> longest-first paged attention -> delayed commit mask
-> history update), in the launch configuration bench.py times.

The importance delta is compared with the oracle within tolerance. The
integer decisions taken from it (budget, selection) are recomputed by the
oracle from the GPU's own fp32 delta, so both sides decide in the same
precision, and must agree exactly; everything downstream of the selection
(compaction, scatter, commit mask, history) is bit-exact, and the attention
output is within tolerance of the oracle's."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.chain as oc
import workloads as W
from helpers import assert_close, say

pytestmark = pytest.mark.gpu

ALPHA = 1.5


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _pool_rows(bt, b, kv_len, page):
    """Physical pool rows of sequence b's logical positions 0 .. kv_len-1."""
    p = np.arange(int(kv_len), dtype=np.int64)
    return bt[b, p // page].astype(np.int64) * page + p % page


def _check_full_step(fc, ac, page, sample, fused=False):
    from block_token_eviction_amd.chain import FocusFullStep
    say(f"full step {fc.name} batch={fc.batch} page={page} sample={len(sample)} fused={fused}")
    x = W.focus_full_inputs(fc, ac, page_size=page, device="cuda")
    n, B = fc.batch, fc.block
    bt = x["block_table"].cpu().numpy()
    kv_len = x["kv_len"].cpu().numpy()
    state0 = {k: x[k].cpu().numpy().copy()
              for k in ("token_sum", "total_steps", "rightmost_processed", "cached")}
    # pre-images of the sampled sequences' pool rows
    rows_of = {int(b): _pool_rows(bt, int(b), kv_len[b], page) for b in sample}
    pre = {b: (_bits(x["pool_k"][torch.from_numpy(r).cuda()]),
               _bits(x["pool_v"][torch.from_numpy(r).cuda()])) for b, r in rows_of.items()}
    per_token = [x["hidden_rows"], x["residual"], x["rope_pos"], x["cache_idx"]]
    step = FocusFullStep(n, B, fc.hq, fc.head_dim,
                         [(t.shape[2:], t.dtype) for t in per_token], fc.dtype, "cuda",
                         hkv=fc.hkv)
    step.run(q0=x["q0"], k0=x["k0"], q1=x["q1"], k1=x["k1"], decoded=x["decoded"],
             decoded_now=x["decoded_now"], pool_kernel=fc.pool_kernel, alpha=ALPHA,
             token_sum=x["token_sum"], total_steps=x["total_steps"],
             rightmost_processed=x["rightmost_processed"], cached=x["cached"],
             per_token=per_token, new_k=x["new_k_full"], new_v=x["new_v_full"],
             q_kept=x["q_full"], pos_base=x["pos_base"], block_table=x["block_table"],
             page_size=page, pool_k=x["pool_k"], pool_v=x["pool_v"], kv_len=x["kv_len"],
             fused=fused)
    torch.cuda.synchronize()
    dec = x["decoded"].cpu().numpy().astype(bool)
    now = x["decoded_now"].cpu().numpy().astype(bool)
    sample = np.asarray(sample)

    # delta against the oracle (float tolerance), on the sampled sequences
    g_delta = step.delta.cpu().numpy()
    ref_delta = oracle.focus_importance_delta(_f64(x["q0"][sample]), _f64(x["k0"][sample]),
                                              _f64(x["q1"][sample]), _f64(x["k1"][sample]),
                                              dec[sample].astype(np.uint8), fc.hq, fc.hkv,
                                              fc.pool_kernel)
    assert_close(g_delta[sample], ref_delta, "delta")

    # budget and selection from the GPU's delta: exact, every sequence
    k_ref = oracle.focus_budget(g_delta, state0["token_sum"], state0["total_steps"], ALPHA)
    np.testing.assert_array_equal(step.k.cpu().numpy(), k_ref)
    r_idx, r_cnt, r_cu, r_rp = oracle.focus_select(g_delta, k_ref, dec,
                                                   state0["rightmost_processed"])
    np.testing.assert_array_equal(step.idx.cpu().numpy(), r_idx)
    np.testing.assert_array_equal(step.count.cpu().numpy(), r_cnt)
    np.testing.assert_array_equal(step.cu.cpu().numpy(), r_cu)
    np.testing.assert_array_equal(x["rightmost_processed"].cpu().numpy(), r_rp)
    assert r_cnt.min() >= 1

    # commit mask and history: exact, every sequence
    w_commit, w_cached, w_done = oracle.commit_mask(dec, state0["cached"].astype(bool))
    np.testing.assert_array_equal(step.commit.cpu().numpy().astype(bool), w_commit)
    np.testing.assert_array_equal(x["cached"].cpu().numpy().astype(bool), w_cached)
    np.testing.assert_array_equal(step.block_done.cpu().numpy(), w_done)
    w_ts, w_st = oracle.history_update(dec, now, state0["token_sum"], state0["total_steps"])
    np.testing.assert_array_equal(x["token_sum"].cpu().numpy(), w_ts)
    np.testing.assert_array_equal(x["total_steps"].cpu().numpy(), w_st)

    # compaction, scatter and attention of the sampled sequences
    one = np.array([0], np.int32)
    pos_base = x["pos_base"].cpu().numpy()
    scale = 1.0 / math.sqrt(fc.head_dim)
    for b in sample:
        b = int(b)
        cnt, c0 = int(r_cnt[b]), int(r_cu[b])
        sel = r_idx[b:b + 1, :cnt]
        cnt1, cu1 = np.array([cnt], np.int32), np.array([0, cnt], np.int32)
        for src, out in zip(per_token, step.rows):
            h = src[b:b + 1].cpu()
            h = h.view(torch.int16) if h.dtype == torch.bfloat16 else h
            o = out[c0:c0 + cnt].cpu()
            o = o.view(torch.int16) if o.dtype == torch.bfloat16 else o
            np.testing.assert_array_equal(o.numpy(), oracle.gather_rows(h.numpy(), sel, cnt1, cu1))
        # the sequence's pool rows after the scatter, in logical order
        rows = torch.from_numpy(rows_of[b]).cuda()
        got_k, got_v = _bits(x["pool_k"][rows]), _bits(x["pool_v"][rows])
        nk, nv = _bits(x["new_k_full"][c0:c0 + cnt]), _bits(x["new_v_full"][c0:c0 + cnt])
        # the oracle's paged scatter on a one-sequence pool laid out contiguously
        ident = np.arange((int(kv_len[b]) + page - 1) // page, dtype=np.int32)[None, :]
        pk0, pv0 = pre[b]
        padk = np.zeros((ident.size * page,) + pk0.shape[1:], pk0.dtype)
        padv = padk.copy()
        padk[:kv_len[b]], padv[:kv_len[b]] = pk0, pv0
        rk, rv = oracle.kv_scatter_paged(nk, nv, sel, cnt1, cu1, pos_base[b:b + 1], ident, page,
                                         padk, padv)
        np.testing.assert_array_equal(got_k, rk[:kv_len[b]])
        np.testing.assert_array_equal(got_v, rv[:kv_len[b]])
        ref_o = oracle.reduced_attention(oc.bf16_bits_to_f64(_bits(x["q_full"][c0:c0 + cnt])),
                                         cnt1, cu1, oc.bf16_bits_to_f64(rk[:kv_len[b]]),
                                         oc.bf16_bits_to_f64(rv[:kv_len[b]]), one,
                                         np.array([kv_len[b]]), fc.hq, fc.hkv, scale)
        assert_close(_f64(step.out[c0:c0 + cnt]), ref_o, f"attention seq {b}")


FUSED = pytest.mark.parametrize("fused", [False, True], ids=["scatter_then_attention",
                                                              "fused_scatter_attention"])


@FUSED
def test_full_step_small_every_sequence(fused):
    fc = W.FocusCfg("full_small", seed=52, batch=40)
    ac = W.AttnCfg("full_small", seed=52, batch=40, kept=None, prefix_lo=20, prefix_hi=600)
    _check_full_step(fc, ac, 16, list(range(40)), fused=fused)


@FUSED
def test_full_step_b1024_sampled(fused):
    """The benchmarked extended step itself (batch 1024, prefixes 1024..4096, pages of 64)."""
    sample = sorted(np.random.default_rng(11).choice(1024, size=24, replace=False).tolist())
    _check_full_step(W.CHAIN_FOCUS_B1024, W.CHAIN_ATTN_B1024, 64, sample, fused=fused)


@FUSED
def test_full_step_graph_replays_match_eager(fused):
    """The extended step captured in a HIP graph and replayed three times, with the
    per-sequence state restored and the outputs cleared eagerly in between: every
    replay equals the eager step bit for bit (outputs, state, KV pool)."""
    from block_token_eviction_amd.chain import FocusFullStep
    fc = W.FocusCfg("full_graph", seed=53, batch=48)
    ac = W.AttnCfg("full_graph", seed=53, batch=48, kept=None, prefix_lo=30, prefix_hi=500)
    say(f"extended step under graph capture fused={fused}")
    page = 16
    x = W.focus_full_inputs(fc, ac, page_size=page, device="cuda")
    per_token = [x["hidden_rows"], x["residual"], x["rope_pos"], x["cache_idx"]]
    step = FocusFullStep(fc.batch, fc.block, fc.hq, fc.head_dim,
                         [(t.shape[2:], t.dtype) for t in per_token], fc.dtype, "cuda",
                         hkv=fc.hkv)
    state = [x[k] for k in ("token_sum", "total_steps", "rightmost_processed", "cached")]
    state0 = [t.clone() for t in state]
    pool0 = (x["pool_k"].clone(), x["pool_v"].clone())
    args = dict(q0=x["q0"], k0=x["k0"], q1=x["q1"], k1=x["k1"], decoded=x["decoded"],
                decoded_now=x["decoded_now"], pool_kernel=fc.pool_kernel, alpha=ALPHA,
                token_sum=x["token_sum"], total_steps=x["total_steps"],
                rightmost_processed=x["rightmost_processed"], cached=x["cached"],
                per_token=per_token, new_k=x["new_k_full"], new_v=x["new_v_full"],
                q_kept=x["q_full"], pos_base=x["pos_base"], block_table=x["block_table"],
                page_size=page, pool_k=x["pool_k"], pool_v=x["pool_v"], kv_len=x["kv_len"],
                fused=fused)

    def reset():
        for t, t0 in zip(state, state0):
            t.copy_(t0)
        x["pool_k"].copy_(pool0[0])
        x["pool_v"].copy_(pool0[1])
        step.out.zero_()
        for r in step.rows:
            r.zero_()

    reset()
    step.run(**args)
    torch.cuda.synchronize()
    n = int(step.cu[-1])
    outs = lambda: [step.delta, step.k, step.idx, step.count, step.cu, step.commit,
                    step.block_done, step.out[:n]] + [r[:n] for r in step.rows] + state + \
                   [x["pool_k"], x["pool_v"]]
    want = [t.clone() for t in outs()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                  # warm-up on the capture stream
        reset()
        step.run(**args)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(g):
        step.run(**args)
    for rep in range(3):
        reset()                                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs(), want)):
            assert torch.equal(a, b), f"replay {rep}, tensor {i}"
