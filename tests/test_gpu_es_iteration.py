"""GPU parity: ES-dLLM skip-layer score with the in-place hidden-cache update,
the ragged-source gather, the iteration bookkeeping and whole iterations of
the skip pipeline (ES-dLLM notes page, key designs 1 and 2) against the
float64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import assert_close, dev, say

pytestmark = pytest.mark.gpu


def _bte():
    import block_token_eviction_amd as bte
    return bte


def _bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


def test_score_update_equals_score_then_cache_write():
    """Batch 8, 256 survivors, 768 positions, hidden 4096, bf16: the fused call gives the
    scores of bte_esdllm_score bit for bit, and the cache afterwards holds every survivor's
    new row at its position and the old rows elsewhere."""
    bte = _bte()
    cfg = W.ES_B8
    g = dev(W.esdllm_inputs(cfg))
    L = cfg.prompt + cfg.generated
    say("esdllm score_update, batch 8")
    want = bte.esdllm_score(g["h_new"], g["h_prev"], g["surv_pos"], g["conf"], g["alpha"])
    cache0 = _bits(g["h_prev"]).copy()
    got = bte.esdllm_score_update(g["h_new"], g["h_prev"], g["surv_pos"], g["conf"], g["alpha"])
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    n = cfg.generated
    rows = _bits(g["h_new"]).reshape(cfg.batch * n, -1)
    ident = np.tile(np.arange(n, dtype=np.int32), (cfg.batch, 1))
    ref, _ = oracle.kv_scatter(rows, rows, ident, np.full(cfg.batch, n, np.int32),
                               np.arange(cfg.batch + 1, dtype=np.int32) * n,
                               np.arange(cfg.batch) * L, cache0.reshape(cfg.batch * L, -1),
                               cache0.reshape(cfg.batch * L, -1),
                               pos_map=g["surv_pos"].cpu().numpy())
    np.testing.assert_array_equal(_bits(g["h_prev"]).reshape(cfg.batch * L, -1), ref)


def _ragged_inputs(seed, counts, L, hidden, dtype, cap):
    r = np.random.default_rng(seed)
    batch = len(counts)
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    surv = np.concatenate([np.sort(r.choice(L, size=c, replace=False)) for c in counts]
                          ).astype(np.int32)
    cache = W.normal((batch, L, hidden), seed, 1, dtype)
    b_of = np.repeat(np.arange(batch), counts)
    rows = cache.reshape(batch * L, hidden)[torch.from_numpy(b_of * L + surv)].to(torch.float32)
    noise = W.normal(rows.shape, seed, 2, W.F32, std=0.05)
    hit = torch.from_numpy(r.random(rows.shape[0]) < 0.3)
    rows[hit] += noise[hit]
    conf = torch.from_numpy(r.beta(0.5, 2.0, size=(batch, L)).astype(np.float32))
    return dict(cache=cache, h_rows=rows.to(dtype), surv=torch.from_numpy(surv),
                count=torch.from_numpy(np.array(counts, np.int32)), cu=torch.from_numpy(cu),
                conf=conf, cap=cap)


@pytest.mark.parametrize("counts,cap,L,hidden,dtype", [
    ([256, 128, 0, 256, 37, 1, 200, 128], 256, 768, 4096, W.BF16),
    ([5, 0, 9, 3], 9, 40, 200, W.F32),
    ([64] * 3 + [0], 64, 64, 128, W.BF16),
], ids=["b8_h4096", "f32_odd", "full_block"])
def test_score_update_ragged(counts, cap, L, hidden, dtype):
    """Survivor sets of different sizes, compacted by (count, cu): scores within tolerance of
    the oracle (-inf past count), the cache updated bit for bit at the survivors only."""
    bte = _bte()
    x = _ragged_inputs(50 + len(counts), counts, L, hidden, dtype, cap)
    g = dev(x)
    cache0 = x["cache"].clone()
    say(f"esdllm score_update ragged counts={counts}")
    got = bte.esdllm_score_update(g["h_rows"], g["cache"], g["surv"], g["conf"], 0.5,
                                  count=g["count"], cu=g["cu"], cap=cap)
    torch.cuda.synchronize()
    k = np.array(counts)          # keep everyone: the selection is the identity
    score, _, _, _, _, _, new_cache = oracle.esdllm_skip_layer_ragged(
        W.to_f64(x["h_rows"]), W.to_f64(cache0), x["surv"].numpy(), x["count"].numpy(),
        x["cu"].numpy(), x["conf"].numpy(), 0.5, k, cap)
    assert_close(got.cpu().numpy(), score, "ragged score")
    batch = len(counts)
    idx = np.full((batch, cap), -1, np.int32)
    for b, c in enumerate(counts):
        idx[b, :c] = np.arange(c)
    rows, c0 = _bits(x["h_rows"]), _bits(cache0).reshape(batch * L, -1)
    want_cache, _ = oracle.kv_scatter(rows, rows, idx, x["count"].numpy(), x["cu"].numpy(),
                                      np.arange(batch) * L, c0, c0, pos_map=_surv_map(x, cap))
    np.testing.assert_array_equal(_bits(g["cache"]).reshape(len(counts) * L, -1), want_cache)
    np.testing.assert_array_equal(W.to_f64(g["cache"]), new_cache)


def _surv_map(x, cap):
    """pos_map[b, s] = position of sequence b's survivor s (rows compacted by cu)."""
    counts, cu, surv = x["count"].numpy(), x["cu"].numpy(), x["surv"].numpy()
    pm = np.zeros((len(counts), cap), np.int32)
    for b, c in enumerate(counts):
        pm[b, :c] = surv[cu[b]:cu[b] + c]
    return pm


def test_gather_rows_multi_ragged():
    bte = _bte()
    r = np.random.default_rng(61)
    counts = np.array([5, 0, 12, 1, 7], np.int32)
    src_cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(src_cu[-1]) + 3
    hid = W.normal((rows, 512), 61, 1, W.BF16)
    pos = torch.from_numpy(r.integers(0, 1000, rows).astype(np.int32))
    keep = np.array([3, 0, 12, 1, 0], np.int32)
    k_max = 12
    idx = np.full((5, k_max), -1, np.int32)
    for b in range(5):
        idx[b, :keep[b]] = np.sort(r.choice(counts[b], size=keep[b], replace=False))
    cu = np.concatenate([[0], np.cumsum(keep)]).astype(np.int32)
    t = lambda a: torch.from_numpy(a).cuda()
    say("gather_rows_multi_ragged")
    outs = bte.gather_rows_multi_ragged([hid.cuda(), pos.cuda()], t(src_cu), t(idx), t(keep), t(cu))
    torch.cuda.synchronize()
    n = int(cu[-1])
    np.testing.assert_array_equal(_bits(outs[0])[:n],
                                  oracle.gather_rows_ragged(_bits(hid), src_cu, idx, keep, cu))
    np.testing.assert_array_equal(outs[1].cpu().numpy()[:n],
                                  oracle.gather_rows_ragged(pos.numpy(), src_cu, idx, keep, cu))


@pytest.mark.parametrize("batch,period,block_len,keep", [
    (1, 3, 256, [128, 64]), (7, 0, 5, [3, 1]), (300, 1, 32, [16]), (5000, 7, 256, [128, 64]),
    (64, 4, 100, [60, 60, 2, 0]), (9, 2, 256, []),
])
def test_schedule_matches_oracle(batch, period, block_len, keep):
    bte = _bte()
    r = np.random.default_rng(batch + period)
    it = r.integers(0, 40, batch).astype(np.int32)
    it[: min(3, batch)] = 0
    start = r.integers(0, 4096, batch).astype(np.int32)
    g_it = torch.from_numpy(it).cuda()
    say(f"esdllm schedule batch={batch} period={period} keep={keep}")
    surv, cnt, cu, kout, ref_ = bte.esdllm_schedule(g_it, torch.from_numpy(start).cuda(), block_len,
                                                    period, keep)
    torch.cuda.synchronize()
    want = oracle.esdllm_schedule(it, start, block_len, period, keep)
    np.testing.assert_array_equal(surv.cpu().numpy(), want["surv_pos"])
    np.testing.assert_array_equal(cnt.cpu().numpy(), want["count"])
    np.testing.assert_array_equal(cu.cpu().numpy(), want["cu"])
    np.testing.assert_array_equal(kout.cpu().numpy()[:len(keep)], want["keep"])
    np.testing.assert_array_equal(ref_.cpu().numpy().astype(bool), want["refresh"])
    np.testing.assert_array_equal(g_it.cpu().numpy(), want["iter"])


def test_iterations_of_the_skip_pipeline():
    """Batch 8, a 256-position block at the end of 768 positions, hidden 4096, bf16, two
    skip layers keeping 128 then 64 (r = 0.5), refresh period 3, sequences starting at
    iteration counters 0..7: four iterations, checked layer by layer. Per layer: scores
    within tolerance of the oracle; the selection equal to the oracle's top-K of the same
    fp32 scores; kept rows, positions, counts and the updated cache bit for bit."""
    from block_token_eviction_amd.chain import EsIteration
    cfg = W.ES_B8
    batch, L, h = cfg.batch, cfg.prompt + cfg.generated, cfg.hidden
    blk, keep, period = cfg.generated, [128, 64], 3
    x = W.es_pipeline_inputs(cfg, layers=2, device="cuda")
    it = torch.arange(batch, dtype=torch.int32, device="cuda")
    start = torch.full((batch,), cfg.prompt, dtype=torch.int32, device="cuda")
    run = EsIteration(batch, blk, h, keep, period, cfg.dtype, "cuda")

    def states(l, rows, count, cu):
        r = torch.arange(rows.shape[0], device="cuda")
        b = torch.searchsorted(cu[1:].contiguous(), r.to(torch.int32), right=True).clamp_(max=batch - 1)
        p = rows.long().clamp(0, L - 1)
        return x["h_cur"][l].view(batch * L, h).index_select(0, b * L + p)

    for step in range(4):
        it0 = it.cpu().numpy().copy()
        sch = oracle.esdllm_schedule(it0, start.cpu().numpy(), blk, period, keep)
        say(f"es iteration {step}: counters {it0.tolist()}")
        surv, count, cu, kout, refresh = run.schedule(it, start)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(refresh.cpu().numpy().astype(bool), sch["refresh"])
        np.testing.assert_array_equal(kout.cpu().numpy(), sch["keep"])
        rows = surv.view(-1)
        for l in range(2):
            h_rows = states(l, rows, count, cu)
            cache0 = x["h_cache"][l].clone()
            n_rows = int(cu[-1])
            rows_np, cnt_np, cu_np = rows.cpu().numpy()[:n_rows], count.cpu().numpy(), cu.cpu().numpy()
            _, rows2, count2, cu2 = run.layer(l, h_rows, rows, count, cu, x["h_cache"][l],
                                              x["conf"], x["alpha"])
            torch.cuda.synchronize()
            k_l = sch["keep"][l]
            ref = oracle.esdllm_skip_layer_ragged(
                W.to_f64(h_rows[:n_rows]), W.to_f64(cache0), rows_np, cnt_np, cu_np,
                x["conf"].cpu().numpy(), x["alpha"], k_l, blk)
            g_score = run.score[l].cpu().numpy()
            assert_close(g_score, ref[0], f"iteration {step} layer {l} score")
            r_idx, r_cnt, r_cu = oracle.topk_select(g_score, k_l, blk)
            np.testing.assert_array_equal(run.idx[l].cpu().numpy(), r_idx)
            np.testing.assert_array_equal(count2.cpu().numpy(), r_cnt)
            np.testing.assert_array_equal(cu2.cpu().numpy(), r_cu)
            m = int(r_cu[-1])
            np.testing.assert_array_equal(
                _bits(run.h_next[l])[:m],
                oracle.gather_rows_ragged(_bits(h_rows[:n_rows]), cu_np, r_idx, r_cnt, r_cu))
            np.testing.assert_array_equal(
                rows2.cpu().numpy()[:m], oracle.gather_rows_ragged(rows_np, cu_np, r_idx, r_cnt, r_cu))
            np.testing.assert_array_equal(W.to_f64(x["h_cache"][l]), ref[6])
            rows, count, cu = rows2, count2, cu2
        want_last = np.where(sch["refresh"], blk, keep[-1])
        np.testing.assert_array_equal(count.cpu().numpy(), want_last)
        np.testing.assert_array_equal(it.cpu().numpy(), it0 + 1)
