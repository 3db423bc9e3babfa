"""GPU parity of the FOCUS dynamic budget, history update and constrained
selection against the oracle, bit for bit, on the same fp32 deltas."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bte():
    import block_token_eviction_amd as bte
    return bte


def _cuda(a, dtype):
    return torch.as_tensor(np.ascontiguousarray(a)).to(dtype).cuda()


def _rand_delta(r, batch, block, p_dec=0.4):
    d = r.standard_normal((batch, block)).astype(np.float32)
    d[r.random((batch, block)) < 0.1] = 0.0                     # ties at zero
    w = min(2, block)
    d[:, :w][r.random((batch, w)) < 0.3] = -0.0
    dec = r.random((batch, block)) < p_dec
    d[dec] = -np.inf
    if batch > 3:
        d[0, :] = -np.inf                                         # everything decoded
        dec[0, :] = True
        d[1, :] = 0.5                                             # all masked, all equal
        dec[1, :] = False
        d[2, 1:] = -np.inf                                        # one masked position
        dec[2, 1:] = True
        dec[2, 0] = False
        d[2, 0] = 0.25
    return d, dec


def test_budget_worked_example():
    bte = _bte()
    fx = json.load(open(os.path.join(GOLDEN, "focus_budget_example.json")))
    say("focus_budget worked example")
    k = bte.focus_budget(_cuda(fx["delta"], torch.float32), _cuda(fx["token_sum"], torch.int32),
                         _cuda(fx["total_steps"], torch.int32), fx["alpha"])
    assert k.cpu().tolist() == fx["budget"]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("block", [1, 17, 32, 64])
def test_budget_random(mode, block):
    bte = _bte()
    r = np.random.default_rng(100 + block + mode)
    batch = 700
    d, _ = _rand_delta(r, batch, block)
    ts = r.integers(0, 200, batch).astype(np.int32)
    st = r.integers(0, 40, batch).astype(np.int32)
    ts[st == 0] = 0
    say(f"focus_budget block={block} mode={mode}")
    for alpha in (1.0, 1.5, 2.25, 3.7):
        k = bte.focus_budget(_cuda(d, torch.float32), _cuda(ts, torch.int32),
                             _cuda(st, torch.int32), alpha, mode).cpu().numpy()
        np.testing.assert_array_equal(k, oracle.focus_budget(d, ts, st, alpha, mode))


def test_budget_on_real_deltas():
    """The budget over the delta kernel's own output at batch 256."""
    bte = _bte()
    fc = W.FOCUS_B256
    fi = W.focus_inputs(fc, device="cuda")
    say("focus_budget on real deltas, batch 256")
    delta = bte.focus_importance_delta(fi["q0"], fi["k0"], fi["q1"], fi["k1"], fi["decoded"],
                                       fc.pool_kernel)
    r = np.random.default_rng(7)
    ts = r.integers(0, 100, fc.batch).astype(np.int32)
    st = r.integers(0, 30, fc.batch).astype(np.int32)
    for mode in (0, 1):
        k = bte.focus_budget(delta, _cuda(ts, torch.int32), _cuda(st, torch.int32), 1.5, mode)
        np.testing.assert_array_equal(k.cpu().numpy(),
                                      oracle.focus_budget(delta.cpu().numpy(), ts, st, 1.5, mode))


def test_history_update():
    bte = _bte()
    r = np.random.default_rng(8)
    batch, block = 1000, 32
    prev = r.random((batch, block)) < 0.3
    now = prev | (r.random((batch, block)) < 0.2)
    ts = r.integers(0, 50, batch).astype(np.int32)
    st = r.integers(0, 9, batch).astype(np.int32)
    g_ts, g_st = _cuda(ts, torch.int32), _cuda(st, torch.int32)
    say("focus_history_update")
    bte.focus_history_update(_cuda(prev, torch.uint8), _cuda(now, torch.uint8), g_ts, g_st)
    w_ts, w_st = oracle.history_update(prev, now, ts, st)
    np.testing.assert_array_equal(g_ts.cpu().numpy(), w_ts)
    np.testing.assert_array_equal(g_st.cpu().numpy(), w_st)


def _check_select(d, dec, k, rp, name):
    bte = _bte()
    g_rp = _cuda(rp, torch.int32)
    say(f"focus_select {name} batch={d.shape[0]} block={d.shape[1]}")
    idx, cnt, cu = bte.focus_select(_cuda(d, torch.float32), _cuda(k, torch.int32),
                                    _cuda(dec, torch.uint8), g_rp)
    w_idx, w_cnt, w_cu, w_rp = oracle.focus_select(d, k, dec, rp)
    np.testing.assert_array_equal(cnt.cpu().numpy(), w_cnt)
    np.testing.assert_array_equal(idx.cpu().numpy(), w_idx)
    np.testing.assert_array_equal(cu.cpu().numpy(), w_cu)
    np.testing.assert_array_equal(g_rp.cpu().numpy(), w_rp)


@pytest.mark.parametrize("block", [1, 2, 17, 32, 33, 64])
def test_select_random(block):
    r = np.random.default_rng(200 + block)
    batch = 900
    d, dec = _rand_delta(r, batch, block)
    d[5, 3 % block] = np.nan
    k = r.integers(-1, block + 3, batch).astype(np.int32)
    k[3] = 0
    rp = r.integers(-1, block, batch).astype(np.int32)
    rp[:50] = -1
    _check_select(d, dec, k, rp, "random")


def test_select_on_real_deltas_with_budget():
    """delta kernel -> budget -> constrained selection at batch 1024, as a step runs them."""
    bte = _bte()
    fc = W.CHAIN_FOCUS_B1024
    fi = W.focus_inputs(fc, device="cuda")
    say("delta -> budget -> select, batch 1024")
    delta = bte.focus_importance_delta(fi["q0"], fi["k0"], fi["q1"], fi["k1"], fi["decoded"],
                                       fc.pool_kernel)
    r = np.random.default_rng(9)
    ts = r.integers(0, 100, fc.batch).astype(np.int32)
    st = r.integers(1, 30, fc.batch).astype(np.int32)
    k = bte.focus_budget(delta, _cuda(ts, torch.int32), _cuda(st, torch.int32), 1.5)
    rp = r.integers(-1, 20, fc.batch).astype(np.int32)
    d = delta.cpu().numpy()
    kk = k.cpu().numpy()
    np.testing.assert_array_equal(kk, oracle.focus_budget(d, ts, st, 1.5))
    _check_select(d, fi["decoded"].cpu().numpy().astype(bool), kk, rp, "chain")


@pytest.mark.parametrize("block", [1, 3, 32, 64, 1000])
def test_commit_mask(block):
    bte = _bte()
    r = np.random.default_rng(300 + block)
    batch = 500
    dec = r.random((batch, block)) < r.random((batch, 1))
    dec[:20] = True                                           # whole blocks decoded
    cac = dec & (r.random((batch, block)) < 0.5)
    g_cac = _cuda(cac, torch.uint8)
    say(f"commit mask block={block}")
    commit, done = bte.focus_commit_mask(_cuda(dec, torch.uint8), g_cac)
    w_commit, w_cac, w_done = oracle.commit_mask(dec, cac)
    np.testing.assert_array_equal(commit.cpu().numpy().astype(bool), w_commit)
    np.testing.assert_array_equal(g_cac.cpu().numpy().astype(bool), w_cac)
    np.testing.assert_array_equal(done.cpu().numpy(), w_done)


def test_gather_multi():
    """Hidden rows (bf16 8 KB), residual (fp32 16 KB), RoPE positions (int32)
    and cache indices (int64) compacted in one launch, after a constrained
    selection, against the oracle's gather of each."""
    bte = _bte()
    r = np.random.default_rng(13)
    batch, block = 300, 32
    d, dec = _rand_delta(r, batch, block)
    k = r.integers(0, 12, batch).astype(np.int32)
    rp = np.full(batch, -1, np.int32)
    idx, cnt, cu = bte.focus_select(_cuda(d, torch.float32), _cuda(k, torch.int32),
                                    _cuda(dec, torch.uint8), _cuda(rp, torch.int32))
    srcs = [torch.randn(batch, block, 4096, device="cuda").to(torch.bfloat16),
            torch.randn(batch, block, 4096, device="cuda"),
            torch.randint(0, 1 << 20, (batch, block), dtype=torch.int32, device="cuda"),
            torch.randint(0, 1 << 40, (batch, block), dtype=torch.int64, device="cuda")]
    say("gather multi")
    outs = bte.gather_rows_multi(srcs, idx, cnt, cu)
    torch.cuda.synchronize()
    i_h, c_h, u_h = idx.cpu().numpy(), cnt.cpu().numpy(), cu.cpu().numpy()
    total = int(u_h[-1])
    for s_, o in zip(srcs, outs):
        host = s_.cpu()
        host = host.view(torch.int16) if host.dtype == torch.bfloat16 else host
        want = oracle.gather_rows(host.numpy(), i_h, c_h, u_h)
        got = o[:total].cpu()
        got = got.view(torch.int16) if got.dtype == torch.bfloat16 else got
        np.testing.assert_array_equal(got.numpy(), want)
