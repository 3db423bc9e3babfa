"""GPU parity: FOCUS importance delta (HIP) vs the float64 oracle."""
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


def _run(cfg, inputs=None):
    bte = _bte()
    fi = inputs if inputs is not None else W.focus_inputs(cfg)
    g = dev(fi)
    say(f"focus {cfg}")
    out = bte.focus_importance_delta(g["q0"], g["k0"], g["q1"], g["k1"], g["decoded"], cfg.pool_kernel)
    torch.cuda.synchronize()
    f64 = W.to_f64
    ref = oracle.focus_importance_delta(f64(fi["q0"]), f64(fi["k0"]), f64(fi["q1"]), f64(fi["k1"]),
                                        fi["decoded"].numpy(), cfg.hq, cfg.hkv, cfg.pool_kernel)
    return out.cpu().numpy(), ref, g


def test_tiny_fp32():
    got, ref, _ = _run(W.TINY_FOCUS)
    assert_close(got, ref, "tiny")


def test_focus_b256_full_size():
    """Batch 256, 32q/8kv heads, head dim 128, bf16, MaxPool 7: every output."""
    got, ref, _ = _run(W.FOCUS_B256)
    assert_close(got, ref, "focus_b256")


# Blocks of 32 or 64 with 32 query / 8 KV heads in bf16 and a pooling radius up to 3 take
# several sequences per workgroup at large batches: 2 per workgroup at batches 257-512,
# 4 at 1,000-1,024 (the launch's cost model), the last workgroup possibly partial (511:
# one sequence in it; 1,021-1,023: one to three); 1,027 takes one per workgroup. Every
# sequence's delta must be bitwise the one a workgroup per sequence gives (the same
# inputs in slices of 256 sequences, which take that path) and match the oracle.
@pytest.mark.parametrize("batch,pool,block", [(511, 7, 32), (1024, 3, 32), (1021, 7, 32),
                                              (1022, 1, 32), (1023, 5, 32), (1027, 7, 32),
                                              (511, 3, 64), (1021, 7, 64)])
def test_focus_sequences_per_workgroup(batch, pool, block):
    bte = _bte()
    cfg = W.FocusCfg("multi", seed=41, batch=batch, block=block, pool_kernel=pool, hidden=64)
    fi = W.focus_inputs(cfg)
    g = dev(fi)
    say(f"focus several sequences per workgroup: batch={batch} pool={pool} block={block}")
    out = bte.focus_importance_delta(g["q0"], g["k0"], g["q1"], g["k1"], g["decoded"], pool)
    parts = [bte.focus_importance_delta(g["q0"][i:i + 256], g["k0"][i:i + 256], g["q1"][i:i + 256],
                                        g["k1"][i:i + 256], g["decoded"][i:i + 256], pool)
             for i in range(0, batch, 256)]
    torch.cuda.synchronize()
    assert torch.equal(out, torch.cat(parts))
    f64 = W.to_f64
    ref = oracle.focus_importance_delta(f64(fi["q0"]), f64(fi["k0"]), f64(fi["q1"]), f64(fi["k1"]),
                                        fi["decoded"].numpy(), cfg.hq, cfg.hkv, pool)
    assert_close(out.cpu().numpy(), ref, f"multi {batch}")


# Blocks of 16 run in pairs as blocks of 32 (the same memory), the two kept apart by a mask;
# an odd last block runs on its own. Batches 2-7 (one to three pairs, odd and even), 512 and
# 1,024 (two and four pairs per workgroup at the 32/8-head shape), pools up to the whole row
# and a runtime radius wider than the block, other head shapes, fp32.
PAIR_CASES = [
    # batch, hq, hkv, head_dim, pool, dtype
    (2, 32, 8, 128, 7, W.BF16),
    (7, 32, 8, 128, 7, W.BF16),
    (5, 32, 8, 128, 1, W.BF16),
    (6, 32, 8, 128, 31, W.BF16),      # window covers the whole block
    (3, 32, 8, 128, 41, W.BF16),      # runtime radius 20, wider than the block
    (4, 8, 2, 64, 5, W.BF16),         # waves loop over nothing: runtime group count
    (5, 16, 16, 128, 3, W.BF16),      # more KV heads than waves
    (3, 8, 8, 128, 7, W.F32),
    (512, 32, 8, 128, 7, W.BF16),
    (1024, 32, 8, 128, 7, W.BF16),
    (1025, 32, 8, 128, 3, W.BF16),
]


@pytest.mark.parametrize("case", PAIR_CASES, ids=[str(c[:5]) for c in PAIR_CASES])
def test_blocks_of_16_in_pairs(case):
    batch, hq, hkv, D, pool, dt = case
    cfg = W.FocusCfg("pairs", seed=17, batch=batch, block=16, hq=hq, hkv=hkv, head_dim=D,
                     dtype=dt, pool_kernel=pool, hidden=64)
    got, ref, _ = _run(cfg)
    assert_close(got, ref, str(case))


def test_blocks_of_16_spike_at_the_pair_edge():
    """The spike closed form of a block of 16 with the spike at its last position, whose
    pooling window would reach into the paired block: the neighbour block (spike-free,
    uniform) must stay exactly uniform, and the spiked block must follow the closed form
    with the window cut at the block's edge."""
    bte = _bte()
    B, hq, D = 16, 4, 64
    q0 = torch.zeros((4, B, hq, D))
    k0 = torch.randn((4, B, hq, D), generator=torch.Generator().manual_seed(3))
    q1 = torch.zeros((4, B, hq, D)); q1[..., 0] = 1.0
    k1 = torch.zeros((4, B, hq, D)); k1[0, 15, :, 0] = 5.5; k1[3, 0, :, 0] = 5.5
    dec = torch.zeros((4, B), dtype=torch.uint8)
    say("focus spike, blocks of 16 in pairs")
    got = bte.focus_importance_delta(q0.cuda(), k0.cuda(), q1.cuda(), k1.cuda(), dec.cuda(), 7).cpu().numpy()
    es = np.exp(5.5 / 8.0)
    for b, p in ((0, 15), (3, 0)):
        nw = min(B - 1, p + 3) - max(0, p - 3) + 1
        den = nw * es + (B - nw)
        win = np.zeros(B, bool); win[max(0, p - 3):min(B - 1, p + 3) + 1] = True
        want = np.where(win, hq * (B * es / den - 1.0), hq * (B / den - 1.0))
        np.testing.assert_allclose(got[b], want, rtol=2e-2, atol=1e-3)
    # blocks 1 and 2 (each paired with a spiked block) have identical layers: exactly +0.0
    assert np.all(got[1] == 0.0) and np.all(got[2] == 0.0)


CASES = [
    # block, hq, hkv, head_dim, pool, dtype
    (32, 32, 8, 128, 3, W.BF16),
    (32, 32, 8, 128, 1, W.BF16),
    (32, 32, 8, 64, 5, W.BF16),
    (32, 16, 16, 128, 7, W.BF16),     # more KV heads than waves: waves loop over groups
    (20, 8, 2, 64, 5, W.BF16),        # ragged block
    (16, 32, 8, 128, 7, W.BF16),      # half block: padding keys next to the edge
    (31, 32, 8, 128, 3, W.BF16),
    (17, 16, 4, 64, 41, W.BF16),      # runtime radius on a ragged block
    (7, 4, 1, 128, 9, W.BF16),        # runtime pooling radius, single KV head
    (32, 8, 4, 64, 63, W.BF16),       # window covers the whole row
    (32, 8, 4, 64, 41, W.BF16),       # window wider than a half row
    (1, 2, 1, 64, 7, W.F32),          # one-token block
    (32, 64, 8, 128, 7, W.BF16),      # 8 query heads per KV head
    (32, 12, 4, 128, 7, W.BF16),      # odd group size 3
    (32, 8, 8, 128, 7, W.F32),        # fp32 at head dim 128
    (16, 8, 2, 128, 3, W.F32),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[:5]) for c in CASES])
def test_shapes_and_pool_sizes(case):
    B, hq, hkv, D, pool, dt = case
    cfg = W.FocusCfg("edge", seed=11, batch=5, block=B, hq=hq, hkv=hkv, head_dim=D, dtype=dt,
                     pool_kernel=pool, hidden=64)
    got, ref, _ = _run(cfg)
    assert_close(got, ref, str(case))


def test_identical_layers_give_exact_zero_and_runs_are_bitwise_equal():
    bte = _bte()
    cfg = W.FocusCfg("det", seed=12, batch=16)
    g = dev(W.focus_inputs(cfg))
    say("focus determinism")
    a = bte.focus_importance_delta(g["q0"], g["k0"], g["q0"], g["k0"], g["decoded"], 7)
    b1 = bte.focus_importance_delta(g["q0"], g["k0"], g["q1"], g["k1"], g["decoded"], 7)
    b2 = bte.focus_importance_delta(g["q0"], g["k0"], g["q1"], g["k1"], g["decoded"], 7)
    torch.cuda.synchronize()
    a = a.cpu().numpy()
    dec = g["decoded"].cpu().numpy() != 0
    assert np.all(np.isneginf(a[dec]))
    assert np.all(a[~dec] == 0.0) and not np.any(np.signbit(a[~dec]))
    assert torch.equal(b1, b2)


def test_all_decoded_and_spike_closed_form():
    bte = _bte()
    B, hq, D = 32, 4, 64
    q0 = torch.zeros((2, B, hq, D))
    k0 = torch.randn((2, B, hq, D), generator=torch.Generator().manual_seed(1))
    q1 = torch.zeros((2, B, hq, D)); q1[..., 0] = 1.0
    k1 = torch.zeros((2, B, hq, D)); k1[0, 10, :, 0] = 5.5; k1[1, 0, :, 0] = 5.5   # bf16-exact spike
    dec = torch.zeros((2, B), dtype=torch.uint8)
    say("focus spike")
    got = bte.focus_importance_delta(q0.cuda(), k0.cuda(), q1.cuda(), k1.cuda(), dec.cuda(), 7).cpu().numpy()
    es, p_list = np.exp(5.5 / 8.0), (10, 0)
    for b, p in enumerate(p_list):
        nw = min(B - 1, p + 3) - max(0, p - 3) + 1
        Z = nw * es + B - nw
        want = np.where(np.abs(np.arange(B) - p) <= 3, hq * (B * es / Z - 1), hq * (B / Z - 1))
        assert_close(got[b], want, f"spike {p}")
    dec[:] = 1
    got = bte.focus_importance_delta(q0.cuda(), k0.cuda(), q1.cuda(), k1.cuda(), dec.cuda(), 7).cpu().numpy()
    assert np.all(np.isneginf(got))


# Blocks of 33..64 positions (the FOCUS paper runs blocks of 16, 32 and 64,
# Section 5.3 "Impact of Block Size"): two key tiles and two query-row tiles.
WIDE_CASES = [
    # block, hq, hkv, head_dim, pool, dtype
    (64, 32, 8, 128, 7, W.BF16),      # the workload head shape, static tile sequence
    (64, 32, 8, 128, 1, W.BF16),
    (64, 32, 8, 128, 3, W.BF16),
    (64, 32, 8, 128, 5, W.BF16),
    (63, 32, 8, 128, 7, W.BF16),      # one padding key and query row
    (48, 32, 8, 128, 7, W.BF16),
    (33, 32, 8, 128, 3, W.BF16),      # one real row in the second tiles
    (64, 32, 8, 128, 9, W.BF16),      # runtime radius 4 (dilation rounds)
    (64, 32, 8, 128, 127, W.BF16),    # window covers the whole row
    (40, 16, 4, 64, 41, W.BF16),      # runtime radius 20 on a ragged block
    (50, 8, 2, 64, 99, W.BF16),       # whole row on a ragged block
    (64, 16, 16, 128, 7, W.BF16),     # more KV heads than waves
    (64, 12, 4, 128, 7, W.BF16),      # odd group size 3
    (64, 64, 8, 128, 7, W.BF16),      # 8 query heads per KV head
    (37, 4, 1, 64, 7, W.BF16),        # single KV head
    (64, 4, 4, 64, 7, W.F32),
    (48, 8, 8, 128, 5, W.F32),        # fp32 at head dim 128
    (64, 8, 2, 128, 11, W.F32),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=[str(c[:5]) for c in WIDE_CASES])
def test_wide_blocks(case):
    B, hq, hkv, D, pool, dt = case
    cfg = W.FocusCfg("wide", seed=13, batch=5, block=B, hq=hq, hkv=hkv, head_dim=D, dtype=dt,
                     pool_kernel=pool, hidden=64)
    got, ref, _ = _run(cfg)
    assert_close(got, ref, str(case))


def test_focus_b64_full_size():
    """Batch 256, block 64, 32q/8kv heads, head dim 128, bf16, MaxPool 7: every output."""
    cfg = W.FocusCfg("focus_b256_block64", seed=2, batch=256, block=64)
    got, ref, _ = _run(cfg)
    assert_close(got, ref, "focus_b256_block64")


@pytest.mark.parametrize("B,p,pool", [(64, 40, 7), (64, 0, 7), (64, 63, 3), (48, 47, 9), (64, 20, 1)])
def test_wide_spike_closed_form(B, p, pool):
    """Spike input (layer-0 queries zero, layer-1 rows e0, one key s*sqrt(D)*e0): the delta
    is Hq (B e^s / Z - 1) inside the pooling window around p and Hq (B / Z - 1) outside,
    Z = n_w e^s + B - n_w."""
    bte = _bte()
    hq, D = 4, 64
    q0 = torch.zeros((1, B, hq, D))
    k0 = torch.randn((1, B, hq, D), generator=torch.Generator().manual_seed(2))
    q1 = torch.zeros((1, B, hq, D)); q1[..., 0] = 1.0
    k1 = torch.zeros((1, B, hq, D)); k1[0, p, :, 0] = 5.5          # s = 5.5 / sqrt(64)
    dec = torch.zeros((1, B), dtype=torch.uint8)
    say(f"wide spike B={B} p={p} pool={pool}")
    got = bte.focus_importance_delta(q0.cuda(), k0.cuda(), q1.cuda(), k1.cuda(), dec.cuda(),
                                     pool).cpu().numpy()[0]
    r = (pool - 1) // 2
    es = np.exp(5.5 / 8.0)
    nw = min(B - 1, p + r) - max(0, p - r) + 1
    Z = nw * es + B - nw
    want = np.where(np.abs(np.arange(B) - p) <= r, hq * (B * es / Z - 1), hq * (B / Z - 1))
    assert_close(got, want, f"spike B={B} p={p}")


def test_wide_identical_layers_give_exact_zero_and_runs_are_bitwise_equal():
    bte = _bte()
    cfg = W.FocusCfg("det_wide", seed=14, batch=16, block=64)
    g = dev(W.focus_inputs(cfg))
    say("focus determinism, block 64")
    a = bte.focus_importance_delta(g["q0"], g["k0"], g["q0"], g["k0"], g["decoded"], 7)
    b1 = bte.focus_importance_delta(g["q0"], g["k0"], g["q1"], g["k1"], g["decoded"], 7)
    b2 = bte.focus_importance_delta(g["q0"], g["k0"], g["q1"], g["k1"], g["decoded"], 7)
    torch.cuda.synchronize()
    a = a.cpu().numpy()
    dec = g["decoded"].cpu().numpy() != 0
    assert np.all(np.isneginf(a[dec]))
    assert np.all(a[~dec] == 0.0) and not np.any(np.signbit(a[~dec]))
    assert torch.equal(b1, b2)
