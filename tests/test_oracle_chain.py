"""Pins of the oracle's composed FOCUS step (oracle/chain.py), no GPU.

* ``bf16_bits_to_f64`` against torch's own bfloat16 -> float64 conversion on
  all 65,536 bit patterns (sign of zero, subnormals, infinities, NaNs).
* ``focus_step`` against its parts called one by one (each pinned in its own
  test file), on the tiny fp32 workload and on a small bf16 one passed as raw
  16-bit patterns: this pins the wiring (row_base, the kept-query slice,
  k_max, the bf16 widening before the attention).
* ``focus_step`` on a hand-worked step whose every output is known without
  the oracle: a spike input with a closed-form delta (FOCUS paper Section 3.1
  Eq. 2 and Section 3.2 Eq. 3), a kept set that follows from it under the tie
  rule (score descending, index ascending), byte-exact gather and scatter,
  and attention over identical value rows, whose output is that row.
"""
import math

import numpy as np
import torch

import oracle
import workloads as W
from oracle.chain import bf16_bits_to_f64, focus_step


def test_bf16_bits_to_f64_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):           # signalling-NaN patterns
        got = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 * 127                # exponent all ones, nonzero mantissa, both signs
    assert np.array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64))   # -0.0 too
    assert got[0x3F80] == 1.0 and got[0xBF80] == -1.0 and got[0x0001] == 2.0 ** -133
    assert got[0x7F80] == np.inf and got[0xFF80] == -np.inf


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _step_inputs(fcfg, acfg):
    x = W.chain_inputs(fcfg, acfg)
    as_host = _bits if fcfg.dtype == W.BF16 else (lambda t: t.numpy())
    return dict(q0=W.to_f64(x["q0"]), k0=W.to_f64(x["k0"]), q1=W.to_f64(x["q1"]),
                k1=W.to_f64(x["k1"]), decoded=x["decoded"].numpy(), k=x["k"].numpy(),
                hidden_rows=as_host(x["hidden_rows"]), pool_kernel=fcfg.pool_kernel,
                new_k=as_host(x["new_k"]), new_v=as_host(x["new_v"]), q_kept=as_host(x["q_kept"]),
                cache_k=as_host(x["cache_k"]), cache_v=as_host(x["cache_v"]),
                seq_start=x["seq_start"].numpy(), kv_len=x["kv_len"].numpy(),
                row_base=x["row_base"].numpy())


def _check_composition(fcfg, acfg):
    inp = _step_inputs(fcfg, acfg)
    hq, hkv, k_max = fcfg.hq, fcfg.hkv, fcfg.k_hi
    scale = 1.0 / math.sqrt(fcfg.head_dim)
    got = focus_step(**inp, hq=hq, hkv=hkv, k_max=k_max, scale=scale)

    delta = oracle.focus_importance_delta(inp["q0"], inp["k0"], inp["q1"], inp["k1"],
                                          inp["decoded"], hq, hkv, fcfg.pool_kernel)
    idx, count, cu = oracle.topk_select(delta, inp["k"], k_max)
    gathered = oracle.gather_rows(inp["hidden_rows"], idx, count, cu)
    ck, cv = oracle.kv_scatter(inp["new_k"], inp["new_v"], idx, count, cu, inp["row_base"],
                               inp["cache_k"], inp["cache_v"])
    n = int(cu[-1])
    widen = bf16_bits_to_f64 if ck.dtype == np.uint16 else (lambda a: a)
    out = oracle.reduced_attention(widen(inp["q_kept"][:n]), count, cu, widen(ck), widen(cv),
                                   inp["seq_start"], inp["kv_len"], hq, hkv, scale)

    np.testing.assert_array_equal(got["delta"], delta)
    for name, ref in (("idx", idx), ("count", count), ("cu", cu), ("gathered", gathered),
                      ("cache_k", ck), ("cache_v", cv), ("out", out)):
        assert np.array_equal(got[name], ref), name
    assert got["out"].shape == (n, hq, fcfg.head_dim) and np.all(np.isfinite(got["out"]))
    assert 0 < n <= fcfg.batch * k_max
    return got


def test_focus_step_tiny_equals_its_parts():
    got = _check_composition(W.TINY_FOCUS, W.TINY_ATTN)
    assert int(got["count"][0]) == 8                # K = 8 of the 32 - decoded positions


def test_focus_step_bf16_equals_its_parts():
    f = W.FocusCfg("chain_small", seed=9, batch=3, block=32, hq=8, hkv=2, head_dim=64,
                   k_lo=2, k_hi=6, hidden=128)
    a = W.AttnCfg("chain_small", seed=9, batch=3, kept=None, k_lo=2, k_hi=6, hq=8, hkv=2,
                  head_dim=64, prefix_lo=5, prefix_hi=40)
    _check_composition(f, a)


def test_focus_step_hand_worked():
    """Two sequences, block B = 8, two query heads on one KV head, D = 4, pool 1.

    Layer 0 has zero queries, so every softmax row is uniform and I0_j = hq = 2.
    Layer 1's queries are all e0 and its keys are zero except s*sqrt(D)*e0 at the
    spike key p, so every score row is s at p and 0 elsewhere. With s = ln 3 and
    B = 8, each row's softmax is 3/10 at p and 1/10 elsewhere, so I1 = 2*8*3/10 = 4.8
    at p and 1.6 elsewhere: delta = 2.8 at p and -0.4 at every other masked key.

    Sequence 0: p = 4, decoded {1, 5}, K = 3: p first, then the tie at -0.4 goes to
    the lowest indices 0 and 2 -> kept {0, 2, 4}.
    Sequence 1: p = 6, decoded {0, 1, 2}, K = 5 but k_max = 4: p, then 3, 4, 5
    -> kept {3, 4, 5, 6}.
    Every value row (cache and new) is the same vector per KV head, so each
    kept query's output is exactly that vector up to float64 rounding.
    """
    B, hq, hkv, D, s = 8, 2, 1, 4, math.log(3.0)
    spikes, decoded_at, ks = (4, 6), ((1, 5), (0, 1, 2)), (3, 5)
    q0 = np.zeros((2, B, hq, D))
    q1 = np.zeros((2, B, hq, D))
    q1[..., 0] = 1.0
    k0 = np.random.default_rng(0).normal(size=(2, B, hkv, D))     # irrelevant: q0 = 0
    k1 = np.zeros((2, B, hkv, D))
    decoded = np.zeros((2, B), np.uint8)
    for b in range(2):
        k1[b, spikes[b], :, 0] = s * math.sqrt(D)
        decoded[b, list(decoded_at[b])] = 1
    hidden = (np.arange(2 * B * 3, dtype=np.float32) + 100.0).reshape(2, B, 3)
    prefix = np.array([5, 2])
    kv_len = (prefix + B).astype(np.int32)
    seq_start = np.array([0, kv_len[0]], np.int64)
    rows = int(kv_len.sum())
    vrow = np.array([0.5, -1.25, 2.0, 3.0], np.float32)
    cache_k = np.random.default_rng(1).normal(size=(rows, hkv, D)).astype(np.float32)
    cache_v = np.broadcast_to(vrow, (rows, hkv, D)).copy()
    k_max = 4
    new_k = (np.arange(2 * k_max * D, dtype=np.float32) - 7.0).reshape(2 * k_max, hkv, D)
    new_v = np.broadcast_to(vrow, (2 * k_max, hkv, D)).copy()
    q_kept = np.random.default_rng(2).normal(size=(2 * k_max, hq, D)).astype(np.float32)
    got = focus_step(q0=q0, k0=k0, q1=q1, k1=k1, decoded=decoded, k=np.array(ks, np.int32),
                     hidden_rows=hidden, pool_kernel=1, new_k=new_k, new_v=new_v, q_kept=q_kept,
                     cache_k=cache_k, cache_v=cache_v, seq_start=seq_start, kv_len=kv_len,
                     row_base=seq_start + prefix, hq=hq, hkv=hkv, k_max=k_max, scale=0.5)

    for b in range(2):
        want = np.full(B, -0.4)
        want[spikes[b]] = 2.8
        want[list(decoded_at[b])] = -np.inf
        np.testing.assert_allclose(got["delta"][b], want, rtol=0, atol=1e-12)
    kept = ([0, 2, 4], [3, 4, 5, 6])
    np.testing.assert_array_equal(got["count"], [3, 4])
    np.testing.assert_array_equal(got["cu"], [0, 3, 7])
    np.testing.assert_array_equal(got["idx"], [[0, 2, 4, -1], [3, 4, 5, 6]])
    np.testing.assert_array_equal(got["gathered"], np.concatenate([hidden[0, kept[0]],
                                                                   hidden[1, kept[1]]]))
    ck = cache_k.copy()
    for b, t0 in ((0, 0), (1, 3)):
        for t, j in enumerate(kept[b]):
            ck[seq_start[b] + prefix[b] + j] = new_k[t0 + t]
    np.testing.assert_array_equal(got["cache_k"], ck)
    np.testing.assert_array_equal(got["cache_v"], cache_v)
    assert got["out"].shape == (7, hq, D)
    np.testing.assert_allclose(got["out"], np.broadcast_to(vrow, (7, hq, D)), rtol=1e-14, atol=0)
