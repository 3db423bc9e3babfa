"""The seeded generators are deterministic and produce the documented shapes."""
import numpy as np
import torch

import workloads as W


def test_focus_inputs_deterministic_and_shaped():
    a = W.focus_inputs(W.TINY_FOCUS)
    b = W.focus_inputs(W.TINY_FOCUS)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert a["q0"].shape == (1, 32, 4, 64) and a["q0"].dtype == torch.float32
    assert a["decoded"].dtype == torch.uint8
    c = W.focus_inputs(W.FocusCfg("t", seed=9, batch=6, hq=8, hkv=2, head_dim=16, hidden=32))
    assert c["q1"].dtype == torch.bfloat16 and c["k1"].shape == (6, 32, 2, 16)
    assert int(c["k"].min()) >= 4 and int(c["k"].max()) <= 12


def test_attention_inputs_layout():
    a = W.attention_inputs(W.AttnCfg("t", seed=3, batch=5, hq=8, hkv=2, head_dim=16,
                                     prefix_lo=10, prefix_hi=40))
    kv = a["kv_len"].numpy().astype(np.int64)
    ss = a["seq_start"].numpy()
    assert ss[0] == 0 and np.all(ss[1:] == np.cumsum(kv)[:-1])
    assert a["cache_k"].shape[0] == kv.sum() == a["rows"]
    assert np.all(a["row_base"].numpy() == ss + a["prefix"].numpy())
    idx, cnt = a["idx"].numpy(), a["count"].numpy()
    for b in range(5):
        assert np.all(np.diff(idx[b, :cnt[b]]) > 0) and idx[b, :cnt[b]].max() < 32


def test_esdllm_inputs_copy_structure():
    cfg = W.EsCfg("t", seed=4, batch=2, prompt=16, generated=32, hidden=64, heads=2,
                  head_dim=8, keep=16)
    a = W.esdllm_inputs(cfg)
    same = (a["h_new"] == a["h_prev"][:, 16:]).all(-1)
    assert torch.equal(~same | a["perturbed"], a["perturbed"])    # only perturbed rows differ
    assert int(a["perturbed"].sum()) == 2 * 3
