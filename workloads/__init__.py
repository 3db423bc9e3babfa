"""Seeded synthetic inputs for the block token-eviction path.

This module only draws random numbers and lays them out in the shapes the
path consumes. It holds none of the method's arithmetic (no scores, no
pooling, no softmax, no selection, no attention), so that both the CPU
oracle and the HIP path can take their inputs from it without sharing any
computation.

Every tensor is drawn from its own stream: ``torch.Generator`` seeded with
``seed * 1000 + tensor_id`` on the device the tensor is made on. The same
(config, device) therefore always yields the same bytes. Small integer and
Beta draws use ``numpy.random.default_rng([seed, tensor_id])`` on the host.
Floating inputs are drawn in fp32 and rounded once (round-to-nearest-even)
to the compute dtype.

Workload shapes follow the pages' serving setting: block size B=32 and
roughly 2-4 tokens decodable per step (FOCUS paper, Section 2 and
Section 5 "Default Settings"), batch 256 (FOCUS notes page, main
experiment), an 8B-class GQA layout (32 query heads, 8 KV heads, head dim
128), and ES-dLLM's 512-token prompt with 256 generated positions and a
50 % skip ratio (ES-dLLM notes page, key design 2). The public datasets
the pages measure on are not used; these draws stand in for them.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

BF16 = torch.bfloat16
F32 = torch.float32


@dataclasses.dataclass(frozen=True)
class FocusCfg:
    """Inputs of the FOCUS scoring step (two layers of block Q/K)."""
    name: str
    seed: int
    batch: int
    block: int = 32
    hq: int = 32
    hkv: int = 8
    head_dim: int = 128
    dtype: torch.dtype = BF16
    pool_kernel: int = 7
    k_lo: int = 4             # per-sequence budget K ~ U{k_lo..k_hi}
    k_hi: int = 12
    hidden: int = 4096        # hidden size of the rows that get gathered
    decoded_frac: float | None = None   # fixed Bernoulli p; None -> p_b ~ U[0, 0.9]
    key_shift: bool = True    # shift layer-1 keys of 10 % of masked positions


@dataclasses.dataclass(frozen=True)
class AttnCfg:
    """Inputs of the KV scatter + reduced-query attention step."""
    name: str
    seed: int
    batch: int
    kept: int | None = 8      # fixed kept count; None -> K_b ~ U{k_lo..k_hi}
    k_lo: int = 4
    k_hi: int = 12
    block: int = 32
    hq: int = 32
    hkv: int = 8
    head_dim: int = 128
    dtype: torch.dtype = BF16
    prefix_lo: int = 256
    prefix_hi: int = 2048


@dataclasses.dataclass(frozen=True)
class EsCfg:
    """Inputs of the ES-dLLM early-skip scoring step."""
    name: str
    seed: int
    batch: int = 8
    prompt: int = 512
    generated: int = 256
    hidden: int = 4096
    heads: int = 32
    head_dim: int = 128
    dtype: torch.dtype = BF16
    alpha: float = 0.5
    keep: int = 128
    perturb_frac: float = 0.10
    perturb_std: float = 0.05


# The five workloads. 1: tiny fp32 step. 2: FOCUS scoring at batch 256.
# 3: attention + scatter at batch 256. 4: ES-dLLM scoring at batch 8.
# 5: the whole chain at batch 1024.
TINY_FOCUS = FocusCfg("tiny", seed=1, batch=1, block=32, hq=4, hkv=4, head_dim=64,
                      dtype=F32, pool_kernel=7, k_lo=8, k_hi=8, hidden=256,
                      decoded_frac=0.4, key_shift=False)
TINY_ATTN = AttnCfg("tiny", seed=1, batch=1, kept=8, hq=4, hkv=4, head_dim=64, dtype=F32,
                    prefix_lo=128, prefix_hi=128)
FOCUS_B256 = FocusCfg("focus_b256", seed=2, batch=256)
ATTN_B256 = AttnCfg("attn_b256", seed=3, batch=256, kept=8, prefix_lo=256, prefix_hi=2048)
ES_B8 = EsCfg("esdllm_b8", seed=4)
CHAIN_FOCUS_B1024 = FocusCfg("chain_b1024", seed=5, batch=1024)
CHAIN_ATTN_B1024 = AttnCfg("chain_b1024", seed=5, batch=1024, kept=None,
                           prefix_lo=1024, prefix_hi=4096)


def _gen(device, seed: int, tid: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + tid)
    return g


def _np(seed: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([seed, tid])


def normal(shape, seed: int, tid: int, dtype=F32, device="cpu", std: float = 1.0):
    """N(0, std^2) drawn in fp32 on `device`, then rounded to `dtype`."""
    x = torch.randn(shape, generator=_gen(device, seed, tid), device=device, dtype=F32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a (possibly bf16, possibly device) tensor to float64."""
    return t.detach().to("cpu", torch.float64).numpy()


def focus_inputs(cfg: FocusCfg, device="cpu") -> dict:
    """Layer-0/1 block Q,K ~ N(0,1), decoded mask, budgets, hidden rows.

    decoded[b, j] ~ Bernoulli(p_b); p_b ~ U[0, 0.9] unless fixed.
    Layer-1 keys: for each sequence, round(0.1 * n_masked) masked positions
    (at least 0) get +0.5 times the mean layer-1 query of the same KV head
    group (mean over block rows and the group's query heads), added in fp32
    before the rounding to the compute dtype.
    """
    B, hq, hkv, D = cfg.block, cfg.hq, cfg.hkv, cfg.head_dim
    G = hq // hkv
    n = cfg.batch
    q0 = normal((n, B, hq, D), cfg.seed, 1, cfg.dtype, device)
    k0 = normal((n, B, hkv, D), cfg.seed, 2, cfg.dtype, device)
    q1 = normal((n, B, hq, D), cfg.seed, 3, cfg.dtype, device)
    k1f = normal((n, B, hkv, D), cfg.seed, 4, F32, device)
    rng = _np(cfg.seed, 5)
    if cfg.decoded_frac is None:
        p = rng.uniform(0.0, 0.9, size=(n, 1))
    else:
        p = np.full((n, 1), cfg.decoded_frac)
    decoded = (rng.uniform(size=(n, B)) < p).astype(np.uint8)
    if cfg.key_shift:
        # mean layer-1 query per (sequence, kv head): [n, hkv, D]
        qm = q1.to(F32).reshape(n, B, hkv, G, D).mean(dim=(1, 3))
        rng2 = _np(cfg.seed, 6)
        rows, cols = [], []
        for b in range(n):
            masked = np.flatnonzero(decoded[b] == 0)
            m = int(math.floor(0.1 * masked.size + 0.5))
            if m:
                pick = rng2.choice(masked, size=m, replace=False)
                rows.extend([b] * m)
                cols.extend(pick.tolist())
        if rows:
            rb = torch.tensor(rows, device=device)
            cj = torch.tensor(cols, device=device)
            k1f[rb, cj] += 0.5 * qm[rb]
    k1 = k1f.to(cfg.dtype)
    kb = rng.integers(cfg.k_lo, cfg.k_hi + 1, size=n).astype(np.int32)
    hidden = normal((n, B, cfg.hidden), cfg.seed, 7, cfg.dtype, device)
    return dict(q0=q0, k0=k0, q1=q1, k1=k1,
                decoded=torch.from_numpy(decoded).to(device),
                k=torch.from_numpy(kb).to(device), hidden=hidden)


def attention_inputs(cfg: AttnCfg, device="cpu", capacity_rows: int | None = None) -> dict:
    """Contiguous ragged KV cache, kept-row indices, new K/V and kept queries.

    Sequence b holds L_b = P_b + B rows starting at seq_start[b]; the block
    occupies rows seq_start[b] + P_b .. + B - 1 (row_base[b] = seq_start[b] + P_b).
    P_b ~ U{prefix_lo..prefix_hi}. Kept block positions: `kept` (or
    K_b ~ U{k_lo..k_hi}) distinct positions drawn uniformly from the block,
    sorted ascending. Cache K/V, new K/V and queries ~ N(0,1).
    """
    n, B = cfg.batch, cfg.block
    rng = _np(cfg.seed, 20)
    prefix = rng.integers(cfg.prefix_lo, cfg.prefix_hi + 1, size=n).astype(np.int64)
    kv_len = (prefix + B).astype(np.int32)
    seq_start = np.zeros(n, np.int64)
    seq_start[1:] = np.cumsum(kv_len.astype(np.int64))[:-1]
    rows = int(kv_len.astype(np.int64).sum())
    if cfg.kept is None:
        count = rng.integers(cfg.k_lo, cfg.k_hi + 1, size=n).astype(np.int32)
    else:
        count = np.full(n, cfg.kept, np.int32)
    k_max = cfg.k_hi if cfg.kept is None else cfg.kept
    idx = np.full((n, k_max), -1, np.int32)
    rng2 = _np(cfg.seed, 21)
    for b in range(n):
        idx[b, :count[b]] = np.sort(rng2.choice(B, size=count[b], replace=False))
    cu = np.zeros(n + 1, np.int32)
    cu[1:] = np.cumsum(count)
    total = int(cu[-1]) if capacity_rows is None else max(capacity_rows, int(cu[-1]))
    hkv, hq, D = cfg.hkv, cfg.hq, cfg.head_dim
    cache_k = normal((rows, hkv, D), cfg.seed, 22, cfg.dtype, device)
    cache_v = normal((rows, hkv, D), cfg.seed, 23, cfg.dtype, device)
    new_k = normal((total, hkv, D), cfg.seed, 24, cfg.dtype, device)
    new_v = normal((total, hkv, D), cfg.seed, 25, cfg.dtype, device)
    q = normal((total, hq, D), cfg.seed, 26, cfg.dtype, device)
    t = lambda a: torch.from_numpy(a).to(device)
    return dict(cache_k=cache_k, cache_v=cache_v, new_k=new_k, new_v=new_v, q=q,
                prefix=t(prefix), kv_len=t(kv_len), seq_start=t(seq_start),
                row_base=t(seq_start + prefix), idx=t(idx), count=t(count), cu=t(cu),
                k_max=k_max, rows=rows, max_kv_len=int(kv_len.max()))


def esdllm_inputs(cfg: EsCfg, device="cpu") -> dict:
    """ES-dLLM scoring inputs: previous hidden states, survivors' new states.

    H_prev[b] ~ N(0,1) over all prompt + generated positions. The survivor
    set is every generated position (surv_pos = prompt .. prompt+generated-1).
    H_new equals H_prev at the survivor positions, except on
    round(perturb_frac * generated) survivors per sequence, which get
    + N(0, perturb_std^2) noise (added in fp32 before rounding).
    Confidence c ~ Beta(0.5, 2) in fp32 over all positions.
    """
    n, L, h = cfg.batch, cfg.prompt + cfg.generated, cfg.hidden
    hprev_f = normal((n, L, h), cfg.seed, 30, F32, device)
    h_prev = hprev_f.to(cfg.dtype)
    surv = np.tile(np.arange(cfg.prompt, L, dtype=np.int32), (n, 1))
    hnew_f = h_prev[:, cfg.prompt:].to(F32).clone()
    noise = normal((n, cfg.generated, h), cfg.seed, 31, F32, device, std=cfg.perturb_std)
    rng = _np(cfg.seed, 32)
    m = int(math.floor(cfg.perturb_frac * cfg.generated + 0.5))
    mask = np.zeros((n, cfg.generated), bool)
    for b in range(n):
        mask[b, rng.choice(cfg.generated, size=m, replace=False)] = True
    mt = torch.from_numpy(mask).to(device)
    hnew_f[mt] += noise[mt]
    h_new = hnew_f.to(cfg.dtype)
    conf = _np(cfg.seed, 33).beta(0.5, 2.0, size=(n, L)).astype(np.float32)
    kkeep = np.full(n, cfg.keep, np.int32)
    D = cfg.head_dim
    new_k = normal((n * cfg.keep, cfg.heads, D), cfg.seed, 34, cfg.dtype, device)
    new_v = normal((n * cfg.keep, cfg.heads, D), cfg.seed, 35, cfg.dtype, device)
    cache_k = normal((n * L, cfg.heads, D), cfg.seed, 36, cfg.dtype, device)
    cache_v = normal((n * L, cfg.heads, D), cfg.seed, 37, cfg.dtype, device)
    t = lambda a: torch.from_numpy(a).to(device)
    return dict(h_new=h_new, h_prev=h_prev, surv_pos=t(surv), conf=t(conf),
                perturbed=t(mask), k=t(kkeep), new_k=new_k, new_v=new_v,
                cache_k=cache_k, cache_v=cache_v,
                row_base=t(np.arange(n, dtype=np.int64) * L), alpha=cfg.alpha)


def es_pipeline_inputs(cfg: EsCfg, layers: int = 2, device="cpu") -> dict:
    """Inputs of ES-dLLM's skip layers (one per layer in `layers`): per layer,
    the previous iteration's hidden states h_cache [batch, L, h] ~ N(0,1) and
    this iteration's h_cur = h_cache + N(0, perturb_std^2) on
    round(perturb_frac * L) positions per sequence (exact copy elsewhere);
    one confidence c ~ Beta(0.5, 2) [batch, L]; the first skip layer's
    survivors are every generated position. h_cur stands for the layer's
    output, which the pages' model would compute for the survivors."""
    n, L, h = cfg.batch, cfg.prompt + cfg.generated, cfg.hidden
    out = {"h_cache": [], "h_cur": []}
    m = int(math.floor(cfg.perturb_frac * L + 0.5))
    for layer in range(layers):
        base = normal((n, L, h), cfg.seed, 50 + 10 * layer, F32, device)
        cur = base.clone()
        noise = normal((n, L, h), cfg.seed, 51 + 10 * layer, F32, device, std=cfg.perturb_std)
        rng = _np(cfg.seed, 52 + 10 * layer)
        mask = np.zeros((n, L), bool)
        for b in range(n):
            mask[b, rng.choice(L, size=m, replace=False)] = True
        mt = torch.from_numpy(mask).to(device)
        cur[mt] += noise[mt]
        out["h_cache"].append(base.to(cfg.dtype))
        out["h_cur"].append(cur.to(cfg.dtype))
    out["conf"] = torch.from_numpy(_np(cfg.seed, 59).beta(0.5, 2.0, size=(n, L)).astype(np.float32)).to(device)
    out["surv_pos"] = torch.from_numpy(np.tile(np.arange(cfg.prompt, L, dtype=np.int32), (n, 1))).to(device)
    out["alpha"] = cfg.alpha
    return out


def chain_inputs(fcfg: FocusCfg, acfg: AttnCfg, device="cpu") -> dict:
    """Inputs of one full FOCUS step: scoring inputs of `fcfg` plus the KV cache,
    capacity-sized new K/V and kept-query buffers (batch * k_hi rows) of `acfg`."""
    assert fcfg.batch == acfg.batch and fcfg.block == acfg.block
    fi = focus_inputs(fcfg, device)
    ai = attention_inputs(acfg, device, capacity_rows=fcfg.batch * fcfg.k_hi)
    return dict(q0=fi["q0"], k0=fi["k0"], q1=fi["q1"], k1=fi["k1"], decoded=fi["decoded"],
                k=fi["k"], hidden_rows=fi["hidden"], pool_kernel=fcfg.pool_kernel,
                new_k=ai["new_k"], new_v=ai["new_v"], q_kept=ai["q"], cache_k=ai["cache_k"],
                cache_v=ai["cache_v"], seq_start=ai["seq_start"], kv_len=ai["kv_len"],
                row_base=ai["row_base"], prefix=ai["prefix"], rows=ai["rows"])


def page_table(kv_len, page_size: int, seed: int, spare: int = 0):
    """A shuffled page pool for sequences of kv_len rows: block_table int32
    [batch, max_pages] (sequence b's logical page p lives in pool page
    block_table[b, p]; -1 past its last page) and the pool's page count.
    Pages are handed out in a random permutation of the pool, so the pages
    of one sequence are scattered over it."""
    kv_len = np.asarray(kv_len, np.int64)
    need = (kv_len + page_size - 1) // page_size
    n_pages = int(need.sum()) + spare
    perm = _np(seed, 70).permutation(n_pages).astype(np.int32)
    bt = np.full((kv_len.size, int(need.max())), -1, np.int32)
    at = 0
    for b in range(kv_len.size):
        bt[b, :need[b]] = perm[at:at + need[b]]
        at += int(need[b])
    return bt, n_pages


def focus_full_inputs(fcfg: FocusCfg, acfg: AttnCfg, page_size: int = 64, device="cpu",
                      base: dict | None = None) -> dict:
    """Inputs of the extended FOCUS step (device budget, constrained selection,
    multi-tensor compaction, paged KV pool, delayed commit, history update), on
    top of `chain_inputs` (passed as `base` or drawn here).

    Per-sequence decode state, drawn once:
      total_steps ~ U{0..30}; token_sum ~ U{2 total_steps .. 4 total_steps}
        (2-4 tokens per past step);
      rightmost_processed ~ U{-1..B-1};
      cached = decoded AND Bernoulli(0.5);
      decoded_now = decoded plus U{2..4} of the masked positions (all of them
        if fewer are masked): the tokens this step decodes.
    Per-token tensors compacted with the kept rows: the hidden rows of
    `chain_inputs`, an fp32 residual [batch, B, hidden] ~ N(0,1), RoPE
    positions P_b + j (int32) and cache row indices seq_start[b] + P_b + j
    (int64). Capacity buffers hold batch * B rows (|S| can reach B). The KV
    pool is `page_table`'s shuffled pages of `page_size` rows, K/V ~ N(0,1).
    """
    x = chain_inputs(fcfg, acfg, device) if base is None else base
    n, B, H = fcfg.batch, fcfg.block, fcfg.hidden
    hq, hkv, D = acfg.hq, acfg.hkv, acfg.head_dim
    seed = fcfg.seed
    rng = _np(seed, 60)
    steps = rng.integers(0, 31, size=n).astype(np.int64)
    token_sum = np.array([rng.integers(2 * s, 4 * s + 1) for s in steps], np.int64)
    rp = rng.integers(-1, B, size=n).astype(np.int32)
    dec = x["decoded"].cpu().numpy().astype(bool)
    cached = dec & (rng.uniform(size=(n, B)) < 0.5)
    now = dec.copy()
    rng2 = _np(seed, 61)
    for b in range(n):
        masked = np.flatnonzero(~dec[b])
        m = min(masked.size, int(rng2.integers(2, 5)))
        if m:
            now[b, rng2.choice(masked, size=m, replace=False)] = True
    prefix = x["prefix"].cpu().numpy().astype(np.int64)
    seq_start = x["seq_start"].cpu().numpy().astype(np.int64)
    j = np.arange(B, dtype=np.int64)
    rope_pos = (prefix[:, None] + j[None, :]).astype(np.int32)
    cache_idx = (seq_start + prefix)[:, None] + j[None, :]
    bt, n_pages = page_table(x["kv_len"].cpu().numpy(), page_size, seed, spare=3)
    cap = n * B
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(
        x, decoded_now=t(now.astype(np.uint8)), token_sum=t(token_sum.astype(np.int32)),
        total_steps=t(steps.astype(np.int32)), rightmost_processed=t(rp),
        cached=t(cached.astype(np.uint8)),
        residual=normal((n, B, H), seed, 62, F32, device), rope_pos=t(rope_pos),
        cache_idx=t(cache_idx), pos_base=t(prefix.astype(np.int32)),
        new_k_full=normal((cap, hkv, D), seed, 63, acfg.dtype, device),
        new_v_full=normal((cap, hkv, D), seed, 64, acfg.dtype, device),
        q_full=normal((cap, hq, D), seed, 65, acfg.dtype, device),
        block_table=t(bt), page_size=page_size,
        pool_k=normal((n_pages * page_size, hkv, D), seed, 66, acfg.dtype, device),
        pool_v=normal((n_pages * page_size, hkv, D), seed, 67, acfg.dtype, device))
