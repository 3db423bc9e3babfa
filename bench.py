"""Throughput of the block token-eviction hot path on one MI355X.

One step = one pass of the FOCUS chain over the batch-1024 workload
(block 32, 32 query / 8 KV heads, head dim 128, bf16, MaxPool 7, budgets
K ~ U{4..12}, prefixes ~ U{1024..4096}, hidden 4096), all on one stream:

    importance delta (layers 0/1) -> top-K -> gather -> KV scatter
        -> longest-first attention order -> reduced attention

Prints one JSON line: block tokens/s (batch * block / step time, with the K
timed steps captured as one HIP graph and replayed once; the eager step time,
launched call by call, is reported beside it), per-kernel average durations
from HIP events recorded on the launch stream in the eager loop, the
roofline of the dominant kernel (reduced attention, HBM-bound) from its
algorithmic bytes, and the CPU oracle timed on a bounded sample of the same
workload.

Other legs, each reported under its own key:
  focus_b256           FOCUS scoring at batch 256 (delta -> top-K -> gather),
  attn_b256            KV scatter -> order -> attention at batch 256,
  focus_b1024_block64  the scoring path with blocks of 64 positions,
  focus_b2048_block16  the scoring path with blocks of 16 positions,
  es_mode              ES-dLLM score -> top-K -> gather -> KV scatter, batch 8,
  es_pipeline          two ES-dLLM skip layers (256 -> 128 -> 64 survivors),
  es_iteration         ES-dLLM iterations with the device bookkeeping and a
                       refresh every third iteration,
  fused_scatter_attention, full_step, score_resident (see their functions).
The batch-256, block-64 and ES legs read a 1 GiB buffer before every timed
iteration (outside the events), so their inputs come from HBM and not from the
256 MB Infinity Cache, and time each kernel with HIP events (medians).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--legs all|main|name,name,...]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
ALPHA = 1.5                    # FOCUS budget multiplier of the pages' worked example
PAGE = 64                      # KV pool page size (rows) of the extended step
FLUSH_BYTES = 1 << 30          # read before each timed iteration of the flushed legs
LEG_ITERS = 30                 # timed iterations of each flushed leg
METRIC = "block tokens/s through score→top-K→gather→reduced attn; % of HBM/MFMA roofline"
LEGS = ["focus_b256", "attn_b256", "focus_b1024_block64", "chain_b1024_block64",
        "focus_b2048_block16", "es_mode",
        "es_pipeline",
        "es_iteration", "fused_scatter_attention", "full_step", "score_resident"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--legs", default="all",
                    help="'all', 'main' (the main step only) or a comma list of leg names")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path shards by sequence with no exchange, "
              "so run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    legs = LEGS if args.legs == "all" else ([] if args.legs == "main" else args.legs.split(","))
    unknown = [l for l in legs if l not in LEGS]
    if unknown:
        print(f"unknown legs {unknown}; known: {LEGS}", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_token_eviction_amd as bte
    from block_token_eviction_amd.chain import FocusStep
    import workloads as W

    dev = torch.device("cuda:0")
    fc, ac = W.CHAIN_FOCUS_B1024, W.CHAIN_ATTN_B1024
    log("generating inputs on the device")
    x = W.chain_inputs(fc, ac, device=dev)
    # length order for the attention: with at most 12 kept rows (48 query rows per KV head)
    # every sequence is one 64-row query pass, so weighing by passes would change nothing
    step = FocusStep(fc.batch, fc.block, fc.hidden, fc.hq, fc.head_dim, fc.k_hi, fc.dtype, dev)
    run_args = {k: x[k] for k in ("q0", "k0", "q1", "k1", "decoded", "k", "hidden_rows",
                                  "pool_kernel", "new_k", "new_v", "q_kept", "cache_k", "cache_v",
                                  "seq_start", "kv_len", "row_base")}
    stages = [
        ("focus_importance_delta", lambda: step.score(x["q0"], x["k0"], x["q1"], x["k1"], x["decoded"], fc.pool_kernel)),
        ("topk_select", lambda: step.select(x["k"])),
        ("gather_rows", lambda: step.gather(x["hidden_rows"])),
        ("kv_scatter", lambda: step.scatter(x["new_k"], x["new_v"], x["row_base"], x["cache_k"], x["cache_v"])),
        ("attention_order", lambda: step.schedule(x["kv_len"])),
        ("reduced_attention", lambda: step.attend(x["q_kept"], x["cache_k"], x["cache_v"], x["seq_start"], x["kv_len"])),
    ]
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step.run(**run_args)
    torch.cuda.synchronize()

    # timed region: exactly `steps` full steps, per-stage events on the launch stream
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in stages] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, (_, fn) in enumerate(stages):
            ev[s][i][0].record()
            fn()
            ev[s][i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    step_ms = sorted(ev[s][0][0].elapsed_time(ev[s][-1][1]) for s in range(args.steps))
    stage_ms = {name: float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]))
                for i, (name, _) in enumerate(stages)}

    # algorithmic bytes per launch (counts read back after the timed region)
    count = step.count.cpu().numpy().astype(np.int64)
    sum_k = int(count.sum())
    kv_len = x["kv_len"].cpu().numpy().astype(np.int64)
    es = 2
    B, hq, hkv, D, H = fc.block, fc.hq, fc.hkv, fc.head_dim, fc.hidden
    bytes_ = {
        "focus_importance_delta": delta_bytes(fc.batch, B, hq, hkv, D, es),
        "topk_select": fc.batch * B * 4 + fc.batch * 4 + fc.batch * (fc.k_hi + 2) * 4,
        "gather_rows": 2 * sum_k * H * es,
        "kv_scatter": 2 * 2 * sum_k * hkv * D * es,
        "attention_order": 2 * fc.batch * 4,
        "reduced_attention": attention_bytes(kv_len, sum_k, hq, hkv, D, es),
    }
    flops_attn = attention_flops(count, kv_len, hq, D)
    kernels = {n: {"ms": round(stage_ms[n], 4), "algo_bytes": int(bytes_[n]),
                   "GB/s": round(bytes_[n] / (stage_ms[n] * 1e-3) / 1e9, 1),
                   "hbm_frac": round(bytes_[n] / (stage_ms[n] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
               for n in stage_ms}
    # matrix-core work of the score tiles: S = Q K^T for 2 layers, every (sequence, query head)
    flops_score = score_flops(fc.batch, B, hq, D)
    kernels["focus_importance_delta"]["tflops"] = round(
        flops_score / (stage_ms["focus_importance_delta"] * 1e-3) / 1e12, 2)
    kernels["reduced_attention"]["tflops"] = round(
        flops_attn / (stage_ms["reduced_attention"] * 1e-3) / 1e12, 2)
    dom = "reduced_attention"
    achieved = bytes_[dom] / (stage_ms[dom] * 1e-3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "algo_bytes_per_launch": int(bytes_[dom]), "event_us": round(stage_ms[dom] * 1e3, 1),
                "tflops": round(flops_attn / (stage_ms[dom] * 1e-3) / 1e12, 2)}
    roofline.update(trace_roofline(dom, bytes_[dom]))
    copy_gbs = copy_bandwidth(dev)
    roofline["copy_GBps"] = round(copy_gbs, 1)
    roofline["frac_of_copy"] = round(achieved / copy_gbs, 4)
    # the gather and the scatter are copies (every byte read once, written once): their
    # rate against the same measured device copy as well
    for n in ("gather_rows", "kv_scatter"):
        kernels[n]["frac_of_copy"] = round(kernels[n]["GB/s"] / copy_gbs, 4)

    # The K timed steps captured as one HIP graph and replayed once: the same
    # kernels in the same order, without the host's per-launch gaps (the way a
    # serving loop runs the step). `value` is taken from this replay; the eager
    # loop above gives the per-kernel event times and the eager step time.
    graph_ms = graph_step_ms(lambda: step.run(**run_args), args.steps)
    timing = "hip_graph" if graph_ms is not None else "eager"
    ms_value = graph_ms if graph_ms is not None else ms_step
    value = fc.batch * fc.block / (ms_value * 1e-3)

    flush = Flush(dev)
    out_legs = {}
    leg_fns = {
        "focus_b256": lambda: focus_b256_leg(dev, flush),
        "attn_b256": lambda: attn_b256_leg(dev, flush),
        "focus_b1024_block64": lambda: focus_block64_leg(dev, flush),
        "chain_b1024_block64": lambda: chain_block64_leg(dev, args.steps, args.warmup),
        "focus_b2048_block16": lambda: focus_block16_leg(dev, flush),
        "es_mode": lambda: es_mode_leg(dev, flush, args.steps),
        "es_pipeline": lambda: es_pipeline_leg(dev, flush, args.steps),
        "es_iteration": lambda: es_iteration_leg(dev, flush),
        "fused_scatter_attention": lambda: fused_scatter_attention_leg(step, x, args.steps, bytes_),
        "full_step": lambda: full_step_leg(x, fc, ac, args.steps, args.warmup, dev),
        "score_resident": lambda: score_resident_leg(dev),
    }
    for name in legs:
        log(f"leg {name}")
        out_legs[name] = leg_fns[name]()
        torch.cuda.synchronize()
    del flush

    if args.copy_calibration:
        src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    roofline["traffic"] = measured_traffic(dom)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, fc, ac)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "block tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_value, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/hidden, Bernoulli decoded mask, U{4..12} budgets)",
        "config": {"workload": "chain_b1024", "batch": fc.batch, "block": fc.block, "hq": hq,
                   "hkv": hkv, "head_dim": D, "hidden": H, "pool_kernel": fc.pool_kernel,
                   "k_range": [fc.k_lo, fc.k_hi], "prefix_range": [ac.prefix_lo, ac.prefix_hi],
                   "kept_rows": sum_k, "kv_rows": int(kv_len.sum()), "parallelism": "none (1 GPU)"},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels, "timing": timing,
        "eager_ms_per_step": round(ms_step, 4),
        "graph_ms_per_step": round(graph_ms, 4) if graph_ms is not None else None,
        "eager_step_ms_p10_p50_p90": [round(percentile(step_ms, q), 4) for q in (10, 50, 90)],
    }
    line.update(out_legs)
    print(json.dumps(line), flush=True)


COPY_CAL_BYTES = 256 << 20


def delta_bytes(batch: int, block: int, hq: int, hkv: int, head_dim: int, es: int) -> int:
    """Importance delta: Q and K of both layers read once, the mask read and the delta written."""
    return 2 * batch * block * (hq + hkv) * head_dim * es + batch * block * (1 + 4)


def attention_bytes(kv_len, sum_k: int, hq: int, hkv: int, head_dim: int, es: int) -> int:
    """Reduced attention: every K and V row of every sequence read once, the kept queries
    read and their outputs written."""
    return int(kv_len.sum()) * hkv * head_dim * es * 2 + 2 * sum_k * hq * head_dim * es


def attention_flops(count, kv_len, hq: int, head_dim: int) -> int:
    return int(sum(4 * int(c) * hq * int(l) * head_dim for c, l in zip(count, kv_len)))


class Flush:
    """A 1 GiB device buffer read (one reduction) before each timed iteration of a
    flushed leg, so that the leg's inputs are not served from the L2 or the 256 MB
    Infinity Cache. Reading leaves clean lines behind: a buffer written instead
    leaves the caches full of dirty lines, whose write-back then lands in the timed
    kernels (measured: +6 to 7 us on the batch-256 attention, +2 us on the delta)."""

    def __init__(self, dev, nbytes: int = FLUSH_BYTES):
        import torch
        self.buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)

    def __call__(self):
        self.buf.sum()


def timed_stages(stages, iters: int, flush, warm: int = 3, between=None):
    """Per-stage HIP-event times (ms) of `iters` iterations, with flush() before each
    (outside the events). between(i) runs before stage i (outside the events: work that
    stands for the model, not the path). Returns ({stage: sorted times}, sorted step
    times from the first stage's start to the last one's end, [per-iteration sums])."""
    import torch
    E = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(warm):
        flush()
        for i, (_, fn) in enumerate(stages):
            if between:
                between(i)
            fn()
    torch.cuda.synchronize()
    ev = [[(E(), E()) for _ in stages] for _ in range(iters)]
    for it in range(iters):
        flush()
        for i, (_, fn) in enumerate(stages):
            if between:
                between(i)
            ev[it][i][0].record()
            fn()
            ev[it][i][1].record()
    torch.cuda.synchronize()
    per = {name: sorted(ev[it][i][0].elapsed_time(ev[it][i][1]) for it in range(iters))
           for i, (name, _) in enumerate(stages)}
    sums = [sum(ev[it][i][0].elapsed_time(ev[it][i][1]) for i in range(len(stages)))
            for it in range(iters)]
    step = sorted(ev[it][0][0].elapsed_time(ev[it][-1][1]) for it in range(iters))
    return per, step, sums


def leg_kernels(per: dict, bytes_: dict, flops: dict | None = None) -> dict:
    """Median time, algorithmic bytes, the HBM bound on that many bytes (8 TB/s) and the
    achieved fraction of it, per kernel."""
    out = {}
    for name, ts in per.items():
        ms = percentile(ts, 50)
        b = int(bytes_[name])
        k = {"ms_p50": round(ms, 4), "ms_p10_p90": [round(percentile(ts, 10), 4),
                                                    round(percentile(ts, 90), 4)],
             "algo_bytes": b, "bound_us": round(b / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
             "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
             "hbm_frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if flops and name in flops:
            k["tflops"] = round(flops[name] / (ms * 1e-3) / 1e12, 2)
            k["frac_of_bf16_dense_peak"] = round(flops[name] / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
        out[name] = k
    return out


FLUSHED = "eager, 1 GiB buffer read before each iteration, per-kernel HIP events (medians)"


def focus_b256_leg(dev, flush):
    """FOCUS scoring at batch 256 (32 query / 8 KV heads, head dim 128, bf16, MaxPool 7,
    K ~ U{4..12}, hidden 4096): importance delta -> top-K -> gather."""
    import torch
    from block_token_eviction_amd.chain import FocusStep
    import workloads as W

    cfg = W.FOCUS_B256
    fi = W.focus_inputs(cfg, device=dev)
    st = FocusStep(cfg.batch, cfg.block, cfg.hidden, cfg.hq, cfg.head_dim, cfg.k_hi, cfg.dtype, dev)
    stages = [
        ("focus_importance_delta", lambda: st.score(fi["q0"], fi["k0"], fi["q1"], fi["k1"], fi["decoded"], cfg.pool_kernel)),
        ("topk_select", lambda: st.select(fi["k"])),
        ("gather_rows", lambda: st.gather(fi["hidden"])),
    ]
    per, step, _ = timed_stages(stages, LEG_ITERS, flush)
    sum_k = int(st.count.sum().item())
    n, B = cfg.batch, cfg.block
    bytes_ = {"focus_importance_delta": delta_bytes(n, B, cfg.hq, cfg.hkv, cfg.head_dim, 2),
              "topk_select": n * B * 4 + n * 4 + n * (cfg.k_hi + 2) * 4,
              "gather_rows": 2 * sum_k * cfg.hidden * 2}
    flops = {"focus_importance_delta": score_flops(n, B, cfg.hq, cfg.head_dim)}
    med = percentile(step, 50)
    return {"workload": "focus_b256 (batch 256, block 32, 32q/8kv heads, head dim 128, bf16, "
                        "MaxPool 7, K ~ U{4..12}, hidden 4096)", "timing": FLUSHED,
            "kept_rows": sum_k,
            "ms_per_step_p10_p50_p90": [round(percentile(step, q), 4) for q in (10, 50, 90)],
            "block tokens/s": round(n * B / (med * 1e-3), 1),
            "kernels": leg_kernels(per, bytes_, flops)}


def attn_b256_leg(dev, flush):
    """KV scatter + reduced attention at batch 256: 8 kept queries per sequence, 32q/8kv
    heads, head dim 128, bf16, prefixes ~ U{256..2048} plus the 32-position block."""
    import numpy as np
    import torch
    import block_token_eviction_amd as bte
    import workloads as W

    cfg = W.ATTN_B256
    ai = W.attention_inputs(cfg, device=dev)
    order = torch.empty((cfg.batch,), dtype=torch.int32, device=dev)
    out = torch.empty_like(ai["q"])
    stages = [
        ("kv_scatter", lambda: bte.kv_scatter(ai["new_k"], ai["new_v"], ai["idx"], ai["count"], ai["cu"], ai["row_base"], ai["cache_k"], ai["cache_v"])),
        ("attention_order", lambda: bte.attention_order(ai["kv_len"], out=order)),
        ("reduced_attention", lambda: bte.reduced_attention(ai["q"], ai["count"], ai["cu"], ai["cache_k"], ai["cache_v"], ai["seq_start"], ai["kv_len"], ai["k_max"], out=out, order=order)),
    ]
    per, step, _ = timed_stages(stages, LEG_ITERS, flush)
    count = ai["count"].cpu().numpy().astype(np.int64)
    kv_len = ai["kv_len"].cpu().numpy().astype(np.int64)
    sum_k = int(count.sum())
    bytes_ = {"kv_scatter": 2 * 2 * sum_k * cfg.hkv * cfg.head_dim * 2,
              "attention_order": 2 * cfg.batch * 4,
              "reduced_attention": attention_bytes(kv_len, sum_k, cfg.hq, cfg.hkv, cfg.head_dim, 2)}
    flops = {"reduced_attention": attention_flops(count, kv_len, cfg.hq, cfg.head_dim)}
    med = percentile(step, 50)
    return {"workload": "attn_b256 (batch 256, 8 kept per sequence, 32q/8kv heads, head dim 128, "
                        "bf16, prefixes U{256..2048} + 32)", "timing": FLUSHED,
            "kept_rows": sum_k, "kv_rows": int(kv_len.sum()),
            "ms_per_step_p10_p50_p90": [round(percentile(step, q), 4) for q in (10, 50, 90)],
            "block tokens/s": round(cfg.batch * cfg.block / (med * 1e-3), 1),
            "kernels": leg_kernels(per, bytes_, flops)}


def focus_block_leg(dev, flush, batch: int, block: int, k_lo: int, k_hi: int, seed: int):
    """The scoring path at another block size: delta -> top-K -> gather, 32q/8kv heads,
    head dim 128, bf16, MaxPool 7, hidden 4096, K ~ U{k_lo..k_hi}."""
    from block_token_eviction_amd.chain import FocusStep
    import workloads as W

    name = f"focus_b{batch}_block{block}"
    cfg = W.FocusCfg(name, seed=seed, batch=batch, block=block, k_lo=k_lo, k_hi=k_hi)
    fi = W.focus_inputs(cfg, device=dev)
    st = FocusStep(cfg.batch, cfg.block, cfg.hidden, cfg.hq, cfg.head_dim, cfg.k_hi, cfg.dtype, dev)
    stages = [
        ("focus_importance_delta", lambda: st.score(fi["q0"], fi["k0"], fi["q1"], fi["k1"], fi["decoded"], cfg.pool_kernel)),
        ("topk_select", lambda: st.select(fi["k"])),
        ("gather_rows", lambda: st.gather(fi["hidden"])),
    ]
    per, step, _ = timed_stages(stages, LEG_ITERS // 2, flush)
    sum_k = int(st.count.sum().item())
    n, B = cfg.batch, cfg.block
    bytes_ = {"focus_importance_delta": delta_bytes(n, B, cfg.hq, cfg.hkv, cfg.head_dim, 2),
              "topk_select": n * B * 4 + n * 4 + n * (cfg.k_hi + 2) * 4,
              "gather_rows": 2 * sum_k * cfg.hidden * 2}
    flops = {"focus_importance_delta": score_flops(n, B, cfg.hq, cfg.head_dim)}
    med = percentile(step, 50)
    res = {"workload": f"{name} (batch {batch}, block {block}, 32q/8kv heads, head dim 128, "
                       f"bf16, MaxPool 7, K ~ U{{{k_lo}..{k_hi}}}, hidden 4096)", "timing": FLUSHED,
           "kept_rows": sum_k,
           "ms_per_step_p10_p50_p90": [round(percentile(step, q), 4) for q in (10, 50, 90)],
           "block tokens/s": round(n * B / (med * 1e-3), 1),
           "kernels": leg_kernels(per, bytes_, flops)}
    del fi
    return res


def focus_block64_leg(dev, flush):
    """Blocks of 64 positions (the FOCUS paper's largest block) at batch 1024; K ~ U{8..24},
    the batch-256 budget range scaled with the block."""
    return focus_block_leg(dev, flush, 1024, 64, 8, 24, seed=6)


def chain_block64_leg(dev, steps: int, warmup: int):
    """The whole step at blocks of 64 (batch 1024, K ~ U{8..24}, prefixes 1024..4096 + 64):
    delta -> top-K -> gather -> scatter -> order -> attention, timed like the main step
    (per-stage events over `steps` eager steps after `warmup`, and the warm HIP-graph
    replay). Up to 96 query rows per KV head: the attention takes the query split."""
    import numpy as np
    import torch

    from block_token_eviction_amd.chain import FocusStep
    import workloads as W

    name = "chain_b1024_block64"
    fc = W.FocusCfg(name, seed=8, batch=1024, block=64, k_lo=8, k_hi=24)
    ac = W.AttnCfg(name, seed=8, batch=1024, kept=None, k_lo=8, k_hi=24, block=64,
                   prefix_lo=1024, prefix_hi=4096)
    x = W.chain_inputs(fc, ac, device=dev)
    st = FocusStep(fc.batch, fc.block, fc.hidden, fc.hq, fc.head_dim, fc.k_hi, fc.dtype, dev)
    run_args = {k: x[k] for k in ("q0", "k0", "q1", "k1", "decoded", "k", "hidden_rows",
                                  "pool_kernel", "new_k", "new_v", "q_kept", "cache_k", "cache_v",
                                  "seq_start", "kv_len", "row_base")}
    stages = [
        ("focus_importance_delta", lambda: st.score(x["q0"], x["k0"], x["q1"], x["k1"], x["decoded"], fc.pool_kernel)),
        ("topk_select", lambda: st.select(x["k"])),
        ("gather_rows", lambda: st.gather(x["hidden_rows"])),
        ("kv_scatter", lambda: st.scatter(x["new_k"], x["new_v"], x["row_base"], x["cache_k"], x["cache_v"])),
        ("attention_order", lambda: st.schedule(x["kv_len"])),
        ("reduced_attention", lambda: st.attend(x["q_kept"], x["cache_k"], x["cache_v"], x["seq_start"], x["kv_len"])),
    ]
    for _ in range(warmup):
        st.run(**run_args)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[(E(), E()) for _ in stages] for _ in range(steps)]
    for it in range(steps):
        for i, (_, fn) in enumerate(stages):
            ev[it][i][0].record()
            fn()
            ev[it][i][1].record()
    torch.cuda.synchronize()
    stage_ms = {n_: float(np.mean([ev[it][i][0].elapsed_time(ev[it][i][1]) for it in range(steps)]))
                for i, (n_, _) in enumerate(stages)}
    graph_ms = graph_step_ms(lambda: st.run(**run_args), steps)
    count = st.count.cpu().numpy().astype(np.int64)
    sum_k = int(count.sum())
    kv_len = x["kv_len"].cpu().numpy().astype(np.int64)
    n, B, hq, hkv, D, H = fc.batch, fc.block, fc.hq, fc.hkv, fc.head_dim, fc.hidden
    bytes_ = {"focus_importance_delta": delta_bytes(n, B, hq, hkv, D, 2),
              "topk_select": n * B * 4 + n * 4 + n * (fc.k_hi + 2) * 4,
              "gather_rows": 2 * sum_k * H * 2,
              "kv_scatter": 2 * 2 * sum_k * hkv * D * 2,
              "attention_order": 2 * n * 4,
              "reduced_attention": attention_bytes(kv_len, sum_k, hq, hkv, D, 2)}
    kernels = {k: {"ms": round(v, 4), "algo_bytes": int(bytes_[k]),
                   "GB/s": round(bytes_[k] / (v * 1e-3) / 1e9, 1),
                   "hbm_frac": round(bytes_[k] / (v * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
               for k, v in stage_ms.items()}
    kernels["reduced_attention"]["tflops"] = round(
        attention_flops(count, kv_len, hq, D) / (stage_ms["reduced_attention"] * 1e-3) / 1e12, 2)
    ms = graph_ms if graph_ms is not None else float(np.mean(
        [ev[it][0][0].elapsed_time(ev[it][-1][1]) for it in range(steps)]))
    res = {"workload": f"{name} (batch 1024, block 64, 32q/8kv heads, head dim 128, bf16, "
                       "MaxPool 7, K ~ U{8..24}, hidden 4096, prefixes U{1024..4096} + 64)",
           "timing": "warm HIP-graph replay for the step; eager per-kernel HIP events",
           "kept_rows": sum_k, "sequences_above_64_rows": int((count * (hq // hkv) > 64).sum()),
           "ms_per_step": round(ms, 4), "block tokens/s": round(n * B / (ms * 1e-3), 1),
           "kernels": kernels}
    del x, st
    torch.cuda.empty_cache()
    return res


def focus_block16_leg(dev, flush):
    """Blocks of 16 positions (the FOCUS paper's smallest block) at batch 2048, the same
    bytes as the main step's delta; K ~ U{2..6}, the budget range scaled with the block.
    The delta runs the blocks in pairs as blocks of 32."""
    return focus_block_leg(dev, flush, 2048, 16, 2, 6, seed=7)


def es_mode_leg(dev, flush, steps: int):
    """ES-dLLM mode at batch 8 (512 prompt + 256 generated positions, hidden 4096, keep 128
    of 256): score -> top-K -> gather -> KV scatter (32 heads x 128). Flushed per-kernel
    events; the K-step HIP-graph replay without flushes is reported beside them."""
    import torch
    from block_token_eviction_amd.chain import EsStep
    import workloads as W

    ec = W.ES_B8
    ei = W.esdllm_inputs(ec, device=dev)
    st = EsStep(ec.batch, ec.generated, ec.hidden, ec.keep, ec.dtype, dev)
    args = dict(h_new=ei["h_new"], h_prev=ei["h_prev"], surv_pos=ei["surv_pos"], conf=ei["conf"],
                alpha=ei["alpha"], k=ei["k"], new_k=ei["new_k"], new_v=ei["new_v"],
                row_base=ei["row_base"], cache_k=ei["cache_k"], cache_v=ei["cache_v"])
    import block_token_eviction_amd as bte
    stages = [
        ("esdllm_score", lambda: bte.esdllm_score(ei["h_new"], ei["h_prev"], ei["surv_pos"], ei["conf"], ei["alpha"], out=st.score)),
        ("topk_select", lambda: bte.topk_select(st.score, ei["k"], st.k_max, st.idx, st.count, st.cu)),
        ("gather_rows", lambda: bte.gather_rows(ei["h_new"], st.idx, st.count, st.cu, out=st.gathered)),
        ("kv_scatter", lambda: bte.kv_scatter(ei["new_k"], ei["new_v"], st.idx, st.count, st.cu, ei["row_base"], ei["cache_k"], ei["cache_v"], pos_map=ei["surv_pos"])),
    ]
    per, step, _ = timed_stages(stages, LEG_ITERS, flush)
    graph_ms = graph_step_ms(lambda: st.run(**args), steps)
    n_s, kept, h = ec.batch * ec.generated, int(st.count.sum().item()), ec.hidden
    bytes_ = {"esdllm_score": 2 * n_s * h * 2 + n_s * (4 + 4 + 4),
              "topk_select": n_s * 4 + ec.batch * (ec.keep + 3) * 4,
              "gather_rows": 2 * kept * h * 2,
              "kv_scatter": 2 * 2 * kept * ec.heads * ec.head_dim * 2}
    med = percentile(step, 50)
    return {"workload": "esdllm_b8 (batch 8, 512+256 positions, hidden 4096, keep 128 of 256)",
            "timing": FLUSHED,
            "ms_per_step_p10_p50_p90": [round(percentile(step, q), 4) for q in (10, 50, 90)],
            "survivor positions/s": round(n_s / (med * 1e-3), 1),
            "graph_ms_per_step_unflushed": round(graph_ms, 4) if graph_ms is not None else None,
            "kernels": leg_kernels(per, bytes_)}


def es_pipeline_leg(dev, flush, steps: int):
    """Two ES-dLLM skip layers (r = 0.5 each: 256 -> 128 -> 64 survivors, hidden 4096,
    bf16), each score + in-place hidden-cache update -> top-K -> compaction of the kept
    rows and positions. Each layer's survivor states stand for the model's layers before
    it; they are prepared once, outside the timed region."""
    import torch
    import block_token_eviction_amd as bte
    from block_token_eviction_amd.chain import EsSkipLayer
    import workloads as W

    ec = W.ES_B8
    px = W.es_pipeline_inputs(ec, layers=2, device=dev)
    L = ec.prompt + ec.generated
    sizes = [ec.generated, ec.generated // 2, ec.generated // 4]
    skip = [EsSkipLayer(ec.batch, sizes[i], sizes[i + 1], L, ec.hidden, ec.dtype, dev) for i in range(2)]
    arange = torch.arange(ec.batch + 1, dtype=torch.int32, device=dev)

    def survivor_states(layer, surv):
        n = surv.shape[1]
        cnt = torch.full((ec.batch,), n, dtype=torch.int32, device=dev)
        return bte.gather_rows(px["h_cur"][layer], surv, cnt, arange * n).view(ec.batch, n, -1)

    h0 = survivor_states(0, px["surv_pos"])
    _, s1 = skip[0].run(h0, px["h_cache"][0], px["surv_pos"], px["conf"], px["alpha"])
    s1 = s1.view(ec.batch, -1).clone()
    h1 = survivor_states(1, s1)
    torch.cuda.synchronize()
    stages = []
    for i, (h, sv) in enumerate(((h0, px["surv_pos"]), (h1, s1))):
        sk = skip[i]
        stages += [
            (f"layer{i}_esdllm_score_update", lambda sk=sk, h=h, sv=sv, i=i: bte.esdllm_score_update(h, px["h_cache"][i], sv, px["conf"], px["alpha"], out=sk.score)),
            (f"layer{i}_topk_select", lambda sk=sk: bte.topk_select(sk.score, sk.k, sk.keep, sk.idx, sk.count, sk.cu)),
            (f"layer{i}_gather_rows_multi", lambda sk=sk, h=h, sv=sv: bte.gather_rows_multi([h, sv], sk.idx, sk.count, sk.cu, outs=[sk.h_next, sk.surv_next])),
        ]
    per, step, _ = timed_stages(stages, LEG_ITERS, flush)

    def both_layers():
        skip[0].run(h0, px["h_cache"][0], px["surv_pos"], px["conf"], px["alpha"])
        skip[1].run(h1, px["h_cache"][1], s1, px["conf"], px["alpha"])
    graph_ms = graph_step_ms(both_layers, steps)
    bytes_ = {}
    for i in range(2):
        n, k, h = ec.batch * sizes[i], ec.batch * sizes[i + 1], ec.hidden
        bytes_[f"layer{i}_esdllm_score_update"] = 3 * n * h * 2 + n * (4 + 4 + 4)
        bytes_[f"layer{i}_topk_select"] = n * 4 + ec.batch * (sizes[i + 1] + 3) * 4
        bytes_[f"layer{i}_gather_rows_multi"] = 2 * k * (h * 2 + 4)
    med = percentile(step, 50)
    return {"workload": "esdllm_b8 skip layers (r = 0.5 at two layers: 256 -> 128 -> 64 "
                        "survivors, hidden 4096, bf16)", "timing": FLUSHED,
            "ms_per_iteration_p10_p50_p90": [round(percentile(step, q), 4) for q in (10, 50, 90)],
            "survivor positions/s": round(ec.batch * ec.generated / (med * 1e-3), 1),
            "graph_ms_per_iteration_unflushed": round(graph_ms, 4) if graph_ms is not None else None,
            "kernels": leg_kernels(per, bytes_)}


def es_iteration_leg(dev, flush, iters: int = 12, period: int = 3):
    """ES-dLLM iterations with the device-side bookkeeping (batch 8, a 256-position block
    after a 512-token prompt, hidden 4096, bf16, two skip layers keeping 128 and 64, a
    refresh without skipping every third iteration; the sequences' counters start at
    0..7, so each iteration mixes refreshing and skipping sequences). Each skip layer's
    survivor states stand for the model's layer output: they are taken from a fixed
    tensor by torch indexing between the library calls, outside the events. Reports the
    library's time per iteration (sum of its kernels' events)."""
    import numpy as np
    import torch
    import block_token_eviction_amd as bte
    from block_token_eviction_amd.chain import EsIteration
    import workloads as W

    ec = W.ES_B8
    batch, L, h, blk, keep = ec.batch, ec.prompt + ec.generated, ec.hidden, ec.generated, [128, 64]
    px = W.es_pipeline_inputs(ec, layers=2, device=dev)
    it = torch.arange(batch, dtype=torch.int32, device=dev)
    start = torch.full((batch,), ec.prompt, dtype=torch.int32, device=dev)
    run = EsIteration(batch, blk, h, keep, period, ec.dtype, dev)
    state = {}

    def states(l, rows, cu):
        r = torch.arange(rows.shape[0], device=dev, dtype=torch.int32)
        b = torch.searchsorted(cu[1:].contiguous(), r, right=True).clamp_(max=batch - 1)
        return px["h_cur"][l].view(batch * L, h).index_select(0, b * L + rows.long().clamp(0, L - 1))

    def between(i):                       # the model's layer output for the survivors
        if i == 1:
            state["rows"], state["cnt"], state["cu"] = run.surv0.view(-1), run.count0, run.cu0
            state["h"] = states(0, state["rows"], state["cu"])
        elif i == 4:
            state["rows"], state["cnt"], state["cu"] = run.surv_next[0], run.count[0], run.cu[0]
            state["h"] = states(1, state["rows"], state["cu"])

    def layer_stages(l):
        return [
            (f"layer{l}_esdllm_score_update", lambda: bte.esdllm_score_update(state["h"], px["h_cache"][l], state["rows"], px["conf"], px["alpha"], count=state["cnt"], cu=state["cu"], cap=blk, out=run.score[l])),
            (f"layer{l}_topk_select", lambda: bte.topk_select(run.score[l], run.keep_out[l], blk, run.idx[l], run.count[l], run.cu[l])),
            (f"layer{l}_gather_rows_multi_ragged", lambda: bte.gather_rows_multi_ragged([state["h"], state["rows"]], state["cu"], run.idx[l], run.count[l], run.cu[l], outs=[run.h_next[l], run.surv_next[l]])),
        ]
    stages = [("esdllm_schedule", lambda: run.schedule(it, start))] + layer_stages(0) + layer_stages(1)
    for i, (_, fn) in enumerate(stages):          # one untimed pass, then counters back to 0..7
        between(i)
        fn()
    it.copy_(torch.arange(batch, dtype=torch.int32, device=dev))
    refresh = []
    per, _, sums = timed_stages(stages, iters, flush, warm=0, between=between)
    it_host = it.cpu().numpy()
    # the counters ran 0..7 + iters: refreshes per iteration follow from them
    for i in range(iters):
        c = np.arange(batch) + i
        refresh.append(int(((c == 0) | (c % period == 0)).sum()))
    per_ms = float(np.median(sums))
    return {"workload": "esdllm_b8 iterations (block 256 after 512 prompt positions, hidden 4096, "
                        "keep 128 -> 64, refresh every 3rd iteration, counters 0..7)",
            "timing": FLUSHED + "; model stand-in between the calls is not timed",
            "iterations": iters, "refreshing_sequences_per_iteration": refresh,
            "counters_after": it_host.tolist(),
            "library_ms_per_iteration_p50": round(per_ms, 4),
            "library_ms_per_iteration_min_max": [round(min(sums), 4), round(max(sums), 4)],
            "survivor positions/s": round(batch * blk / (per_ms * 1e-3), 1),
            "kernels_ms_p50": {k: round(percentile(v, 50), 4) for k, v in per.items()}}


def fused_scatter_attention_leg(step, x, steps: int, bytes_: dict):
    """The KV scatter fused into the attention (one launch, bitwise the same
    caches and outputs) against the two launches of the main step, alternated
    step by step in one process on the batch-1024 workload; HIP events on the
    launch stream. The fused launch reads the kept rows' K/V once (from the new
    rows) and writes them into the cache while the K/V stream runs."""
    import numpy as np
    import torch

    pos_base = x["prefix"].to(torch.int32)
    step.schedule(x["kv_len"])
    ev = lambda: torch.cuda.Event(enable_timing=True)
    sep, fus = [], []
    for _ in range(steps + 2):
        e = [ev() for _ in range(4)]
        e[0].record()
        step.scatter(x["new_k"], x["new_v"], x["row_base"], x["cache_k"], x["cache_v"])
        step.attend(x["q_kept"], x["cache_k"], x["cache_v"], x["seq_start"], x["kv_len"])
        e[1].record()
        e[2].record()
        step.scatter_attend(x["q_kept"], x["new_k"], x["new_v"], pos_base, x["cache_k"],
                            x["cache_v"], x["seq_start"], x["kv_len"])
        e[3].record()
        torch.cuda.synchronize()
        sep.append(e[0].elapsed_time(e[1]))
        fus.append(e[2].elapsed_time(e[3]))
    sep, fus = float(np.median(sep[2:])), float(np.median(fus[2:]))
    fused_bytes = bytes_["reduced_attention"] + bytes_["kv_scatter"] // 2   # + the cache writes
    return {"workload": "chain_b1024 (scatter + attention of the main step)",
            "separate_ms": round(sep, 4), "fused_ms": round(fus, 4),
            "fused_algo_bytes": int(fused_bytes),
            "fused_GB/s": round(fused_bytes / (fus * 1e-3) / 1e9, 1),
            "fused_hbm_frac": round(fused_bytes / (fus * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def score_flops(batch: int, block: int, hq: int, head_dim: int) -> int:
    """MFMA flops of the importance delta: two layers of B x B score tiles per
    (sequence, query head), 2 * D flops per score."""
    return 2 * batch * hq * block * block * head_dim * 2


def score_resident_leg(dev, batch: int = 256, reps: int = 100):
    """Auxiliary, labelled as such: the importance-delta kernel repeated on a
    batch whose inputs (batch 256: 168 MB) fit in the 256 MB Infinity Cache,
    with no flush between launches, and its algorithmic matrix-core rate
    against the bf16 dense peak. The kernel's streaming loads need not keep
    the inputs cached, so this does not guarantee cache-fed reads; not a
    bench figure of the workload."""
    import torch

    import block_token_eviction_amd as bte
    import workloads as W

    cfg = W.FocusCfg("score_resident", seed=5, batch=batch)
    fi = W.focus_inputs(cfg, device=dev)
    out = torch.empty((batch, cfg.block), dtype=torch.float32, device=dev)
    run = lambda: bte.focus_importance_delta(fi["q0"], fi["k0"], fi["q1"], fi["k1"], fi["decoded"],
                                             cfg.pool_kernel, out=out)
    for _ in range(10):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    tf = score_flops(batch, cfg.block, cfg.hq, cfg.head_dim) / (ms * 1e-3) / 1e12
    return {"workload": f"focus delta, batch {batch}, repeated without flush (auxiliary)",
            "ms": round(ms, 4), "tflops": round(tf, 1),
            "frac_of_bf16_dense_peak": round(tf / BF16_PEAK_TFLOPS, 4)}


def graph_step_ms(step_fn, steps: int, warm_s: float = 0.6):
    """ms per step of `steps` calls of step_fn captured as one HIP graph and replayed
    once, or None if capture fails. Before the timed replay the same graph is
    replayed back to back for at least warm_s seconds: the GPU clocks down while the
    host captures and instantiates the graph (or sits idle), and the step then runs
    about 3 % slower for the next 0.1-0.3 s of load (measured at the batch-1,024
    step: 1,944-1,950 us per step in a replay right after capture, 1,880-1,884 us
    once warm; the attention kernel alone 1,780-1,786 against 1,715-1,725 us)."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_fn()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                step_fn()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        one = time.perf_counter() - t0
        for _ in range(max(1, math.ceil(warm_s / max(one, 1e-6)))):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        del graph
        return ms
    except RuntimeError as err:
        log(f"graph capture failed: {err}")
        return None


def percentile(sorted_vals, q):
    """Nearest-rank percentile of an ascending list."""
    i = max(0, min(len(sorted_vals) - 1, math.ceil(q / 100 * len(sorted_vals)) - 1))
    return sorted_vals[i]


def copy_bandwidth(dev, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Device-to-device copy rate (read + write bytes per second, GB/s): the
    measured second reference for the roofline fraction."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    return gbs


def full_step_leg(x, fc, ac, steps: int, warmup: int, dev):
    """The extended FOCUS step on the batch-1024 workload: per-kernel average
    durations from HIP events on the launch stream, and the step time from the
    first kernel's start to the last one's end. The per-sequence state that the
    step updates in place (history, rightmost processed position, cached
    mask) is restored after each step, outside the events, so that every
    timed step starts from the same state."""
    import numpy as np
    import torch

    from block_token_eviction_amd.chain import FocusFullStep
    import workloads as W

    log("extended step: generating the paged pool and decode state")
    y = W.focus_full_inputs(fc, ac, page_size=PAGE, device=dev, base=x)
    per_token = [y["hidden_rows"], y["residual"], y["rope_pos"], y["cache_idx"]]
    st = FocusFullStep(fc.batch, fc.block, fc.hq, fc.head_dim,
                       [(t.shape[2:], t.dtype) for t in per_token], fc.dtype, dev, hkv=fc.hkv)
    state = [y[k] for k in ("token_sum", "total_steps", "rightmost_processed", "cached")]
    saved = [t.clone() for t in state]
    stages = [
        ("focus_importance_delta", lambda: st.score(y["q0"], y["k0"], y["q1"], y["k1"], y["decoded"], fc.pool_kernel)),
        ("focus_budget", lambda: st.budget(y["token_sum"], y["total_steps"], ALPHA)),
        ("focus_select", lambda: st.select(y["decoded"], y["rightmost_processed"])),
        ("gather_rows_multi", lambda: st.compact(per_token)),
        ("kv_scatter_paged", lambda: st.scatter(y["new_k_full"], y["new_v_full"], y["pos_base"], y["block_table"], PAGE, y["pool_k"], y["pool_v"])),
        ("attention_order", lambda: st.schedule(y["kv_len"])),
        ("reduced_attention_paged", lambda: st.attend(y["q_full"], y["pool_k"], y["pool_v"], y["block_table"], PAGE, y["kv_len"])),
        ("focus_commit_mask", lambda: st.commit_mask(y["decoded"], y["cached"])),
        ("focus_history_update", lambda: st.history(y["decoded"], y["decoded_now"], y["token_sum"], y["total_steps"])),
    ]

    def restore():
        for t, t0 in zip(state, saved):
            t.copy_(t0)

    for _ in range(warmup):
        for _, fn in stages:
            fn()
        restore()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in stages] for _ in range(steps)]
    log(f"extended step: timing {steps} steps")
    for s in range(steps):
        for i, (_, fn) in enumerate(stages):
            ev[s][i][0].record()
            fn()
            ev[s][i][1].record()
        restore()
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)]))
                for i, (name, _) in enumerate(stages)}
    step_ms = sorted(ev[s][0][0].elapsed_time(ev[s][-1][1]) for s in range(steps))

    count = st.count.cpu().numpy().astype(np.int64)
    n_sel = int(count.sum())
    kv_len = y["kv_len"].cpu().numpy().astype(np.int64)
    n, B, H = fc.batch, fc.block, fc.hidden
    hq, hkv, D, es = fc.hq, fc.hkv, fc.head_dim, 2
    pages = int(((kv_len + PAGE - 1) // PAGE).sum())
    bytes_ = {
        "focus_importance_delta": 2 * n * B * (hq + hkv) * D * es + n * B * (1 + 4),
        "focus_budget": n * (B * 4 + 12),
        "focus_select": n * (B * 4 + 4 + B + 8 + B * 4 + 4) + (n + 1) * 4,
        "gather_rows_multi": 2 * n_sel * (H * 2 + H * 4 + 4 + 8),
        "kv_scatter_paged": 2 * 2 * n_sel * hkv * D * es,
        "attention_order": 2 * n * 4,
        "reduced_attention_paged": int(kv_len.sum()) * hkv * D * es * 2 + 2 * n_sel * hq * D * es
                                   + pages * 4,
        "focus_commit_mask": n * (4 * B + 4),
        "focus_history_update": n * (2 * B + 16),
    }
    kernels = {k: {"ms": round(stage_ms[k], 4), "algo_bytes": int(bytes_[k]),
                   "GB/s": round(bytes_[k] / (stage_ms[k] * 1e-3) / 1e9, 1),
                   "hbm_frac": round(bytes_[k] / (stage_ms[k] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
               for k in stage_ms}
    med = percentile(step_ms, 50)
    return {"workload": f"chain_b1024 extended (alpha {ALPHA}, pages of {PAGE} rows, shuffled pool; "
                        "decode state drawn per sequence)",
            "ms_per_step_p10_p50_p90": [round(percentile(step_ms, q), 4) for q in (10, 50, 90)],
            "block tokens/s": round(n * B / (med * 1e-3), 1),
            "selected_rows": n_sel, "mean_selected": round(n_sel / n, 2),
            "kernels": kernels}
KERNEL_SOURCES = {"reduced_attention": ["reduced_attention.hip", "bte_device.h"],
                  "focus_importance_delta": ["focus_delta.hip", "bte_device.h"],
                  "rows": ["rows.hip", "bte_device.h"],
                  "esdllm": ["esdllm_score.hip", "bte_device.h"]}


def kernel_source_hash(kernel: str) -> str:
    import hashlib
    h = hashlib.sha1()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "block_token_eviction_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _profile_record(name: str):
    """A committed profile summary (profiles/<name>.json), or None when missing or when the
    kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    key = rec.get("source_key", "reduced_attention")
    if rec.get("kernel_sources_sha1") != kernel_source_hash(key):
        return None
    return rec


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy of known size), or None when the
    kernel's sources changed since the counters were taken."""
    rec = _profile_record(f"{kernel}_chain_b1024_counters")
    return None if rec is None else rec.get("traffic_bytes_per_launch")


def trace_roofline(kernel: str, algo_bytes: int) -> dict:
    """The kernel's average duration over the eager timed loop's dispatches in a committed
    rocprofv3 kernel trace of this bench (same dispatches as the events above), and the
    roofline fraction it gives; None while the kernel's sources differ from the traced ones."""
    rec = _profile_record(f"{kernel}_chain_b1024_trace")
    if rec is None:
        return {"trace_us": None, "frac_trace": None}
    us = rec["trace_avg_us"]
    return {"trace_us": round(us, 1), "frac_trace": round(algo_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "trace_dispatches": rec.get("dispatches"),
            "trace_run_event_us": rec.get("events_same_run_us")}


def cpu_model() -> str:
    """The host CPU's model name (lscpu's "Model name", else /proc/cpuinfo), or "unknown"."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, fc, ac, budget_s: float = 12.0, single_budget_s: float = 5.0):
    """The float64 oracle on the first sequences of the same workload, chunk by chunk until
    about `budget_s` seconds of CPU work, with its BLAS on every thread it is given; then
    the same at one thread for about `single_budget_s`. Block tokens/s of each sample."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle.chain as oc

    def f64(t):
        return t.detach().to("cpu", torch.float64).numpy()

    def bits(t):
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)

    seq_start = x["seq_start"].cpu().numpy()
    kv_len = x["kv_len"].cpu().numpy()

    def run(budget, chunk):
        done, elapsed = 0, 0.0
        while done < fc.batch and elapsed < budget:
            lo, hi = done, min(fc.batch, done + chunk)
            r0, r1 = int(seq_start[lo]), int(seq_start[hi - 1] + kv_len[hi - 1])
            cap = (hi - lo) * fc.k_hi
            inp = dict(q0=f64(x["q0"][lo:hi]), k0=f64(x["k0"][lo:hi]), q1=f64(x["q1"][lo:hi]),
                       k1=f64(x["k1"][lo:hi]), decoded=x["decoded"][lo:hi].cpu().numpy(),
                       k=x["k"][lo:hi].cpu().numpy(), hidden_rows=bits(x["hidden_rows"][lo:hi]),
                       pool_kernel=fc.pool_kernel, new_k=bits(x["new_k"][:cap]),
                       new_v=bits(x["new_v"][:cap]), q_kept=bits(x["q_kept"][:cap]),
                       cache_k=bits(x["cache_k"][r0:r1]), cache_v=bits(x["cache_v"][r0:r1]),
                       seq_start=seq_start[lo:hi] - r0, kv_len=kv_len[lo:hi],
                       row_base=x["row_base"][lo:hi].cpu().numpy() - r0)
            t0 = time.perf_counter()
            oc.focus_step(**inp, hq=fc.hq, hkv=fc.hkv, k_max=fc.k_hi,
                          scale=1.0 / math.sqrt(fc.head_dim))
            elapsed += time.perf_counter() - t0
            done = hi
        return done, elapsed

    log("cpu baseline (oracle)")
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    done, elapsed = run(budget_s, 16)
    with threadpool_limits(limits=1):
        done1, elapsed1 = run(single_budget_s, 4)
    affinity = len(os.sched_getaffinity(0))
    return {"value": round(done * fc.block / elapsed, 1), "unit": "block tokens/s",
            "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "affinity_cpus": affinity,
            "sample": f"first {done} of {fc.batch} sequences of chain_b1024, whole step, "
                      f"{elapsed:.1f} s (numpy float64; BLAS threads = {threads} of "
                      f"{affinity} CPUs in this process's affinity mask)",
            "one_thread": {"value": round(done1 * fc.block / elapsed1, 1),
                           "unit": "block tokens/s", "cores": 1,
                           "sample": f"first {done1} sequences, {elapsed1:.1f} s, BLAS limited "
                                     f"to one thread"}}


if __name__ == "__main__":
    main()
