"""bench.py on the GPU: one short run of the main step, whose JSON line must carry every key
of the reporting contract with consistent values."""
import json
import os
import subprocess
import sys

import pytest

from helpers import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    say("bench.py --steps 3 --warmup 2 --no-cpu-baseline --legs main")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "2", "--no-cpu-baseline", "--legs", "main"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "kernels"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["unit"] == "block tokens/s" and d["higher_is_better"] is True
    assert d["dtype"] == "bf16" and d["vs_baseline"] is None and d["cpu_baseline"] is None
    assert d["config"]["workload"] == "chain_b1024"
    # value is the batch's block positions over the step time
    assert d["value"] == pytest.approx(1024 * 32 / (d["ms_per_step"] * 1e-3), rel=1e-3)
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    assert 0.3 < roof["frac"] < 1.0
    # the attention's achieved rate is its algorithmic bytes over its event time
    att = d["kernels"]["reduced_attention"]
    assert roof["achieved"] == pytest.approx(att["algo_bytes"] / (att["ms"] * 1e-3) / 1e9, rel=1e-3)
    # every stage of the step is timed, and the step fits in the sum of its stages' times
    stages = ("focus_importance_delta", "topk_select", "gather_rows", "kv_scatter",
              "attention_order", "reduced_attention")
    assert set(stages) <= set(d["kernels"])
    assert sum(d["kernels"][s]["ms"] for s in stages) == pytest.approx(d["eager_ms_per_step"], rel=0.25)


def test_bench_block64_chain_leg():
    """The whole-step leg at blocks of 64: its throughput is the batch's block positions over
    its step time, and its attention runs the query split (sequences above 64 rows)."""
    say("bench.py --steps 3 --warmup 2 --no-cpu-baseline --legs chain_b1024_block64")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "2", "--no-cpu-baseline", "--legs", "chain_b1024_block64"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    d = json.loads([l for l in r.stdout.splitlines() if l.strip()][-1])
    leg = d["chain_b1024_block64"]
    assert leg["block tokens/s"] == pytest.approx(1024 * 64 / (leg["ms_per_step"] * 1e-3), rel=1e-3)
    assert 0 < leg["sequences_above_64_rows"] < 1024
    ks = leg["kernels"]
    assert set(ks) == {"focus_importance_delta", "topk_select", "gather_rows", "kv_scatter",
                       "attention_order", "reduced_attention"}
    att = ks["reduced_attention"]
    assert att["hbm_frac"] == pytest.approx(att["algo_bytes"] / (att["ms"] * 1e-3) / 8e12, abs=1e-3)
    assert 0.3 < att["hbm_frac"] < 1.0
