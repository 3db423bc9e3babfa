"""Host-side checks of bench.py and of the committed profile summaries it reads (CPU only)."""
import glob
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    """The path runs on one GPU: --gpus above 1 exits with status 2 and says why, before
    touching any device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unknown_leg_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--legs", "no_such_leg"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "unknown legs" in r.stderr


def test_delta_bytes_at_the_workloads():
    """Q and K of both layers once (bf16), the decoded mask (1 B) and the delta (4 B) per
    position: 671,252,480 B at batch 1,024 and 167,813,120 B at batch 256 (block 32, 32
    query / 8 KV heads, head dim 128)."""
    assert bench.delta_bytes(1024, 32, 32, 8, 128, 2) == 1024 * 32 * (2 * 40 * 128 * 2 + 5)
    assert bench.delta_bytes(1024, 32, 32, 8, 128, 2) == 671_252_480
    assert bench.delta_bytes(256, 32, 32, 8, 128, 2) == 167_813_120


def test_attention_bytes_by_hand():
    """K and V rows of every sequence once, plus the kept queries read and the outputs
    written: two sequences of 3 and 5 positions, 4 kept rows, 8 query / 2 KV heads, head
    dim 64, bf16."""
    kv_len = np.array([3, 5])
    kv = (3 + 5) * 2 * 64 * 2 * 2          # rows x KV heads x D x 2 B x (K and V)
    qo = 4 * 8 * 64 * 2 * 2                # kept rows x query heads x D x 2 B x (q and out)
    assert bench.attention_bytes(kv_len, 4, 8, 2, 64, 2) == kv + qo


def test_attention_flops_by_hand():
    """4 flops per (kept row, query head, key, dimension): S = q.K and P.V."""
    assert bench.attention_flops([2, 1], [10, 7], 8, 64) == 4 * 8 * 64 * (2 * 10 + 1 * 7)


def test_percentile_interpolates():
    vals = [1.0, 2.0, 3.0, 4.0, 5.0]
    assert bench.percentile(vals, 50) == 3.0
    assert bench.percentile(vals, 0) == 1.0
    assert bench.percentile(vals, 100) == 5.0


COUNTERS = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_counters.json")))


@pytest.mark.parametrize("path", COUNTERS, ids=[os.path.basename(p) for p in COUNTERS])
def test_counter_summaries_are_consistent(path):
    """Each counter summary's bytes follow from its raw KiB and the calibration copy: scale =
    copy bytes / what the counter read for the copy, bytes = mean raw KiB x 1024 x scale,
    traffic = fetch + write; it names its source files and the two rocprofv3 commands."""
    rec = json.load(open(path))
    kib = 1024.0
    fscale = rec["copy_bytes"] / (rec["copy_fetch_kib_raw"] * kib)
    wscale = rec["copy_bytes"] / (rec["copy_write_kib_raw"] * kib)
    assert rec["fetch_scale"] == pytest.approx(fscale)
    assert rec["write_scale"] == pytest.approx(wscale)
    assert rec["fetch_bytes_per_launch"] == pytest.approx(rec["fetch_kib_raw"] * kib * fscale, abs=1)
    assert rec["write_bytes_per_launch"] == pytest.approx(rec["write_kib_raw"] * kib * wscale, abs=1)
    assert rec["traffic_bytes_per_launch"] == pytest.approx(
        rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"], abs=2)
    assert rec["source_key"] in bench.KERNEL_SOURCES
    assert len(rec["commands"]) == 2
    assert "FETCH_SIZE" in rec["commands"][0] and "WRITE_SIZE" in rec["commands"][1]
    assert rec["launches"] >= 1


def test_trace_summary_selects_the_eager_loop():
    """The committed trace record averages exactly K dispatches starting after the W
    warm-up launches, and its average agrees with the HIP events of the same run."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "reduced_attention_chain_b1024_trace.json")))
    lo, hi = rec["selected"]
    assert hi - lo == rec["dispatches"] and lo >= 0 and hi <= rec["dispatches_in_trace"]
    assert rec["trace_min_us"] <= rec["trace_avg_us"] <= rec["trace_max_us"]
    assert abs(rec["trace_avg_us"] - rec["events_same_run_us"]) / rec["events_same_run_us"] < 0.02


def test_profile_records_are_gated_by_the_kernel_sources(monkeypatch, tmp_path):
    """bench.py reports committed counter traffic only while the kernel's sources hash to
    the recorded sha1."""
    rec = {"source_key": "rows", "kernel_sources_sha1": "x", "traffic_bytes_per_launch": 5}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "gather_rows_chain_b1024_counters.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda key: "x")
    assert bench.measured_traffic("gather_rows") == 5
    monkeypatch.setattr(bench, "kernel_source_hash", lambda key: "y")
    assert bench.measured_traffic("gather_rows") is None
    assert bench.measured_traffic("no_such_kernel") is None
