"""Host-side pieces of bench.py: algorithmic bytes and the counter record."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_mask_bytes_small_case_by_hand():
    # 130 boxes: 3 row tiles, all in strip 0, so every row writes 3 words
    w = workloads.random_small(0, 130)
    assert bench._dense_band_bytes(w) == 130 * 3 * 8 + 20 * 130


def test_mask_bytes_strip_offsets():
    # 64 * 20 boxes, strips of 8 column tiles: row tiles 0..7 start at column
    # 0 (20 words), 8..15 at column 8 (12 words), 16..19 at column 16 (4 words)
    assert bench.MASK_STRIP == 8
    w = workloads.random_small(0, 64 * 20)
    assert bench._dense_band_bytes(w) == (64 * (8 * 20 + 8 * 12 + 4 * 4) * 8
                                                + 20 * 64 * 20)


def test_sparse_mask_bytes_by_hand():
    # 130 boxes read once (20 B each) and 7 nonzero words written (12 B each)
    w = workloads.random_small(0, 130)
    assert bench._mask_sparse_bytes(w, 7) == 20 * 130 + 12 * 7


def test_traffic_record_is_read_when_sources_match():
    traffic, detail = bench._traffic()
    if traffic is None:
        pytest.skip("counter record is stale or absent: %s" % detail)
    assert traffic == detail["fetch_bytes"] + detail["write_bytes"]


def test_traffic_is_null_when_sources_change(tmp_path, monkeypatch):
    rec = {"source_sha256": "0" * 64, "fetch_bytes": 1, "write_bytes": 2}
    p = tmp_path / "rec.md"
    p.write_text("x\ntraffic-record: " + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(p))
    traffic, why = bench._traffic()
    assert traffic is None and "changed" in why


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "single MI355X" in r.stderr


def test_sweep_dense_bytes_by_hand():
    import numpy as np
    # 130 boxes (3 row tiles); scores descending in index, so sorted position
    # = index; kept boxes at positions 0, 64 and 129
    scores = np.linspace(1.0, 0.5, 130).astype(np.float32)
    w = workloads.Workload("t", np.zeros((130, 4), np.float32), scores, 0.5)
    got = bench._sweep_dense_bytes(w, [0, 64, 129])
    assert got == 8 * 130 + 8 * ((3 - 0 - 1) + (3 - 1 - 1) + (3 - 2 - 1))
