"""Host-side logic of bench.py and of the query sampler it and the parity
tests share (no GPU): the one-GPU guard, the counter-summary lookups keyed
by kernel source hash, the oracle work split and the corner / edge sample."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import WORKLOADS, sample_queries  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_source_hash_follows_the_sources():
    h = bench.kernel_source_hash("attn_bf16")
    assert len(h) == 16 and int(h, 16) >= 0
    assert h != bench.kernel_source_hash("attn_fp8")
    assert h == bench.kernel_source_hash("attn_bf16")


def _write_summary(root, name, d):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", name), "w") as fh:
        json.dump(d, fh)


def test_counter_summaries_used_only_for_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _write_summary(str(tmp_path), "attn_bf16_io_qo_video_block_traffic.json",
                   {"workload": "video_block", "kernel_source_sha256_16": "abc", "hbm_bytes_per_launch": 123.0})
    _write_summary(str(tmp_path), "attn_fp8_io_qo_img256_block_fp8_mfma.json",
                   {"workload": "img256_block_fp8", "kernel_source_sha256_16": "def", "mfma_busy_frac": 0.4,
                    "clock_ghz": 2.1, "valu_per_mfma": 14.0, "other": 1})
    assert bench.measured_traffic("video_block", "abc", "IO_QO") == 123.0
    assert bench.measured_traffic("video_block", "stale", "IO_QO") is None        # kernel changed since
    assert bench.measured_traffic("video_block", "abc", "IO_TILE") is None        # no summary for this form
    assert bench.measured_traffic("video_sliding", "abc", "IO_QO") is None        # nor for this workload
    assert bench.measured_mfma("img256_block_fp8", "def", "IO_QO", "attn_fp8") == {
        "mfma_busy_frac": 0.4, "clock_ghz": 2.1, "valu_per_mfma": 14.0}
    assert bench.measured_mfma("img256_block_fp8", "def", "IO_QO") is None        # other kernel family


def test_counter_summary_with_wrong_workload_is_ignored(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _write_summary(str(tmp_path), "attn_bf16_io_qo_video_block_traffic.json",
                   {"workload": "video_sliding", "kernel_source_sha256_16": "abc", "hbm_bytes_per_launch": 1.0})
    assert bench.measured_traffic("video_block", "abc", "IO_QO") is None


def test_oracle_chunks_cover_every_query_of_every_head_once():
    qs = np.arange(1000) * 3
    tasks = bench._chunks("w", [0, 23], qs, size=64)
    seen = [(h, int(x)) for _, h, c in tasks for x in c]
    assert len(seen) == len(set(seen)) == 2 * len(qs)
    assert all(len(c) <= 64 for _, _, c in tasks)
    assert {n for n, _, _ in tasks} == {"w"}


@pytest.mark.parametrize("name", ["video_block", "video_sliding", "img256_block", "img64_sliding"])
def test_sample_holds_corner_and_edge_tiles(name):
    wl = WORKLOADS[name]
    tq = (4, 8, 8) if wl.grid[0] > 1 else (1, 16, 16)
    qs = sample_queries(wl, tq, n_random=1024, seed_offset=7)
    assert np.all(np.diff(qs) > 0) and qs[0] >= 0 and qs[-1] < wl.tokens
    T, H, W = wl.grid
    lin = lambda t, h, w: (t * H + h) * W + w
    # the grid's 8 corner tokens and the first token of the last (ragged) tile along each axis
    for t in (0, T - 1):
        for h in (0, H - 1):
            for w in (0, W - 1):
                assert lin(t, h, w) in set(qs.tolist())
    last = [(-(-L // t) - 1) * t for L, t in zip(wl.grid, tq)]
    assert lin(last[0], 0, 0) in set(qs.tolist())
    # the same seed gives the same sample, another gives another
    assert np.array_equal(qs, sample_queries(wl, tq, n_random=1024, seed_offset=7))
    assert not np.array_equal(qs, sample_queries(wl, tq, n_random=1024, seed_offset=8))
