"""The analytic model (na_simulate / na_tile_candidates) against the oracle's
brute-force tile statistics, and the pages' perfectly block-sparse claim."""

import math

import numpy as np
import pytest

import oracle
from synth import WORKLOADS


def _dt(na, name):
    return {"bf16": na.NA_BF16, "fp8": na.NA_FP8_E4M3, "f32": na.NA_F32}[name]


def _oracle_stats(grid, window, stride, tq, tk):
    return oracle.tile_map_stats(grid, window, stride, tq, tk)


def _random_geometries(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        grid = tuple(int(x) for x in rng.integers(1, 13, 3))
        window = tuple(int(rng.integers(1, L + 1)) for L in grid)
        stride = tuple(int(rng.integers(1, w + 1)) for w in window)
        out.append((grid, window, stride))
    return out


@pytest.mark.parametrize("geom", _random_geometries(12, 5))
def test_simulated_counts_match_oracle(na, geom):
    grid, window, stride = geom
    rng = np.random.default_rng(sum(grid) * 7 + sum(window))
    for _ in range(3):
        tq = tuple(int(2 ** rng.integers(0, 4)) for _ in range(3))
        tk = tuple(int(2 ** rng.integers(0, 4)) for _ in range(3))
        r = na.na_simulate(1, 1, 128, grid, window, stride, na.NA_BF16, tq, tk)
        o = _oracle_stats(grid, window, stride, tq, tk)
        st = r["stats"]
        for key in ("n_q_tiles", "nnz", "n_full", "n_boundary", "computed_slots", "effective_slots"):
            assert st[key] == o[key], (key, tq, tk)
        assert r["tile_efficiency"] == pytest.approx(o["efficiency"], rel=1e-12)
        assert r["perfectly_block_sparse"] == (o["n_boundary"] == 0)
        assert r["flop_ratio_vs_dense"] == pytest.approx(math.prod(grid) / math.prod(window), rel=1e-12)


@pytest.mark.parametrize("name", ["video_block", "img256_block", "img64_sliding", "img64_block"])
def test_speedup_bound_is_dense_over_sparse_computed_work(na, name):
    wl = WORKLOADS[name]
    dt = _dt(na, wl.dtype)
    r = na.na_simulate(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.window, wl.stride, dt)
    sparse = _oracle_stats(wl.grid, wl.window, wl.stride, r["tile_q"], r["tile_kv"])
    dq, dk = na.na_choose_tiles(wl.grid, wl.grid, (1, 1, 1), wl.head_dim, dt)
    dense = _oracle_stats(wl.grid, wl.grid, (1, 1, 1), dq, dk)
    assert dense["n_boundary"] == 0
    assert r["speedup_bound"] == pytest.approx(dense["computed_slots"] / sparse["computed_slots"], rel=1e-12)
    # never above the FLOP ratio by more than the dense call's own padding
    assert r["speedup_bound"] <= r["flop_ratio_vs_dense"] * dense["computed_slots"] / dense["effective_slots"] + 1e-9


def test_pages_video_config_is_perfectly_block_sparse(na):
    # GNA page, sections 1.1 and 3.1: at stride 16x8x8 on the 30x48x80 video the
    # speed-up matches the FLOP reduction, i.e. KV tiles align with every window
    g, w, s = (30, 48, 80), (18, 24, 24), (16, 8, 8)
    r = na.na_simulate(1, 24, 128, g, w, s, na.NA_BF16, (2, 8, 8), (2, 8, 8))
    assert r["perfectly_block_sparse"] and r["stats"]["n_boundary"] == 0
    assert r["tile_efficiency"] == 1.0 and r["speedup_bound"] == pytest.approx(r["flop_ratio_vs_dense"])
    chosen = na.na_simulate(1, 24, 128, g, w, s, na.NA_BF16)
    assert chosen["perfectly_block_sparse"]
    # stride 1 (sliding window) cannot align: boundary tiles appear
    sl = na.na_simulate(1, 24, 128, g, (30, 40, 40), (1, 1, 1), na.NA_BF16)
    assert not sl["perfectly_block_sparse"] and sl["stats"]["n_boundary"] > 0


def test_candidates_sorted_first_is_chosen(na):
    wl = WORKLOADS["video_block"]
    cs = na.na_tile_candidates(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.window, wl.stride, na.NA_BF16)
    assert len(cs) > 10
    costs = [c["cost"] for c in cs]
    assert costs == sorted(costs)
    tq, tk = na.na_choose_tiles(wl.grid, wl.window, wl.stride, wl.head_dim, na.NA_BF16)
    assert cs[0]["tile_q"] == tuple(tq) and cs[0]["tile_kv"] == tuple(tk)
    for c in cs:   # every candidate is a shape a bf16 kernel exists for
        assert math.prod(c["tile_q"]) in (128, 256) and math.prod(c["tile_kv"]) in (64, 128)
        assert c["tile_kv"][2] >= 8
    r = na.na_simulate(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.window, wl.stride, na.NA_BF16, tq, tk)
    assert r["cost"] == cs[0]["cost"] and r["predicted_kernel_ms"] == cs[0]["predicted_kernel_ms"]


def test_predicted_time_behaves(na):
    g, w, s = (30, 48, 80), (18, 24, 24), (16, 8, 8)
    a = na.na_simulate(1, 24, 128, g, w, s, na.NA_BF16)
    b = na.na_simulate(1, 48, 128, g, w, s, na.NA_BF16)
    launch = 0.015
    assert (b["predicted_kernel_ms"] - launch) == pytest.approx(2 * (a["predicted_kernel_ms"] - launch), rel=0.05)
    f8 = na.na_simulate(1, 24, 128, g, w, s, na.NA_FP8_E4M3)
    assert f8["predicted_kernel_ms"] < a["predicted_kernel_ms"]
    assert a["form"] == 1 and f8["form"] == 1
    assert a["predicted_forward_ms"] > a["predicted_kernel_ms"]   # the k / v permutes
    # fp8 permutes the same k / v in one byte per element instead of two
    assert 0 < f8["predicted_forward_ms"] - f8["predicted_kernel_ms"] < a["predicted_forward_ms"] - a["predicted_kernel_ms"]
    dense = na.na_simulate(1, 24, 128, g, g, (1, 1, 1), na.NA_BF16)
    assert dense["predicted_kernel_ms"] / a["predicted_kernel_ms"] == pytest.approx(a["speedup_bound"], rel=0.1)


def test_simulate_rejects_bad_arguments(na):
    import ctypes
    lib = na.load()
    I3 = na.I3
    r = na.SimResult()
    g, w, s = I3(1, 16, 16), I3(1, 5, 5), I3(1, 1, 1)
    assert lib.na_simulate(1, 1, 64, g, w, s, na.NA_BF16, I3(1, 3, 8), I3(1, 8, 8), ctypes.byref(r)) == \
        na.NA_ERR_INVALID_ARG
    assert lib.na_simulate(1, 1, 64, g, w, s, na.NA_BF16, I3(1, 8, 8), None, ctypes.byref(r)) == na.NA_ERR_INVALID_ARG
    assert lib.na_simulate(1, 1, 48, g, w, s, na.NA_BF16, None, None, ctypes.byref(r)) == na.NA_ERR_UNSUPPORTED
    assert lib.na_simulate(1, 1, 64, g, w, s, na.NA_BF16, None, None, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_tile_candidates(1, 1, 64, g, w, s, na.NA_BF16, None, 4) == na.NA_ERR_INVALID_ARG
    assert lib.na_tile_candidates(1, 1, 64, g, I3(1, 17, 5), s, na.NA_BF16, None, 0) == na.NA_ERR_INVALID_ARG
