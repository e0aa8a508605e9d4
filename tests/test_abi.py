"""CPU-side checks of libna.so: it loads, exports every declared symbol, its
host tile-map builder matches the oracle bit for bit, and bad arguments are
rejected before anything is launched.  No GPU is needed."""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "na.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(na_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(na):
    lib = na.load()
    declared = _declared_symbols()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(na.SYMBOLS)


def _cmp_tile_map(na, grid, window, stride, tq, tk):
    qptr, kv, nf, stats = na.na_build_tile_map(grid, window, stride, tq, tk)
    oq, okv, onf = oracle.tile_map(grid, window, stride, tq, tk)
    np.testing.assert_array_equal(qptr, oq)
    np.testing.assert_array_equal(kv, okv)
    np.testing.assert_array_equal(nf, onf)
    os_ = oracle.tile_map_stats(grid, window, stride, tq, tk)
    assert stats["nnz"] == os_["nnz"] and stats["n_full"] == os_["n_full"]
    assert stats["computed_slots"] == os_["computed_slots"]
    assert stats["effective_slots"] == os_["effective_slots"]


def test_tile_map_matches_oracle_random_sweep(na):
    rng = np.random.default_rng(7)
    for _ in range(300):
        nd = int(rng.integers(1, 4))
        grid = [1, 1, 1]
        window = [1, 1, 1]
        stride = [1, 1, 1]
        tq = [1, 1, 1]
        tk = [1, 1, 1]
        for d in range(3 - nd, 3):
            L = int(rng.integers(1, 13))
            w = int(rng.integers(1, L + 1))
            s = int(rng.integers(1, w + 1))
            grid[d], window[d], stride[d] = L, w, s
            tq[d] = int(2 ** rng.integers(0, 4))
            tk[d] = int(2 ** rng.integers(0, 4))
        _cmp_tile_map(na, grid, window, stride, tq, tk)


@pytest.mark.parametrize("name", ["img16_f32", "img64_sliding", "img64_block", "video_sliding", "video_block",
                                  "img256_block"])
def test_tile_map_matches_oracle_on_workloads(na, name):
    from synth import WORKLOADS
    wl = WORKLOADS[name]
    for dt in (na.NA_F32, na.NA_BF16):
        try:
            tq, tk = na.na_choose_tiles(wl.grid, wl.window, wl.stride, wl.head_dim, dt)
        except na.NAError:
            continue
        _cmp_tile_map(na, wl.grid, wl.window, wl.stride, tq, tk)


def test_chosen_tiles_video_block_are_perfectly_aligned(na):
    from synth import WORKLOADS
    wl = WORKLOADS["video_block"]
    tq, tk = na.na_choose_tiles(wl.grid, wl.window, wl.stride, wl.head_dim, na.NA_BF16)
    _, _, _, st = na.na_build_tile_map(wl.grid, wl.window, wl.stride, tq, tk)
    assert st["n_boundary"] == 0
    assert st["nnz"] == st["n_q_tiles"] * 81


@pytest.mark.parametrize("no_fused", ["1", "0"])
def test_workspace_is_linear_in_tokens(na, monkeypatch, no_fused):
    # no N x N buffer: doubling the grid doubles the workspace (up to padding),
    # for both the all-copies form and the k / v-copies form
    monkeypatch.setenv("NA_NO_FUSED", no_fused)
    a = na.na_workspace_bytes(1, 2, 128, (1, 64, 64), (1, 9, 9), (1, 1, 1), na.NA_BF16)
    b = na.na_workspace_bytes(1, 2, 128, (1, 128, 64), (1, 9, 9), (1, 1, 1), na.NA_BF16)
    assert 1.9 < b / a < 2.1
    N = 64 * 64
    assert a < 8 * N * 2 * 128 * 2 * 4


def _status(na, fn, *args):
    return getattr(na.load(), fn)(*args)


def test_forward_mode_rule(na, monkeypatch):
    for D in (64, 128):
        assert na.na_forward_mode(na.NA_BF16, D, True) == 1
        assert na.na_forward_mode(na.NA_BF16, D, False) == 2
    assert na.na_forward_mode(na.NA_BF16, 32, True) == 0
    assert na.na_forward_mode(na.NA_F32, 128, True) == 0 and na.na_forward_mode(na.NA_F32, 128, False) == 0
    # fp8: grid-order q / out with k, v permuted; no form without a workspace
    assert na.na_forward_mode(na.NA_FP8_E4M3, 128, True) == 1
    assert na.na_forward_mode(na.NA_FP8_E4M3, 128, False) == 1
    monkeypatch.setenv("NA_NO_FUSED", "1")
    assert na.na_forward_mode(na.NA_BF16, 128, True) == 0 and na.na_forward_mode(na.NA_BF16, 128, False) == 0


def test_kv_copy_form_workspace(na, monkeypatch):
    # form 1 holds exactly the k and v tile copies: 2 x B x H x padded tokens x D x 2 bytes
    grid, window, stride = (1, 64, 64), (1, 9, 9), (1, 1, 1)
    tq, tk = na.na_choose_tiles(grid, window, stride, 128, na.NA_BF16)
    padded = math.prod(-(-L // t) * t for L, t in zip(grid, tk))
    kv = 1 * 2 * padded * 128 * 2
    assert na.na_workspace_bytes(1, 2, 128, grid, window, stride, na.NA_BF16) == 2 * ((kv + 255) // 256 * 256)
    # fp8 (one byte per element) takes the same form
    tq8, tk8 = na.na_choose_tiles(grid, window, stride, 128, na.NA_FP8_E4M3)
    kv8 = 1 * 2 * math.prod(-(-L // t) * t for L, t in zip(grid, tk8)) * 128
    assert na.na_workspace_bytes(1, 2, 128, grid, window, stride, na.NA_FP8_E4M3) == 2 * ((kv8 + 255) // 256 * 256)
    monkeypatch.setenv("NA_NO_FUSED", "1")
    assert na.na_workspace_bytes(1, 2, 128, grid, window, stride, na.NA_BF16) > 2 * kv


def test_invalid_arguments_rejected(na, monkeypatch):
    monkeypatch.setenv("NA_NO_FUSED", "1")   # the workspace checks belong to the permute path
    lib = na.load()
    I3 = na.I3
    good = dict(grid=I3(1, 16, 16), window=I3(1, 5, 5), stride=I3(1, 1, 1))
    ws = na.na_workspace_bytes(1, 1, 64, (1, 16, 16), (1, 5, 5), (1, 1, 1), na.NA_BF16)
    fake = 1 << 20   # aligned dummy address: never dereferenced, every call below fails first

    def fwd(q=fake, k=fake, v=fake, out=fake, lse=None, B=1, h=1, D=64, grid=None, window=None, stride=None,
            scale=0.125, dt=na.NA_BF16, ws_ptr=fake, ws_bytes=ws):
        return lib.na_forward(q, k, v, out, lse, B, h, D, grid or good["grid"], window or good["window"],
                              stride or good["stride"], scale, dt, None, ws_ptr, ws_bytes, None)

    assert fwd(window=I3(1, 17, 5)) == na.NA_ERR_INVALID_ARG          # window > grid
    assert fwd(stride=I3(1, 6, 1)) == na.NA_ERR_INVALID_ARG           # stride > window
    assert fwd(stride=I3(1, 0, 1)) == na.NA_ERR_INVALID_ARG           # stride 0
    assert fwd(B=-1) == na.NA_ERR_INVALID_ARG
    assert fwd(B=0, q=None) == na.NA_OK                                # empty problem: nothing launched
    assert fwd(q=None) == na.NA_ERR_INVALID_ARG                        # null pointer
    assert fwd(out=fake + 8) == na.NA_ERR_INVALID_ARG                  # misaligned
    assert fwd(ws_bytes=ws - 1) == na.NA_ERR_WORKSPACE
    assert fwd(dt=na.NA_F32, D=32, ws_ptr=None) == na.NA_ERR_INVALID_ARG   # fp32 needs a workspace
    assert fwd(D=48) == na.NA_ERR_UNSUPPORTED
    assert fwd(dt=7) == na.NA_ERR_INVALID_ARG
    assert fwd(scale=float("nan")) == na.NA_ERR_INVALID_ARG
    assert fwd(scale=-0.5) == na.NA_ERR_INVALID_ARG
    assert "scale" in na.na_last_error()
    # the form-1 kernel entry point: bf16 (head_dim 64 / 128) or fp8 (128), tile_kv checked
    tk = na.I3(*na.na_choose_tiles((1, 16, 16), (1, 5, 5), (1, 1, 1), 64, na.NA_BF16)[1])
    assert lib.na_attend_kv_tiled(fake, fake, fake, fake, None, 1, 1, 64, good["grid"], good["window"],
                                  good["stride"], tk, 0.125, na.NA_FP8_E4M3, None, None) == na.NA_ERR_UNSUPPORTED
    assert lib.na_attend_kv_tiled(fake, fake, fake, fake, None, 1, 1, 64, good["grid"], good["window"],
                                  good["stride"], I3(1, 1, 1), 0.125, na.NA_BF16, None, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_attend_kv_tiled(fake, None, fake, fake, None, 1, 1, 64, good["grid"], good["window"],
                                  good["stride"], tk, 0.125, na.NA_BF16, None, None) == na.NA_ERR_INVALID_ARG
    # permutation kernels
    assert lib.na_permute(fake, fake, 1, 1, 64, I3(1, 16, 16), I3(1, 3, 8), 2, 0, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_permute(fake, None, 1, 1, 64, I3(1, 16, 16), I3(1, 8, 8), 2, 0, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_permute(fake, fake, 1, 1, 6, I3(1, 16, 16), I3(1, 8, 8), 2, 0, None) == na.NA_ERR_UNSUPPORTED
    assert lib.na_unpermute(fake, fake, 1, 1, 64, I3(1, 16, 16), I3(1, 8, 8), 3, None) == na.NA_ERR_INVALID_ARG
    assert lib.na_unpermute_lse(fake, None, 1, 1, I3(1, 16, 16), I3(1, 8, 8), None) == na.NA_ERR_INVALID_ARG
    # tile map capacity
    nnz = ctypes.c_int64()
    buf = (ctypes.c_int32 * 4)()
    qp = (ctypes.c_int32 * 64)()
    nf = (ctypes.c_int32 * 64)()
    st = lib.na_build_tile_map(good["grid"], good["window"], good["stride"], I3(1, 4, 4), I3(1, 4, 4),
                               qp, buf, nf, 4, ctypes.byref(nnz), None)
    assert st == na.NA_ERR_INVALID_ARG and nnz.value == 100
    # the workspace query reports invalid problems as 0 bytes
    assert lib.na_workspace_bytes(1, 1, 64, I3(1, 4, 4), I3(1, 5, 5), I3(1, 1, 1), na.NA_BF16) == 0


def test_last_error_is_per_call(na):
    lib = na.load()
    lib.na_workspace_bytes(1, 1, 64, na.I3(1, 4, 4), na.I3(1, 5, 5), na.I3(1, 1, 1), na.NA_BF16)
    assert na.na_last_error() != ""
    na.na_choose_tiles((1, 16, 16), (1, 5, 5), (1, 1, 1), 64, na.NA_BF16)
    assert na.na_last_error() == ""


def test_backward_arguments_rejected(na):
    lib = na.load()
    I3 = na.I3
    g, w, s = I3(1, 16, 16), I3(1, 5, 5), I3(1, 1, 1)
    fake = 1 << 20
    ws = na.na_backward_workspace_bytes(1, 1, 64, (1, 16, 16), (1, 5, 5), (1, 1, 1), na.NA_BF16)
    assert ws > 0

    def bwd(dt=na.NA_BF16, D=64, ws_bytes=ws, lse=fake, grid=g, ws_ptr=fake):
        return lib.na_backward(fake, fake, fake, fake, fake, lse, fake, fake, fake, 1, 1, D, grid, w, s, 0.125,
                               dt, ws_ptr, ws_bytes, None)

    assert bwd(dt=na.NA_F32) == na.NA_ERR_UNSUPPORTED
    assert bwd(dt=na.NA_FP8_E4M3) == na.NA_ERR_UNSUPPORTED
    assert bwd(D=48) == na.NA_ERR_UNSUPPORTED
    assert bwd(grid=I3(1, 16, 3)) != na.NA_OK          # window 5 > W 3: invalid geometry
    assert bwd(lse=None) == na.NA_ERR_INVALID_ARG
    assert bwd(ws_ptr=None) == na.NA_ERR_INVALID_ARG
    assert bwd(ws_bytes=ws - 1) == na.NA_ERR_WORKSPACE
    # a grid narrower than 8 along W gets tiles padded to 8 along W (the
    # dk/dv kernel works on 8-query groups): a plan, sized for the padding
    narrow = lib.na_backward_workspace_bytes(1, 1, 64, I3(1, 64, 4), I3(1, 5, 3), I3(1, 1, 1), na.NA_BF16)
    assert narrow >= 4 * 64 * 8 * 64 * 2
    # linear in the token count
    a = na.na_backward_workspace_bytes(1, 2, 128, (1, 64, 64), (1, 9, 9), (1, 1, 1), na.NA_BF16)
    b = na.na_backward_workspace_bytes(1, 2, 128, (1, 128, 64), (1, 9, 9), (1, 1, 1), na.NA_BF16)
    assert 1.9 < b / a < 2.1


def test_topk_arguments_rejected(na):
    lib = na.load()
    I3 = na.I3
    g = I3(1, 64, 64)
    fake = 1 << 20
    tq, tk = na.na_topk_tiles((1, 64, 64), 64, na.NA_BF16)
    nk = math.prod(-(-L // t) for L, t in zip((1, 64, 64), tk))
    ws = na.na_topk_workspace_bytes(1, 2, 64, (1, 64, 64), 5, na.NA_BF16)
    assert ws > 0

    def fwd(keep=5, dt=na.NA_BF16, D=64, ws_bytes=ws, q=fake):
        return lib.na_topk_forward(q, fake, fake, fake, None, 1, 2, D, g, keep, 0.125, dt, fake, ws_bytes, None)

    assert fwd(dt=na.NA_F32, D=32) == na.NA_ERR_UNSUPPORTED
    assert fwd(keep=0) == na.NA_ERR_INVALID_ARG and fwd(keep=nk + 1) == na.NA_ERR_INVALID_ARG
    assert fwd(q=None) == na.NA_ERR_INVALID_ARG
    assert fwd(ws_bytes=ws - 1) == na.NA_ERR_WORKSPACE
    assert lib.na_topk_select(fake, fake, 1, 2, 64, g, 5, na.NA_BF16, None, fake, fake, ws, None) == \
        na.NA_ERR_INVALID_ARG
    # the tile map part of the workspace grows with keep
    assert na.na_topk_workspace_bytes(1, 2, 64, (1, 64, 64), nk, na.NA_BF16) > ws


def test_launch_size_limits_rejected(na):
    # one launch holds fewer than 2^32 work-items: problems beyond that (and
    # grids beyond 2^30 tokens) are refused on the host before any launch
    lib = na.load()
    I3 = na.I3
    fake = 1 << 20
    big, one = I3(1, 32768, 32768), I3(1, 1, 1)
    ws = 1 << 40

    def fwd(heads):
        return lib.na_forward(fake, fake, fake, fake, None, 1, heads, 128, big, one, one, 0.125, na.NA_BF16, None,
                              fake, ws, None)

    assert fwd(64) == na.NA_ERR_UNSUPPORTED and "launch" in na.na_last_error()
    assert lib.na_permute(fake, fake, 1, 1, 128, big, I3(1, 8, 8), 2, 0, None) == na.NA_ERR_UNSUPPORTED
    assert lib.na_permute(fake, fake, 1, 1, 128, I3(2, 32768, 32768), I3(1, 16, 16), 2, 0, None) == \
        na.NA_ERR_UNSUPPORTED
    assert lib.na_unpermute(fake, fake, 1, 1, 128, big, I3(1, 8, 8), 2, None) == na.NA_ERR_UNSUPPORTED
    assert lib.na_workspace_bytes(1, 64, 128, big, one, one, na.NA_BF16) == 0


def test_noalloc_arguments_rejected(na):
    # na_forward_noalloc validates everything, the tile map's size against
    # its fixed device buffer included, before any HIP call
    lib = na.load()
    I3 = na.I3
    fake = 1 << 20

    def fwd(dt=na.NA_BF16, D=128, grid=I3(1, 16, 16), window=I3(1, 5, 5), q=fake, out=fake, B=1):
        return lib.na_forward_noalloc(q, fake, fake, out, None, B, 2, D, grid, window, I3(1, 1, 1), 0.125, dt, None)

    assert fwd(dt=na.NA_FP8_E4M3) == na.NA_ERR_UNSUPPORTED
    assert fwd(dt=na.NA_F32, D=32) == na.NA_ERR_UNSUPPORTED
    assert fwd(D=48) == na.NA_ERR_UNSUPPORTED
    assert fwd(window=I3(1, 17, 5)) == na.NA_ERR_INVALID_ARG
    assert fwd(q=None) == na.NA_ERR_INVALID_ARG
    assert fwd(out=fake + 8) == na.NA_ERR_INVALID_ARG
    assert fwd(B=0, q=None) == na.NA_OK
    # dense attention over 600,000 tokens: its tile map (millions of entries)
    # does not fit the fixed buffer
    n = 600000
    tq, tk = na.na_choose_tiles((1, 1, n), (1, 1, n), (1, 1, 1), 128, na.NA_BF16)
    nnz = math.prod(-(-n // t) for t in (tq[2],)) * (-(-n // tk[2]))
    assert 4 * nnz > na.NOALLOC_SCRATCH_BYTES
    assert fwd(grid=I3(1, 1, n), window=I3(1, 1, n)) == na.NA_ERR_UNSUPPORTED
    assert "fixed" in na.na_last_error()
