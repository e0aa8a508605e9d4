"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against something fixed by the pages or by
mathematics: values printed on the pages, a hand-derived example, a library
routine in a case where GNA reduces to it, brute force on tiny inputs,
closed forms and invariants.  Together they are chosen so that a plausible
mistake in the oracle (window offset, leader rule, clamp, a dropped scale,
a transposed operand, a wrong tile split) fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _rand(shape, rng=RNG):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# window geometry
# ---------------------------------------------------------------------------

def _nearest_window_search(i, L, w):
    """Independent statement of sliding NA on one axis: among all placements
    [a, a+w) inside [0, L), take the one whose midpoint is closest to the
    query, ties going to the placement with more keys before the query."""
    best = None
    for a in range(0, L - w + 1):
        d = abs(a + (w - 1) / 2.0 - i)
        if best is None or d < best[0] - 1e-12:
            best = (d, a)
    return best[1]


def test_stride1_window_is_nearest_placement():
    for L in range(1, 14):
        for w in range(1, L + 1):
            for i in range(L):
                assert oracle.window_start(i, L, w, 1) == _nearest_window_search(i, L, w), (L, w, i)


def test_stride_equal_window_gives_disjoint_blocks():
    # s = w with w | L: the windows tile the axis, query i sees block i // w
    for L in range(1, 40):
        for w in range(1, L + 1):
            if L % w:
                continue
            for i in range(L):
                assert oracle.window_start(i, L, w, w) == (i // w) * w


def test_stride_groups_share_one_window_and_jump_by_at_most_s():
    for L, w, s in [(30, 18, 16), (48, 24, 8), (80, 24, 8), (256, 64, 16), (13, 7, 3), (9, 4, 4)]:
        st = oracle.window_starts(L, w, s)
        for i in range(L):
            assert st[i] == st[(i // s) * s]          # one window per group
            assert 0 <= st[i] <= L - w                # inside the grid
        d = np.diff(st)
        assert (d >= 0).all() and (d <= s).all()      # monotone, jumps <= s


def test_worked_1d_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_1d.json")))
    val = lambda x: {"ln3": math.log(3), "ln4": math.log(4), "ln6": math.log(6)}.get(x, x)
    q = np.array([val(x) for x in g["q"]]).reshape(1, 3, 1, 1)
    k = np.array([val(x) for x in g["k"]]).reshape(1, 3, 1, 1)
    v = np.array([val(x) for x in g["v"]]).reshape(1, 3, 1, 1)
    out, lse = oracle.attend(q, k, v, g["grid"], g["window"], g["stride"], g["scale"])
    np.testing.assert_allclose(out[0, :, 0, 0], g["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, :, 0], [val(x) for x in g["lse"]], rtol=0, atol=1e-12)


def test_page_sparsity_table():
    g = json.load(open(os.path.join(GOLDEN, "gna_page_sparsity.json")))
    for row in g["rows"]:
        sp = oracle.sparsity(g["grid"], row["window"])
        assert round(100 * sp, 1) == row["sparsity_percent"]


@pytest.mark.parametrize("grid,window,stride", [
    ((1, 1, 7), (1, 1, 3), (1, 1, 1)),
    ((1, 5, 6), (1, 3, 4), (1, 2, 3)),
    ((3, 4, 5), (2, 3, 2), (1, 2, 2)),
    ((4, 4, 4), (4, 2, 3), (2, 1, 3)),
])
def test_key_set_brute_force(grid, window, stride):
    N = math.prod(grid)
    W = math.prod(window)
    table = oracle.key_index_table(grid, window, stride)
    for qi in range(N):
        coord = np.unravel_index(qi, grid)
        ks = oracle.key_set(coord, grid, window, stride)
        assert len(ks) == W == len(set(ks.tolist()))
        np.testing.assert_array_equal(table[qi], ks)
        # membership by brute force over every key of the grid
        brute = []
        for kj in range(N):
            kc = np.unravel_index(kj, grid)
            ok = all(oracle.window_start(int(c), L, w, s) <= int(x) < oracle.window_start(int(c), L, w, s) + w
                     for c, x, L, w, s in zip(coord, kc, grid, window, stride))
            if ok:
                brute.append(kj)
        np.testing.assert_array_equal(brute, ks)


def test_invalid_geometry_rejected():
    for g, w, s in [((8,), (9,), (1,)), ((8,), (4,), (5,)), ((8,), (4,), (0,)), ((8,), (0,), (1,))]:
        with pytest.raises(ValueError):
            oracle.validate_geometry(g, w, s)


# ---------------------------------------------------------------------------
# attention values
# ---------------------------------------------------------------------------

def _torch_sdpa64(q, k, v, scale):
    """Dense fp64 attention by the library routine; q,k,v [B, N, h, D]."""
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    lse = torch.logsumexp(scale * tq @ tk.transpose(-1, -2), dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


@pytest.mark.parametrize("grid,stride", [((1, 6, 7), (1, 2, 3)), ((3, 4, 5), (1, 1, 1)), ((2, 3, 4), (2, 3, 2))])
def test_window_equal_grid_is_dense_attention(grid, stride):
    B, h, D = 2, 3, 8
    N = math.prod(grid)
    q, k, v = (_rand((B, N, h, D)) for _ in range(3))
    out, lse = oracle.attend(q, k, v, grid, grid, stride, 0.37)
    ro, rl = _torch_sdpa64(q, k, v, 0.37)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid,window", [((1, 8, 12), (1, 4, 3)), ((4, 6, 4), (2, 3, 2)), ((1, 1, 30), (1, 1, 5))])
def test_stride_equal_window_is_block_diagonal_attention(grid, window):
    B, h, D = 1, 2, 4
    T, H, W = grid
    wt, wh, ww = window
    N = math.prod(grid)
    q, k, v = (_rand((B, N, h, D)) for _ in range(3))
    out, lse = oracle.attend(q, k, v, grid, window, window, 0.5)

    def blocks(x):   # [B, N, h, D] -> [B*nblocks, w, h, D]
        x = x.reshape(B, T // wt, wt, H // wh, wh, W // ww, ww, h, D)
        x = x.transpose(0, 1, 3, 5, 2, 4, 6, 7, 8)
        return x.reshape(-1, wt * wh * ww, h, D)

    ro, rl = _torch_sdpa64(blocks(q), blocks(k), blocks(v), 0.5)

    def unblocks(x, last):
        x = x.reshape(B, T // wt, H // wh, W // ww, wt, wh, ww, h, *last)
        nd = x.ndim
        perm = (0, 1, 4, 2, 5, 3, 6) + tuple(range(7, nd))
        return x.transpose(perm).reshape(B, N, h, *last)

    np.testing.assert_allclose(out, unblocks(ro, (D,)), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, unblocks(rl, ()), rtol=0, atol=1e-12)


def test_window_one_returns_v_exactly():
    grid, B, h, D = (2, 5, 6), 1, 2, 8
    N = math.prod(grid)
    q, k, v = (_rand((B, N, h, D)) for _ in range(3))
    out, lse = oracle.attend(q, k, v, grid, (1, 1, 1), (1, 1, 1), 0.3)
    assert np.array_equal(out, v)
    np.testing.assert_allclose(lse, 0.3 * np.einsum("bnhd,bnhd->bnh", q, k), rtol=0, atol=1e-13)


def test_zero_query_gives_window_mean():
    grid, window, stride = (3, 7, 6), (2, 3, 4), (1, 2, 3)
    B, h, D = 1, 2, 5
    N, W = math.prod(grid), math.prod(window)
    q = np.zeros((B, N, h, D))
    k, v = _rand((B, N, h, D)), _rand((B, N, h, D))
    out, lse = oracle.attend(q, k, v, grid, window, stride, 1.0)
    np.testing.assert_allclose(lse, math.log(W), rtol=0, atol=1e-13)
    for qi in range(N):
        ks = oracle.key_set(np.unravel_index(qi, grid), grid, window, stride)
        np.testing.assert_allclose(out[0, qi], v[0, ks].mean(axis=0), rtol=0, atol=1e-13)


def test_algebraic_invariants():
    grid, window, stride = (2, 6, 7), (2, 3, 4), (1, 1, 2)
    B, h, D = 1, 2, 6
    N = math.prod(grid)
    q, k, v = (_rand((B, N, h, D)) for _ in range(3))
    sc = 0.41
    out, lse = oracle.attend(q, k, v, grid, window, stride, sc)
    # constant values -> the constant
    o2, _ = oracle.attend(q, k, np.full_like(v, 2.5), grid, window, stride, sc)
    np.testing.assert_allclose(o2, 2.5, rtol=0, atol=1e-13)
    # k + c*1: output unchanged, lse shifted by scale * <q, c*1>
    c = 0.7
    o3, l3 = oracle.attend(q, k + c, v, grid, window, stride, sc)
    np.testing.assert_allclose(o3, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3, lse + sc * c * q.sum(-1), rtol=0, atol=1e-12)
    # affine in v
    o4, l4 = oracle.attend(q, k, 3.0 * v - 1.25, grid, window, stride, sc)
    np.testing.assert_allclose(o4, 3.0 * out - 1.25, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l4, lse, rtol=0, atol=0)
    # the output is a convex combination of the window's values
    for qi in range(0, N, 5):
        ks = oracle.key_set(np.unravel_index(qi, grid), grid, window, stride)
        assert (out[0, qi] <= v[0, ks].max(0) + 1e-12).all()
        assert (out[0, qi] >= v[0, ks].min(0) - 1e-12).all()


def test_translation_equivariance_sliding_mode():
    # GNA page section 1.1 / 1.2 table: stride 1 keeps translation
    # equivariance.  Grids A = X[:, :L-d] and B = X[:, d:]; a query whose
    # window is not shifted by the border in either grid sees the same keys.
    H, W, w, d = 12, 13, 5, 3
    B_, h, D = 1, 2, 4
    X = [_rand((B_, 1, H, W, h, D)) for _ in range(3)]
    A = [x[:, :, :, : W - d] for x in X]
    Bt = [x[:, :, :, d:] for x in X]
    oa, la = oracle.attend(*A, (1, H, W - d), (1, w, w), (1, 1, 1), 0.5)
    ob, lb = oracle.attend(*Bt, (1, H, W - d), (1, w, w), (1, 1, 1), 0.5)
    oa = oa.reshape(B_, H, W - d, h, D)
    ob = ob.reshape(B_, H, W - d, h, D)
    half = w // 2
    checked = 0
    for y in range(H):
        for x in range(half + d, W - d - half):     # interior of both grids
            if half <= y < H - half:
                np.testing.assert_allclose(ob[0, y, x - d], oa[0, y, x], rtol=0, atol=1e-12)
                checked += 1
    assert checked > 10


def test_block_mode_equivariant_only_for_multiples_of_stride():
    L, w, s = 40, 8, 4
    B_, h, D = 1, 1, 3
    X = [_rand((B_, 1, 1, L, h, D)) for _ in range(3)]

    def run(off, n):
        return oracle.attend(*[x[:, :, :, off:off + n] for x in X], (1, 1, n), (1, 1, w), (1, 1, s), 1.0)[0]

    n = 28
    base = run(0, n)
    shifted = run(s, n)            # shift by a multiple of s: interior agrees
    np.testing.assert_allclose(shifted[0, 8:16], base[0, 12:20], rtol=0, atol=1e-12)
    odd = run(1, n)                # shift by 1: the block pattern moves
    assert not np.allclose(odd[0, 8:16], base[0, 9:17], atol=1e-6)


# ---------------------------------------------------------------------------
# tile map
# ---------------------------------------------------------------------------

def _tile_map_nd_brute(grid, window, stride, tq, tk):
    """Pair counts between every (Q tile, KV tile) by enumerating all N-D
    (query, key) pairs; same ordering rule as the oracle's CSR."""
    N = math.prod(grid)
    nQ = [-(-L // t) for L, t in zip(grid, tq)]
    nK = [-(-L // t) for L, t in zip(grid, tk)]
    pairs = {}
    for qi in range(N):
        qc = np.unravel_index(qi, grid)
        a = tuple(int(c) // t for c, t in zip(qc, tq))
        for kj in oracle.key_set(qc, grid, window, stride):
            kc = np.unravel_index(int(kj), grid)
            c = tuple(int(x) // t for x, t in zip(kc, tk))
            pairs[(a, c)] = pairs.get((a, c), 0) + 1
    qptr, kv, nfull = [0], [], []
    for a in itertools.product(*[range(n) for n in nQ]):
        vq = math.prod(min(t, L - ai * t) for ai, t, L in zip(a, tq, grid))
        full, bnd = [], []
        for c in itertools.product(*[range(n) for n in nK]):
            p = pairs.get((a, c), 0)
            if p == 0:
                continue
            lin = int(np.ravel_multi_index(c, nK))
            (full if p == vq * math.prod(tk) else bnd).append(lin)
        kv += sorted(full) + sorted(bnd)
        nfull.append(len(full))
        qptr.append(len(kv))
    return np.array(qptr), np.array(kv), np.array(nfull), sum(pairs.values())


@pytest.mark.parametrize("grid,window,stride,tq,tk", [
    ((1, 9, 11), (1, 5, 4), (1, 1, 2), (1, 4, 4), (1, 2, 4)),
    ((3, 6, 7), (2, 4, 3), (2, 2, 1), (2, 2, 4), (1, 4, 2)),
    ((1, 1, 17), (1, 1, 6), (1, 1, 3), (1, 1, 8), (1, 1, 4)),
    ((4, 8, 8), (4, 4, 4), (4, 4, 4), (2, 4, 4), (2, 4, 4)),
    ((5, 5, 5), (5, 5, 5), (1, 1, 1), (2, 2, 2), (4, 4, 4)),
])
def test_tile_map_against_nd_brute_force(grid, window, stride, tq, tk):
    qptr, kv, nfull, pr = oracle.tile_map(grid, window, stride, tq, tk, return_pairs=True)
    bq, bkv, bnf, total = _tile_map_nd_brute(grid, window, stride, tq, tk)
    np.testing.assert_array_equal(qptr, bq)
    np.testing.assert_array_equal(kv, bkv)
    np.testing.assert_array_equal(nfull, bnf)
    assert pr.sum() == total == math.prod(grid) * math.prod(window)


@pytest.mark.parametrize("L,w,s,tq,tk", [(11, 4, 2, 4, 2), (17, 6, 3, 8, 4), (9, 9, 1, 4, 8), (5, 1, 1, 2, 2)])
def test_tile_pairs_1d_against_key_sets(L, w, s, tq, tk):
    # the per-axis pair counts against the 1-D key sets, tile by tile, and
    # the invariant that every query holds exactly w keys
    pairs, vq, vk = oracle.tile_pairs_1d(L, w, s, tq, tk)
    want = np.zeros_like(pairs)
    for i in range(L):
        for j in oracle.key_set((0, 0, i), (1, 1, L), (1, 1, w), (1, 1, s)):
            want[i // tq, int(j) // tk] += 1
    np.testing.assert_array_equal(pairs, want)
    assert pairs.sum() == L * w
    assert vq.sum() == L and vk.sum() == L


def test_effective_flops_counts_attended_pairs():
    # 4 D FLOPs (QK^T and PV multiply-adds) per attended (query, key) pair,
    # counted by enumerating the key sets; window = grid gives dense attention
    grid, window, stride, b, h, d = (3, 5, 6), (2, 3, 4), (1, 3, 2), 2, 3, 16
    pairs = sum(len(oracle.key_set(np.unravel_index(i, grid), grid, window, stride))
                for i in range(math.prod(grid)))
    assert oracle.effective_flops(b, h, grid, window, d) == 4.0 * b * h * d * pairs
    n = math.prod(grid)
    assert oracle.effective_flops(1, 1, grid, grid, d) == 4.0 * n * n * d


def test_kv_tile_is_full_against_slot_coordinates():
    # a KV tile is full iff its last slot along every axis is inside the grid
    grid, tile = (3, 10, 12), (2, 4, 8)
    n = [-(-L // t) for L, t in zip(grid, tile)]
    want = [all((c + 1) * t <= L for c, t, L in zip(cc, tile, grid))
            for cc in itertools.product(*[range(k) for k in n])]
    np.testing.assert_array_equal(oracle.kv_tile_is_full(grid, tile), np.array(want))
    assert oracle.kv_tile_is_full((4, 8, 8), (2, 4, 8)).all()


def test_video_block_config_is_perfectly_block_sparse():
    # GNA page sections 1.1 and 3.1: at 91 % sparsity the speed-up matches the
    # FLOP reduction, i.e. the KV tiles align with the windows and no
    # compute is wasted.  With (2,8,8) tiles every listed tile is full.
    st = oracle.tile_map_stats((30, 48, 80), (18, 24, 24), (16, 8, 8), (2, 8, 8), (2, 8, 8))
    assert st["n_boundary"] == 0
    assert st["kv_tiles_per_q_tile"] == 81
    assert st["efficiency"] == 1.0


def test_tile_map_stats_regression():
    # counts of the workloads' tile maps (regression pins for the host builder)
    cases = [
        ((1, 16, 16), (1, 5, 5), (1, 1, 1), (1, 4, 4), (1, 4, 4), 100, 0),
        ((1, 64, 64), (1, 17, 17), (1, 1, 1), (1, 8, 8), (1, 8, 8), 576, 100),
        ((1, 64, 64), (1, 16, 16), (1, 8, 8), (1, 8, 8), (1, 4, 4), 1024, 1024),
        ((30, 48, 80), (30, 40, 40), (1, 1, 1), (2, 8, 8), (2, 8, 8), 432000, 252000),
        ((1, 256, 256), (1, 64, 64), (1, 16, 16), (1, 16, 16), (1, 8, 8), 16384, 16384),
    ]
    for g, w, s, tq, tk, nnz, nfull in cases:
        st = oracle.tile_map_stats(g, w, s, tq, tk)
        assert (st["nnz"], st["n_full"]) == (nnz, nfull), g


# ----------------------------------------------------------------------------
# backward oracle pins
# ----------------------------------------------------------------------------

def _loss(q, k, v, dout, grid, window, stride, scale):
    out, _ = oracle.attend(q, k, v, grid, window, stride, scale)
    return float((out * dout).sum())


@pytest.mark.parametrize("grid,window,stride", [((1, 4, 5), (1, 3, 2), (1, 1, 2)), ((2, 3, 4), (2, 2, 3), (1, 2, 3))])
def test_backward_matches_finite_differences(grid, window, stride):
    # pins the backward to the forward oracle: central differences of
    # L = sum <dout, attend(q, k, v)> in float64
    rng = np.random.default_rng(61)
    N, D, h = math.prod(grid), 3, 2
    q, k, v, do = (rng.standard_normal((1, N, h, D)) for _ in range(4))
    scale = 0.7
    dq, dk, dv = oracle.attend_backward(q, k, v, do, grid, window, stride, scale)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = _loss(q, k, v, do, grid, window, stride, scale)
            x[idx] = x0 - eps
            lm = _loss(q, k, v, do, grid, window, stride, scale)
            x[idx] = x0
            num[idx] = (lp - lm) / (2 * eps)
        assert np.abs(num - g).max() < 1e-7 * max(1.0, np.abs(num).max())


def test_backward_dense_limit_matches_autograd():
    # window = grid: plain softmax attention; torch autograd in float64
    grid, window, stride = (1, 4, 6), (1, 4, 6), (1, 1, 1)
    rng = np.random.default_rng(62)
    N, D, h = 24, 8, 2
    q, k, v, do = (rng.standard_normal((2, N, h, D)) for _ in range(4))
    scale = 0.35
    dq, dk, dv = oracle.attend_backward(q, k, v, do, grid, window, stride, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = torch.einsum("bqhd,bkhd->bhqk", tq, tk) * scale
    out = torch.einsum("bhqk,bkhd->bqhd", torch.softmax(s, dim=-1), tv)
    (out * torch.tensor(do)).sum().backward()
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a - t.grad.numpy()).max() < 1e-12


def test_backward_window_one():
    # each query sees only itself: out = v, so dq = dk = 0 and dv = dout
    grid = (2, 3, 5)
    rng = np.random.default_rng(63)
    q, k, v, do = (rng.standard_normal((1, 30, 2, 4)) for _ in range(4))
    dq, dk, dv = oracle.attend_backward(q, k, v, do, grid, (1, 1, 1), (1, 1, 1), 0.5)
    # p = exp(s - lse) = 1 up to the rounding of s computed twice
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    assert np.abs(dv - do).max() < 1e-14


@pytest.mark.parametrize("grid,window,stride", [((3, 7, 9), (2, 3, 5), (1, 2, 3)), ((1, 12, 12), (1, 5, 5), (1, 1, 1))])
def test_backward_sum_identities(grid, window, stride):
    # sum_j dS_ij = 0 for every query, so the dk rows sum to zero; the rows of
    # p sum to one, so the dv rows sum to the dout rows
    rng = np.random.default_rng(64)
    N = math.prod(grid)
    q, k, v, do = (rng.standard_normal((1, N, 2, 6)) for _ in range(4))
    dq, dk, dv = oracle.attend_backward(q, k, v, do, grid, window, stride, 0.4)
    assert np.abs(dk.sum(axis=1)).max() < 1e-11
    assert np.abs(dv.sum(axis=1) - do.sum(axis=1)).max() < 1e-11


def test_backward_selected_rows_match_full():
    grid, window, stride = (2, 6, 7), (2, 3, 4), (1, 2, 2)
    rng = np.random.default_rng(65)
    N = math.prod(grid)
    q, k, v, do = (rng.standard_normal((2, N, 1, 5)) for _ in range(4))
    full = oracle.attend_backward(q, k, v, do, grid, window, stride, 0.6)
    qs, ks = np.array([0, 5, 41, 83]), np.array([3, 17, 60])
    sel = oracle.attend_backward(q, k, v, do, grid, window, stride, 0.6, queries=qs, keys=ks)
    assert np.abs(sel[0] - full[0][:, qs]).max() < 1e-13
    assert np.abs(sel[1] - full[1][:, ks]).max() < 1e-13
    assert np.abs(sel[2] - full[2][:, ks]).max() < 1e-13
    # the inverse table is the transpose of the key table
    ktab = oracle.key_index_table(grid, window, stride)
    for key, ql in zip(range(N), oracle.query_index_lists(grid, window, stride, np.arange(N))):
        assert np.array_equal(ql, np.nonzero((ktab == key).any(axis=1))[0])


# ----------------------------------------------------------------------------
# content-selected block sparsity (top-k) oracle pins
# ----------------------------------------------------------------------------

def test_topk_all_blocks_is_dense_attention():
    # keep = every KV tile: attention over all keys, i.e. plain softmax
    # attention (torch SDPA in float64)
    grid, tq, tk = (2, 6, 8), (1, 4, 4), (2, 2, 4)
    rng = np.random.default_rng(71)
    N = math.prod(grid)
    q, k, v = (rng.standard_normal((1, N, 2, 8)).astype(np.float32) for _ in range(3))
    nK = math.prod(-(-L // t) for L, t in zip(grid, tk))
    out, lse = oracle.topk_attend(q, k, v, grid, tq, tk, nK, 0.3)
    ref, rlse = _torch_sdpa64(*(x.astype(np.float64) for x in (q, k, v)), 0.3)
    assert np.abs(out - ref).max() < 1e-12 and np.abs(lse - rlse).max() < 1e-12


def test_topk_scores_against_plain_means():
    # the float32-order scores equal the plain float64 definition to float32
    # accuracy, and the selected tiles are the top-k of the float64 scores
    # whenever the gap at the cut is wide
    grid, tq, tk = (3, 5, 9), (1, 4, 4), (1, 2, 4)
    rng = np.random.default_rng(72)
    N = math.prod(grid)
    q, k = (rng.standard_normal((1, N, 1, 16)).astype(np.float32) for _ in range(2))
    qm = oracle.block_means_f32(q, grid, tq)
    km = oracle.block_means_f32(k, grid, tk)
    s32 = oracle.block_scores_f32(qm, km)[0, 0]

    def tiles(tile):
        nt = [-(-L // t) for L, t in zip(grid, tile)]
        lists = []
        for a in range(math.prod(nt)):
            a0, rem = divmod(a, nt[1] * nt[2])
            a1, a2 = divmod(rem, nt[2])
            toks = [(t * grid[1] + y) * grid[2] + x
                    for t in range(a0 * tile[0], min((a0 + 1) * tile[0], grid[0]))
                    for y in range(a1 * tile[1], min((a1 + 1) * tile[1], grid[1]))
                    for x in range(a2 * tile[2], min((a2 + 1) * tile[2], grid[2]))]
            lists.append(toks)
        return lists

    qmean = np.array([q[0, t, 0].astype(np.float64).mean(axis=0) for t in tiles(tq)])
    kmean = np.array([k[0, t, 0].astype(np.float64).mean(axis=0) for t in tiles(tk)])
    s64 = qmean @ kmean.T
    assert np.abs(s32 - s64).max() < 1e-5 * max(1.0, np.abs(s64).max())
    keep = 5
    idx, nf = oracle.topk_select(q, k, grid, tq, tk, keep)
    for a in range(s64.shape[0]):
        srt = np.sort(s64[a])[::-1]
        if srt[keep - 1] - srt[keep] > 1e-4:
            assert set(idx[0, 0, a]) == set(np.argsort(-s64[a])[:keep])


def test_topk_single_dominant_block():
    # keys of one KV tile align with every query, the rest are orthogonal:
    # keep = 1 picks that tile and the attention is over its keys only
    grid, tq, tk = (1, 8, 8), (1, 4, 8), (1, 4, 4)
    N, D = 64, 4
    q = np.zeros((1, N, 1, D), dtype=np.float32)
    k = np.zeros((1, N, 1, D), dtype=np.float32)
    q[..., 0] = 1.0
    k[..., 1] = 1.0
    hot = oracle.topk.__dict__["_tile_tokens"](grid, tk, 3)
    k[0, hot, 0, 0] = 2.0
    idx, nf = oracle.topk_select(q, k, grid, tq, tk, 1)
    assert (idx == 3).all() and (nf == 1).all()
    rng = np.random.default_rng(73)
    v = rng.standard_normal((1, N, 1, D))
    out, lse = oracle.topk_attend(q, k, v, grid, tq, tk, 1, 0.5)
    assert np.abs(out[0, :, 0] - v[0, hot, 0].mean(axis=0)).max() < 1e-12   # equal scores in the tile
    assert np.abs(lse - (0.5 * 2.0 + math.log(len(hot)))).max() < 1e-12


def test_topk_selection_order_and_ties():
    scores = np.array([[[3.0, 1.0, 3.0, 2.0, 3.0]]], dtype=np.float32)
    full = np.array([True, True, False, True, True])
    idx, nf = oracle.select_blocks(scores, 3, full)
    # best three: indices 0, 2, 4 (score 3, ties by index); full ones first
    assert idx.tolist() == [[[0, 4, 2]]] and nf.tolist() == [[2]]
