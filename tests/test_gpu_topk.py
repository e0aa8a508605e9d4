"""GPU parity of content-selected block sparsity: the selected tile map is
compared bit for bit with the oracle's float32-order selection, the attention
over the kept tiles with the oracle's float64 attention."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, say
from synth import WORKLOADS, make_qkv

pytestmark = pytest.mark.gpu

CASES = [
    ("img64_sliding", {}, 5),                                                    # 2-D, D 64
    ("video_sliding", dict(batch=2, heads=2, grid=(5, 19, 27)), 7),              # ragged: padded tiles
    ("video_block", dict(heads=2, grid=(3, 16, 24)), 3),
    ("img64_sliding", dict(batch=1, heads=2, grid=(1, 1, 1500)), 4),             # 1-D, last tiles padded
]


def _wl(name, kw):
    return WORKLOADS[name].with_(seed=600 + len(kw), **kw)


def _oracle_select(na, wl, qc, kc, keep):
    tq, tk = na.na_topk_tiles(wl.grid, wl.head_dim, na.NA_BF16)
    B, H = wl.batch, wl.heads
    q = qc.to(torch.float32).numpy().reshape(B, -1, H, wl.head_dim)
    k = kc.to(torch.float32).numpy().reshape(B, -1, H, wl.head_dim)
    idx, nf = oracle.topk_select(q, k, wl.grid, tq, tk, keep)      # [B, H, nQ, keep], [B, H, nQ]
    return idx.reshape(B * H, -1, keep), nf.reshape(B * H, -1), tq, tk


@pytest.mark.parametrize("name,kw,keep", CASES)
def test_topk_selection_bit_exact(na, name, kw, keep):
    wl = _wl(name, kw)
    say(f"[topk] select {wl.name} grid={wl.grid} D={wl.head_dim} keep={keep}")
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    idx, nf = na.topk_select(qc.cuda(), kc.cuda(), keep)
    ridx, rnf, _, _ = _oracle_select(na, wl, qc, kc, keep)
    assert np.array_equal(idx.cpu().numpy(), ridx) and np.array_equal(nf.cpu().numpy(), rnf)


@pytest.mark.parametrize("name,kw,keep", CASES)
def test_topk_attention_all_queries(na, name, kw, keep):
    wl = _wl(name, kw)
    say(f"[topk] attend {wl.name} grid={wl.grid} keep={keep}")
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    out, lse = na.topk_forward(qc.cuda(), kc.cuda(), vc.cuda(), keep, scale=wl.scale)
    torch.cuda.synchronize()
    _, _, tq, tk = _oracle_select(na, wl, qc, kc, keep)
    f = lambda x: x.to(torch.float32).numpy().reshape(wl.batch, -1, wl.heads, wl.head_dim)
    ro, rl = oracle.topk_attend(f(qc), f(kc), f(vc), wl.grid, tq, tk, keep, wl.scale)
    go = out.cpu().to(torch.float64).numpy().reshape(ro.shape)
    gl = lse.cpu().to(torch.float64).numpy().reshape(rl.shape)
    eo, el = float(np.abs(go - ro).max()), float(np.abs(gl - rl).max())
    say(f"  max|out-oracle|={eo:.3e} max|lse-oracle|={el:.3e}")
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]


def test_topk_keep_all_equals_dense_forward(na):
    # every KV tile kept: the same tiles in the same order as the dense
    # (window = grid) forward, so the results agree bit for bit
    wl = _wl("video_block", dict(heads=2, grid=(3, 16, 24)))
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    tq, tk = na.na_topk_tiles(wl.grid, wl.head_dim, na.NA_BF16)
    nk = math.prod(-(-L // t) for L, t in zip(wl.grid, tk))
    o1, l1 = na.topk_forward(q, k, v, nk, scale=wl.scale)
    o2, l2 = na.forward(q, k, v, wl.grid, (1, 1, 1), scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_topk_video_full_grid_two_heads(na):
    # the video grid at full size (450 Q tiles x 900 KV tiles), 2 heads, 81
    # kept tiles per Q tile (9 %, the block-sparse configuration's density)
    wl = WORKLOADS["video_block"].with_(heads=2, seed=606)
    keep = 81
    say("[topk] video grid, 2 heads, keep 81")
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    idx, nf = na.topk_select(q, k, keep)
    ridx, rnf, tq, tk = _oracle_select(na, wl, qc, kc, keep)
    assert np.array_equal(idx.cpu().numpy(), ridx) and np.array_equal(nf.cpu().numpy(), rnf)
    out, lse = na.topk_forward(q, k, v, keep, scale=wl.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(607)
    qs = np.unique(np.concatenate([rng.integers(0, wl.tokens, 96), [0, wl.tokens - 1]]))
    f = lambda x: x.to(torch.float32).numpy().reshape(1, -1, 2, wl.head_dim)
    ro, rl = oracle.topk_attend(f(qc), f(kc), f(vc), wl.grid, tq, tk, keep, wl.scale, queries=qs)
    go = out.cpu().to(torch.float64).numpy().reshape(1, -1, 2, wl.head_dim)[:, qs]
    gl = lse.cpu().to(torch.float64).numpy().reshape(1, -1, 2)[:, qs]
    eo, el = float(np.abs(go - ro).max()), float(np.abs(gl - rl).max())
    say(f"  {len(qs)} queries: max|out-oracle|={eo:.3e} max|lse-oracle|={el:.3e}")
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]


U32 = 2.0 ** -24   # unit roundoff of float32


def _means64(x, grid, tile):
    """Per tile: float64 means of x ([B, N, heads, D]) over its real tokens,
    and a bound on how far the kernel's float32 mean can be from it (tokens
    summed one by one in in-tile row-major order: each addition errs by at
    most u |partial sum|; then one division).  Returns [B, heads, nTiles, D]
    arrays (mean, bound)."""
    B, N, H, D = x.shape
    nt = [-(-L // t) for L, t in zip(grid, tile)]
    pad = np.zeros((B, nt[0] * tile[0], nt[1] * tile[1], nt[2] * tile[2], H, D))
    cnt = np.zeros(pad.shape[1:4])
    pad[:, :grid[0], :grid[1], :grid[2]] = x.reshape(B, *grid, H, D)
    cnt[:grid[0], :grid[1], :grid[2]] = 1.0
    # [B, tiles, in-tile tokens (row-major), H, D]
    t = pad.reshape(B, nt[0], tile[0], nt[1], tile[1], nt[2], tile[2], H, D).transpose(0, 1, 3, 5, 2, 4, 6, 7, 8)
    t = t.reshape(B, -1, tile[0] * tile[1] * tile[2], H, D)
    n = cnt.reshape(nt[0], tile[0], nt[1], tile[1], nt[2], tile[2]).sum(axis=(1, 3, 5)).reshape(-1)
    part = np.abs(np.cumsum(t, axis=2))[:, :, 1:].sum(axis=2)          # sum_i |S_i|
    mean = t.sum(axis=2) / n[None, :, None, None]
    bound = U32 * part / n[None, :, None, None] + U32 * np.abs(mean)
    return mean.transpose(0, 2, 1, 3), bound.transpose(0, 2, 1, 3)


def _score_bounds(qm, dq, km, dk):
    """float64 scores <qm_a, km_c> and a bound on the float32 evaluation's
    error: input errors, one rounding per product and u |partial sum| per
    addition over the head dimension (in order); doubled for second-order
    terms.  qm [nQ, D], km [nK, D]."""
    s = qm @ km.T
    err = np.abs(dq) @ np.abs(km).T + np.abs(qm) @ np.abs(dk).T + U32 * (np.abs(qm) @ np.abs(km).T)
    for a0 in range(0, qm.shape[0], 32):
        prod = qm[a0:a0 + 32, None, :] * km[None, :, :]
        err[a0:a0 + 32] += U32 * np.abs(np.cumsum(prod, axis=-1))[..., 1:].sum(axis=-1)
    return s, 2.0 * err


@pytest.mark.parametrize("name,kw,keep", CASES + [("video_block", dict(heads=2, seed=606), 81)])
def test_topk_selection_is_top_k_of_float64_scores(na, name, kw, keep):
    # tutorial ("Video-generation inference speed-up: sparse attention
    # configuration tutorial") section 6: score the blocks by their means and
    # keep the best.  The kept set must be the top-k of the float64 scores
    # <mean q, mean k> on every row whose gap at the cut exceeds the float32
    # evaluation's error bound for the two scores there.
    wl = WORKLOADS[name].with_(**kw) if "seed" in kw else _wl(name, kw)
    say(f"[topk] float64 top-k {wl.name} grid={wl.grid} keep={keep}")
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    idx, _ = na.topk_select(qc.cuda(), kc.cuda(), keep)
    tq, tk = na.na_topk_tiles(wl.grid, wl.head_dim, na.NA_BF16)
    B, H, D = wl.batch, wl.heads, wl.head_dim
    f = lambda x: x.to(torch.float64).numpy().reshape(B, -1, H, D)
    qm, dq = _means64(f(qc), wl.grid, tq)
    km, dk = _means64(f(kc), wl.grid, tk)
    gpu = idx.cpu().numpy().reshape(B, H, -1, keep)
    checked = rows = 0
    for b in range(B):
        for h in range(H):
            s64, eps = _score_bounds(qm[b, h], dq[b, h], km[b, h], dk[b, h])
            for a in range(s64.shape[0]):
                rows += 1
                order = np.argsort(-s64[a], kind="stable")
                if keep < len(order):
                    gap = s64[a, order[keep - 1]] - s64[a, order[keep]]
                    if gap <= eps[a, order[keep - 1]] + eps[a, order[keep]]:
                        continue
                checked += 1
                assert set(gpu[b, h, a].tolist()) == set(order[:keep].tolist()), (b, h, a)
    say(f"  {checked} of {rows} rows checked ({100.0 * checked / rows:.1f} %)")
    assert checked >= 0.5 * rows


def _random_topk_cases():
    from test_gpu_random import _geometry
    out = []
    for i in range(16):
        rng = np.random.default_rng(9000 + i)
        grid, _, _ = _geometry(rng)
        D = int(rng.choice([64, 128]))
        batch, heads = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        out.append((f"t{i}", grid, D, batch, heads, float(rng.uniform(0.0, 1.0))))
    return out


RANDOM_TOPK = _random_topk_cases()


@pytest.mark.parametrize("name,grid,D,batch,heads,frac", RANDOM_TOPK, ids=[c[0] for c in RANDOM_TOPK])
def test_topk_random_geometries(na, name, grid, D, batch, heads, frac):
    # seeded random 1-/2-/3-D grids (ragged, tiles padded), keep anywhere
    # from one KV tile to all of them: the kept sets bit for bit, the
    # attention over them on every query against the oracle
    wl = WORKLOADS["img64_sliding"].with_(name=name, batch=batch, heads=heads, grid=grid, window=grid,
                                          stride=(1, 1, 1), head_dim=D, seed=9100 + int(name[1:]))
    tq, tk = na.na_topk_tiles(grid, D, na.NA_BF16)
    nk = math.prod(-(-L // t) for L, t in zip(grid, tk))
    keep = max(1, min(nk, int(round(frac * nk))))
    say(f"[topk] random {name} grid={grid} D={D} B={batch} H={heads} tiles {tq} / {tk} keep {keep} of {nk}")
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    idx, nf = na.topk_select(q, k, keep)
    ridx, rnf, _, _ = _oracle_select(na, wl, qc, kc, keep)
    assert np.array_equal(idx.cpu().numpy(), ridx) and np.array_equal(nf.cpu().numpy(), rnf)
    out, lse = na.topk_forward(q, k, v, keep, scale=wl.scale)
    torch.cuda.synchronize()
    f = lambda x: x.to(torch.float32).numpy().reshape(batch, -1, heads, D)
    ro, rl = oracle.topk_attend(f(qc), f(kc), f(vc), grid, tq, tk, keep, wl.scale)
    go = out.cpu().to(torch.float64).numpy().reshape(ro.shape)
    gl = lse.cpu().to(torch.float64).numpy().reshape(rl.shape)
    eo, el = float(np.abs(go - ro).max()), float(np.abs(gl - rl).max())
    say(f"  max|out-oracle|={eo:.3e} max|lse-oracle|={el:.3e}")
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]
