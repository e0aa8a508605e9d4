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
