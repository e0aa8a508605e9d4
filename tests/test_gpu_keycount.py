"""GPU: exact key counts at full size, and the dense reference against the
oracle.

With scale = 0 every weight of a query's softmax is exactly 1 (bf16 1.0,
e4m3 64), so l is the number of keys the kernel visited for that query and
lse = ln l.  The oracle's key set holds exactly prod(w) keys per query (GNA
page, "GNA Sparse Attention Mechanism: Vision-Transformer Compute
Optimisation in Practice", section 1.1: a fixed-size window per query), so
lse = ln prod(w) on every query of every head, to float32 rounding of one
logarithm.  One key too many or too few anywhere moves lse by at least
ln(W / (W - 1)) ~ 1 / W (2.1e-5 at the 48,000-key sliding window, 8.7e-6 at
the dense 115,200-key one), so the bound used is 1 / (4 W) + 1e-6,
well below that step; the value tolerances of the parity tests cannot see a dropped tile.  out is then
the window mean of v (the oracle with q = 0 gives the same uniform weights),
checked on a sample of queries.

The dense full-window run (window = grid, the speed-up reference of the
video workload, GNA page section 3.1's full-attention row) is compared with
the oracle on sampled queries in the form the benchmark times."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, say, set_path
from synth import WORKLOADS, make_qkv, to_f64

pytestmark = pytest.mark.gpu

CONFIGS = ["img16_f32", "img64_sliding", "img64_block", "video_sliding", "video_block", "video_dense",
           "img256_block", "img256_block_fp8"]


@pytest.fixture(params=["qo", "grid", "tiled"])
def path(request, monkeypatch):
    """The three forms of na_forward (see gpu_util.set_path)."""
    set_path(monkeypatch, request.param)
    return request.param


def _sample(wl, n, seed):
    """The 8 corner tokens of the grid plus n random ones."""
    T, H, W = wl.grid
    corners = [(t * H + y) * W + x for t in (0, T - 1) for y in (0, H - 1) for x in (0, W - 1)]
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([corners, rng.integers(0, wl.tokens, n)])).astype(np.int64)


@pytest.mark.parametrize("name", CONFIGS)
def test_scale_zero_counts_every_key(na, name, path):
    import gpu_util
    wl = WORKLOADS[name]
    if wl.dtype != "bf16" and path == "grid":
        pytest.skip("only bf16 has the form without a workspace")
    if wl.dtype == "f32" and path == "qo":
        pytest.skip("fp32 has one form (the tiled one)")
    W = math.prod(wl.window)
    say(f"[keycount] {name} ({path}) W={W} heads={wl.heads}")
    qc, kc, vc, sc = make_qkv(wl, device="cpu")
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    f = na.Forward(q, k, v, wl.window, wl.stride, scale=0.0, qkv_scale=sc if wl.dtype == "fp8" else None,
                   workspace=gpu_util.USE_WORKSPACE or wl.dtype != "bf16")
    f.out.fill_(float("nan"))
    f.lse.fill_(float("nan"))
    out, lse = f()
    torch.cuda.synchronize()
    # every query of every head: lse = ln prod(w)
    lse_all = lse.double().cpu()
    assert torch.isfinite(lse_all).all()
    dl = float((lse_all - math.log(W)).abs().max())
    bound = 1.0 / (4 * W) + 1e-6
    say(f"  every query: max|lse - ln W| = {dl:.3e} (bound {bound:.2e}, one key ~{1.0 / W:.2e})")
    assert dl <= bound
    # out = window mean of v on a sample (all queries on the small grids)
    qs = None if wl.tokens <= 4096 else _sample(wl, 24 if W > 60000 else 56, wl.seed + 3)
    heads = range(wl.heads) if wl.tokens <= 4096 else (0, wl.heads - 1)
    o_all = out.detach().cpu().double().reshape(wl.batch, wl.tokens, wl.heads, wl.head_dim)
    zq = np.zeros((wl.batch, wl.tokens, 1, wl.head_dim))
    worst = 0.0
    for h in heads:
        kh = to_f64(kc[..., h:h + 1, :], sc[1])
        vh = to_f64(vc[..., h:h + 1, :], sc[2])
        ro, _ = oracle.attend(zq, kh, vh, wl.grid, wl.window, wl.stride, 1.0, queries=qs)
        go = o_all[:, :, h].numpy() if qs is None else o_all[:, qs, h].numpy()
        ref = ro[:, :, 0]
        # unit weights: out = round(fp32 sum / count); half an ulp of the
        # output type plus the fp32 accumulation (<= W * 2^-24 * the largest
        # partial sum, divided by W)
        ulp = 2.0 ** -23 if wl.dtype == "f32" else 2.0 ** -8
        err = np.abs(go - ref) - ulp * np.abs(ref)
        worst = max(worst, float(err.max()))
    say(f"  window mean: max(|out - mean| - ulp*|mean|) = {worst:.3e}")
    assert worst <= 1e-4


def test_dense_reference_full_size_sampled(na, path):
    # window = grid at the video workload's full size, the dense run the
    # benchmark reports as the speed-up reference
    import gpu_util
    if path == "tiled":
        pytest.skip("the tiled form is bit-identical to the others (three-forms test)")
    wl = WORKLOADS["video_dense"]
    say(f"[parity] video_dense full size ({path})")
    qc, kc, vc, sc = make_qkv(wl, device="cpu")
    f = na.Forward(qc.cuda(), kc.cuda(), vc.cuda(), wl.window, wl.stride, scale=wl.scale,
                   workspace=gpu_util.USE_WORKSPACE)
    out, lse = f()
    torch.cuda.synchronize()
    qs = _sample(wl, 16, wl.seed + 5)
    o_all = out.detach().cpu().double().reshape(1, wl.tokens, wl.heads, wl.head_dim)
    l_all = lse.detach().cpu().double().reshape(1, wl.tokens, wl.heads)
    eo = el = 0.0
    for h in (0, 19):
        ro, rl = oracle.attend(to_f64(qc[..., h:h + 1, :]), to_f64(kc[..., h:h + 1, :]), to_f64(vc[..., h:h + 1, :]),
                               wl.grid, wl.window, wl.stride, wl.scale, queries=qs)
        eo = max(eo, float(np.abs(o_all[:, qs, h].numpy() - ro[:, :, 0]).max()))
        el = max(el, float(np.abs(l_all[:, qs, h].numpy() - rl[:, :, 0]).max()))
    say(f"  {len(qs)} queries x 2 heads: max|out-oracle|={eo:.3e} max|lse-oracle|={el:.3e}")
    to, tl = TOL["bf16"]
    assert eo <= to and el <= tl
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
