"""GPU: na_forward_noalloc (the forward whose tile map lives in a fixed
device buffer, for callers that cannot allocate) against na_forward's form 2
(no workspace), which runs the same kernel on a cached map.  Calls in a row
on different geometries -- the second one smaller, then the first again --
share the one buffer; each must equal na_forward bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, say
from synth import WORKLOADS, make_qkv, to_f64

pytestmark = pytest.mark.gpu


def _noalloc(na, wl, q, k, v, out, lse):
    na.na_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), wl.batch,
                          wl.heads, wl.head_dim, wl.grid, wl.window, wl.stride, wl.scale, na.NA_BF16,
                          torch.cuda.current_stream().cuda_stream)


CASES = [
    WORKLOADS["video_block"].with_(name="noalloc_big", heads=3, grid=(20, 24, 40), seed=811),
    WORKLOADS["video_sliding"].with_(name="noalloc_small", batch=2, heads=2, grid=(5, 19, 27), window=(3, 7, 9),
                                     stride=(1, 2, 3), head_dim=64, seed=812),
]


def test_noalloc_matches_forward_on_calls_in_a_row(na):
    inputs = []
    for wl in CASES:
        qc, kc, vc, _ = make_qkv(wl, device="cpu")
        q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
        ref_out, ref_lse = na.forward(q, k, v, wl.window, wl.stride, scale=wl.scale, workspace=False)
        torch.cuda.synchronize()
        inputs.append((wl, qc, kc, vc, q, k, v, ref_out.clone(), ref_lse.clone()))
    for i in (0, 1, 0):   # the second call is smaller; then the first geometry again
        wl, qc, kc, vc, q, k, v, ref_out, ref_lse = inputs[i]
        say(f"[noalloc] {wl.name} grid={wl.grid} w={wl.window} s={wl.stride} D={wl.head_dim}")
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=q.device)
        _noalloc(na, wl, q, k, v, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        # and within the workload tolerance of the oracle on a few queries
        qs = np.random.default_rng(wl.seed).integers(0, wl.tokens, 48)
        ro, rl = oracle.attend(to_f64(qc[..., :1, :]), to_f64(kc[..., :1, :]), to_f64(vc[..., :1, :]), wl.grid,
                               wl.window, wl.stride, wl.scale, queries=qs)
        go = out.cpu().double().reshape(wl.batch, wl.tokens, wl.heads, wl.head_dim)[:, qs, 0].numpy()
        gl = lse.cpu().double().reshape(wl.batch, wl.tokens, wl.heads)[:, qs, 0].numpy()
        eo, el = float(np.abs(go - ro[:, :, 0]).max()), float(np.abs(gl - rl[:, :, 0]).max())
        say(f"  bit-identical to na_forward; max|out-oracle|={eo:.3e} max|lse-oracle|={el:.3e}")
        assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]


def test_noalloc_random_geometries_in_a_row(na):
    # seeded random 1-/2-/3-D geometries, one call after another on the one
    # buffer (large and small maps alternating): each bit for bit equal to
    # na_forward's form 2
    from test_gpu_random import _geometry
    for i in range(12):
        rng = np.random.default_rng(9500 + i)
        grid, window, stride = _geometry(rng)
        D = int(rng.choice([64, 128]))
        wl = WORKLOADS["img64_sliding"].with_(name=f"na{i}", batch=int(rng.integers(1, 3)),
                                              heads=int(rng.integers(1, 4)), grid=grid, window=window,
                                              stride=stride, head_dim=D, seed=9600 + i)
        say(f"[noalloc] random {wl.name} grid={grid} w={window} s={stride} D={D} B={wl.batch} H={wl.heads}")
        qc, kc, vc, _ = make_qkv(wl, device="cpu")
        q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
        ref_out, ref_lse = na.forward(q, k, v, window, stride, scale=wl.scale, workspace=False)
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=q.device)
        _noalloc(na, wl, q, k, v, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_noalloc_replays_in_hip_graphs(na):
    # the callers it is for include code under graph capture: after a first
    # eager call per geometry, each call is a host-to-device copy of the tile
    # map into the fixed buffer plus the kernel, both captured.  Two graphs of
    # different geometries replayed alternately (each rewrites the shared
    # buffer before its kernel), outputs poisoned by eager work in between:
    # every replay equals the eager result bit for bit.
    wls = [WORKLOADS["video_block"].with_(name="g1", grid=(8, 16, 24), window=(6, 8, 8), stride=(4, 4, 4), heads=2,
                                          seed=311),
           WORKLOADS["video_sliding"].with_(name="g2", batch=1, heads=2, grid=(5, 19, 27), window=(3, 7, 9),
                                            stride=(1, 2, 3), head_dim=64, seed=312)]
    st = []
    for wl in wls:
        qc, kc, vc, _ = make_qkv(wl, device="cpu")
        q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
        _noalloc(na, wl, q, k, v, out, lse)
        torch.cuda.synchronize()
        st.append((wl, q, k, v, out, lse, out.clone(), lse.clone()))
    graphs = []
    for wl, q, k, v, out, lse, _, _ in st:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            _noalloc(na, wl, q, k, v, out, lse)
        graphs.append(g)
    for rep in range(3):
        for g, (wl, q, k, v, out, lse, out_e, lse_e) in zip(graphs, st):
            say(f"[noalloc] graph replay {rep} {wl.name}")
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, out_e) and torch.equal(lse, lse_e)
