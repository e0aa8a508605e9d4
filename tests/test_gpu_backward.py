"""GPU parity of the backward pass (na_backward) against the float64 oracle's
gradients, on seeded bf16 inputs."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import say
from synth import WORKLOADS, make_qkv, sample_queries

pytestmark = pytest.mark.gpu

# Max-abs error over max |reference| per gradient tensor.  The kernel rounds
# P and dS to bf16 before the matrix products (8 significant bits: relative
# error up to 2^-8 each), uses the bf16 forward output in D_i = <dout_i,
# out_i>, and rounds dq, dk, dv to bf16; sums over thousands of such terms
# keep the error at a few 2^-8 of the largest entries.  1.5e-2 leaves room
# over the measured ~4e-3.
REL_TOL = 1.5e-2


def _dout(wl, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn((wl.batch, *wl.grid, wl.heads, wl.head_dim), generator=g).to(torch.bfloat16)


def _run(na, wl, q, k, v, do):
    out, lse = na.forward(q, k, v, wl.window, wl.stride, scale=wl.scale)
    dq, dk, dv = na.backward(q, k, v, out, lse, do, wl.window, wl.stride, scale=wl.scale)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def _rel_err(gpu, ref):
    g = gpu.detach().to("cpu").to(torch.float64).numpy()
    return float(np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30))


SMALL = [
    ("img64_sliding", {}),                                                   # 2-D, mostly boundary tiles
    ("video_sliding", dict(batch=2, heads=2, grid=(5, 19, 27), window=(3, 7, 9), stride=(1, 2, 3))),
    ("video_sliding", dict(batch=1, heads=2, grid=(5, 19, 27), window=(3, 7, 9), stride=(1, 2, 3), head_dim=64)),
    ("video_block", dict(heads=2, grid=(8, 16, 24), window=(6, 8, 8), stride=(4, 4, 4))),
    ("img64_sliding", dict(batch=1, heads=2, grid=(1, 1, 1000), window=(1, 1, 65), stride=(1, 1, 1))),  # 1-D
    ("img64_block", dict(batch=1, heads=2, grid=(1, 1, 1000), window=(1, 1, 64), stride=(1, 1, 32))),
    ("img64_sliding", dict(batch=1, heads=2, grid=(1, 24, 40), window=(1, 9, 17), stride=(1, 1, 8),
                           head_dim=128)),                                   # anisotropic window / stride
]


@pytest.fixture(params=["split", "fused"])
def dkdv(request, monkeypatch):
    """The two dk/dv kernels: one wave per gradient and 32 keys (default), or
    one wave for both (NA_DKDV_SPLIT=0)."""
    if request.param == "fused":
        monkeypatch.setenv("NA_DKDV_SPLIT", "0")
    return request.param


@pytest.mark.parametrize("name,kw", SMALL)
def test_backward_small_all_rows(na, name, kw, dkdv):
    wl = WORKLOADS[name].with_(seed=900 + len(kw), **kw)
    say(f"[bwd] {wl.name} ({dkdv}) grid={wl.grid} w={wl.window} s={wl.stride} D={wl.head_dim} B={wl.batch} "
        f"H={wl.heads}")
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    do = _dout(wl, wl.seed + 5)
    _, _, dq, dk, dv = _run(na, wl, qc.cuda(), kc.cuda(), vc.cuda(), do.cuda())
    f64 = lambda x: x.to(torch.float64).numpy()
    rq, rk, rv = oracle.attend_backward(f64(qc), f64(kc), f64(vc), f64(do), wl.grid, wl.window, wl.stride, wl.scale)
    shape = (wl.batch, math.prod(wl.grid), wl.heads, wl.head_dim)
    eq, ek, ev = (_rel_err(g.reshape(shape), r) for g, r in ((dq, rq), (dk, rk), (dv, rv)))
    say(f"  rel err dq={eq:.2e} dk={ek:.2e} dv={ev:.2e}")
    assert eq <= REL_TOL and ek <= REL_TOL and ev <= REL_TOL


def test_backward_full_size_video(na):
    wl = WORKLOADS["video_block"]
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    do = _dout(wl, 4711)
    say("[bwd] video block full size")
    _, _, dq, dk, dv = _run(na, wl, qc.cuda(), kc.cuda(), vc.cuda(), do.cuda())
    # exact identities over every row: sum_j dk_j = 0 and sum_j dv_j = sum_i dout_i
    sk = dk.to(torch.float64).sum(dim=(1, 2, 3))
    sv = dv.to(torch.float64).sum(dim=(1, 2, 3)) - do.cuda().to(torch.float64).sum(dim=(1, 2, 3))
    ak = dk.to(torch.float64).abs().sum(dim=(1, 2, 3))
    av = dv.to(torch.float64).abs().sum(dim=(1, 2, 3))
    say(f"  |sum dk| / sum |dk| = {float((sk.abs() / ak).max()):.2e}, same for dv - dout: {float((sv.abs() / av).max()):.2e}")
    assert float((sk.abs() / ak).max()) < 1e-3 and float((sv.abs() / av).max()) < 1e-3
    # sampled rows against the oracle, head 5
    h = 5
    f64 = lambda x: x[..., h:h + 1, :].to(torch.float64).numpy()
    tq, _ = na.na_choose_tiles(wl.grid, wl.window, wl.stride, wl.head_dim, na.NA_BF16)
    qs = sample_queries(wl, tq, n_random=64)[::8]
    ks = np.array([0, wl.tokens // 2 + 37, wl.tokens - 1, 48 * 80 * 13 + 80 * 20 + 41])
    rq, rk, rv = oracle.attend_backward(f64(qc), f64(kc), f64(vc), f64(do), wl.grid, wl.window, wl.stride, wl.scale,
                                        queries=qs, keys=ks)
    N = wl.tokens
    g = lambda x, rows: x.reshape(1, N, wl.heads, wl.head_dim)[:, rows, h:h + 1, :]
    eq, ek, ev = _rel_err(g(dq, qs), rq), _rel_err(g(dk, ks), rk), _rel_err(g(dv, ks), rv)
    say(f"  {len(qs)} queries, {len(ks)} keys: rel err dq={eq:.2e} dk={ek:.2e} dv={ev:.2e}")
    assert eq <= REL_TOL and ek <= REL_TOL and ev <= REL_TOL


def test_backward_window_one(na):
    # out = v: dv = dout exactly, dq and dk vanish up to fp32 rounding of dS
    wl = WORKLOADS["video_block"].with_(grid=(3, 10, 16), window=(1, 1, 1), stride=(1, 1, 1), heads=2, seed=77)
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    do = _dout(wl, 78)
    _, _, dq, dk, dv = _run(na, wl, qc.cuda(), kc.cuda(), vc.cuda(), do.cuda())
    assert torch.equal(dv.cpu(), do)
    assert float(dq.abs().max()) < 1e-4 and float(dk.abs().max()) < 1e-4


def test_backward_is_deterministic(na):
    wl = WORKLOADS["video_sliding"].with_(batch=1, heads=2, grid=(5, 19, 27), window=(3, 7, 9), stride=(1, 2, 3),
                                          seed=79)
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    do = _dout(wl, 80).cuda()
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    a = _run(na, wl, q, k, v, do)
    b = _run(na, wl, q, k, v, do)
    for x, y in zip(a[2:], b[2:]):
        assert torch.equal(x, y)


def test_backward_empty_batch(na):
    e = torch.empty((0, 1, 16, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((0, 1, 16, 16, 2), dtype=torch.float32, device="cuda")
    dq, dk, dv = na.backward(e, e, e, e, lse, e, (1, 5, 5), (1, 1, 1))
    assert dq.shape == e.shape


def test_dkdv_split_equals_fused_full_size(na, monkeypatch):
    # the split kernel's dK and dV waves run the fused wave's arithmetic in the
    # same order, so dk and dv agree bit for bit (here at full video size)
    wl = WORKLOADS["video_block"]
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    do = _dout(wl, 4712).cuda()
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    say("[bwd] dk/dv split vs fused, video block full size")
    a = _run(na, wl, q, k, v, do)
    monkeypatch.setenv("NA_DKDV_SPLIT", "0")
    b = _run(na, wl, q, k, v, do)
    for x, y in zip(a[2:], b[2:]):
        assert torch.equal(x, y)


def test_backward_replays_in_a_hip_graph(na):
    # na_backward enqueues kernels only once the plan (and its transposed map)
    # exists, so it can be captured; every replay equals the eager gradients
    wl = WORKLOADS["video_sliding"].with_(batch=1, heads=2, grid=(5, 19, 27), window=(3, 7, 9), stride=(1, 2, 3),
                                          seed=81)
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    do = _dout(wl, 82).cuda()
    out, lse, dq_e, dk_e, dv_e = _run(na, wl, q, k, v, do)
    B, H, D = wl.batch, wl.heads, wl.head_dim
    nb = na.na_backward_workspace_bytes(B, H, D, wl.grid, wl.window, wl.stride, na.NA_BF16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    grads = [torch.empty_like(q) for _ in range(3)]
    say("[bwd] graph replay")

    def call():
        na.na_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), do.data_ptr(), lse.data_ptr(),
                       grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(), B, H, D, wl.grid, wl.window,
                       wl.stride, wl.scale, na.NA_BF16, ws.data_ptr(), nb,
                       torch.cuda.current_stream().cuda_stream)

    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        for t in grads:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(grads, (dq_e, dk_e, dv_e)):
            assert torch.equal(t, e)


def _random_bwd_cases():
    from test_gpu_random import _geometry
    out = []
    for i in range(16):
        rng = np.random.default_rng(8000 + i)
        grid, window, stride = _geometry(rng)
        D = int(rng.choice([64, 128]))
        batch, heads = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        out.append((f"b{i}", grid, window, stride, D, batch, heads))
    return out


RANDOM_BWD = _random_bwd_cases()


@pytest.mark.parametrize("name,grid,window,stride,D,batch,heads", RANDOM_BWD, ids=[c[0] for c in RANDOM_BWD])
def test_backward_random_geometries(na, dkdv, name, grid, window, stride, D, batch, heads):
    # seeded random 1-/2-/3-D geometries (ragged extents, 1 <= s <= w <= L),
    # every row of every gradient against the oracle
    wl = WORKLOADS["img64_sliding"].with_(name=name, batch=batch, heads=heads, grid=grid, window=window,
                                          stride=stride, head_dim=D, seed=8100 + int(name[1:]))
    say(f"[bwd] random {name} ({dkdv}) grid={grid} w={window} s={stride} D={D} B={batch} H={heads}")
    qc, kc, vc, _ = make_qkv(wl, device="cpu")
    do = _dout(wl, wl.seed + 5)
    _, _, dq, dk, dv = _run(na, wl, qc.cuda(), kc.cuda(), vc.cuda(), do.cuda())
    f64 = lambda x: x.to(torch.float64).numpy()
    rq, rk, rv = oracle.attend_backward(f64(qc), f64(kc), f64(vc), f64(do), grid, window, stride, wl.scale)
    shape = (batch, math.prod(grid), heads, D)
    eq, ek, ev = (_rel_err(g.reshape(shape), r) for g, r in ((dq, rq), (dk, rk), (dv, rv)))
    say(f"  rel err dq={eq:.2e} dk={ek:.2e} dv={ev:.2e}")
    assert eq <= REL_TOL and ek <= REL_TOL and ev <= REL_TOL
