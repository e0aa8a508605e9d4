"""GPU tests of the permutation kernels and of the method's special cases:
window 1, zero queries, window = grid, stride = window, translation
equivariance, masking forced on full tiles, poisoned outputs, empty batch."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, compare, inputs, run_hip, say, set_path
from synth import WORKLOADS, make_qkv, to_f64

pytestmark = pytest.mark.gpu


def _ref_tile_order(x, tile, transpose):
    """numpy reference of the tile layout: pad, split each axis into
    (tiles, in-tile), move heads out and the in-tile axes inward."""
    B, T, H, W, h, D = x.shape
    tT, tH, tW = tile
    nT, nH, nW = -(-T // tT), -(-H // tH), -(-W // tW)
    p = np.zeros((B, nT * tT, nH * tH, nW * tW, h, D), dtype=x.dtype)
    p[:, :T, :H, :W] = x
    p = p.reshape(B, nT, tT, nH, tH, nW, tW, h, D).transpose(0, 7, 1, 3, 5, 2, 4, 6, 8)
    p = p.reshape(B, h, nT * nH * nW, tT * tH * tW, D)
    return p.transpose(0, 1, 2, 4, 3).copy() if transpose else p


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float8_e4m3fn])
@pytest.mark.parametrize("tile", [(2, 8, 8), (1, 4, 16), (4, 2, 2)])
@pytest.mark.parametrize("transpose", [False, True])
@pytest.mark.parametrize("heads", [3, 11])   # 11: head groups of 8, the last one partial
def test_permute_layout_and_round_trip(na, dtype, tile, transpose, heads):
    if transpose and dtype == torch.float32:
        pytest.skip("fp32 path keeps V untransposed")
    D = 64 if dtype != torch.float8_e4m3fn else 128
    say(f"[permute] {dtype} tile={tile} transpose={transpose} heads={heads}")
    g = torch.Generator("cpu").manual_seed(5)
    x = torch.randn((2, 5, 11, 13, heads, D), generator=g).to(dtype)
    xg = x.cuda()
    xt = na.permute(xg, tile, transpose=transpose)
    torch.cuda.synchronize()
    ib = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.float8_e4m3fn: torch.uint8}[dtype]
    ref = _ref_tile_order(x.view(ib).numpy(), tile, transpose)
    assert np.array_equal(xt.cpu().view(ib).numpy(), ref)
    if not transpose:
        back = na.unpermute(xt, (5, 11, 13), tile)
        torch.cuda.synchronize()
        assert torch.equal(back.cpu().view(ib), x.view(ib))


def _run(na, wl, q, k, v, window=None, stride=None):
    import gpu_util
    ws = gpu_util.USE_WORKSPACE or q.dtype != torch.bfloat16 or q.shape[-1] not in (64, 128)
    f = na.Forward(q, k, v, window or wl.window, stride or wl.stride, scale=wl.scale, workspace=ws)
    out, lse = f()
    torch.cuda.synchronize()
    return out, lse


@pytest.fixture(params=["qo", "grid", "tiled"])
def path(request, monkeypatch):
    """The three forms of the bf16 forward (see gpu_util.set_path)."""
    set_path(monkeypatch, request.param)
    return request.param


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_one_returns_v_exactly(na, dtype, path):
    wl = WORKLOADS["img64_block"].with_(grid=(3, 17, 20), window=(1, 1, 1), stride=(1, 1, 1), dtype=dtype,
                                        head_dim=64, heads=2, seed=91)
    say(f"[special] window 1 {dtype}")
    qc, kc, vc, sc, q, k, v = inputs(wl)
    out, lse = _run(na, wl, q, k, v)
    assert torch.equal(out.cpu(), vc)
    ref = wl.scale * (qc.double() * kc.double()).sum(-1)
    assert float((lse.cpu().double() - ref).abs().max()) <= TOL[dtype][1]


def test_zero_queries_give_window_mean(na, path):
    wl = WORKLOADS["img64_block"].with_(grid=(2, 21, 18), window=(2, 6, 5), stride=(1, 3, 2), heads=2, seed=92)
    say("[special] q = 0")
    qc, kc, vc, sc, q, k, v = inputs(wl)
    qc = torch.zeros_like(qc)
    out, lse = _run(na, wl, qc.cuda(), k, v)
    eo, el = compare(wl, qc, kc, vc, sc, out, lse)
    assert eo <= TOL["bf16"][0]
    assert float((lse.cpu().double() - math.log(math.prod(wl.window))).abs().max()) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_zero_scale_gives_window_mean(na, dtype, path):
    # scale 0: every weight is 1, so out is the window mean of v and
    # lse = ln prod(w) exactly as for q = 0; boundary tiles (masked keys)
    # must not turn 0 * -inf into NaN
    base = WORKLOADS["img64_block"] if dtype == "bf16" else WORKLOADS["img256_block_fp8"]
    wl = base.with_(grid=(2, 21, 18), window=(2, 6, 5), stride=(1, 3, 2), heads=2, seed=95, head_dim=128)
    say(f"[special] scale = 0 ({dtype})")
    qc, kc, vc, sc, q, k, v = inputs(wl)
    f = na.Forward(q, k, v, wl.window, wl.stride, scale=0.0, qkv_scale=sc if dtype == "fp8" else None)
    out, lse = f()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    assert float((lse.cpu().double() - math.log(math.prod(wl.window))).abs().max()) <= 1e-5
    zq = torch.zeros_like(qc)   # the oracle with q = 0 gives the same uniform weights
    eo, _ = compare(wl, zq, kc, vc, sc, out, lse)
    assert eo <= TOL[dtype][0]


@pytest.mark.parametrize("stride", [(1, 1, 1), (2, 3, 4)])
def test_window_equal_grid_is_dense(na, stride, path):
    wl = WORKLOADS["img64_block"].with_(grid=(2, 12, 16), window=(2, 12, 16), stride=stride, heads=2,
                                        head_dim=128, seed=93)
    say(f"[special] window = grid, stride {stride}")
    qc, kc, vc, sc, q, k, v = inputs(wl)
    out, lse = _run(na, wl, q, k, v)
    eo, el = compare(wl, qc, kc, vc, sc, out, lse)
    say(f"  {eo:.3e} {el:.3e}")
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]


def test_stride_equal_window_is_block_diagonal(na, path):
    wl = WORKLOADS["img64_block"].with_(grid=(4, 24, 32), window=(2, 8, 8), stride=(2, 8, 8), heads=2,
                                        head_dim=128, seed=94)
    say("[special] stride = window")
    qc, kc, vc, sc, q, k, v = inputs(wl)
    out, lse = _run(na, wl, q, k, v)
    eo, el = compare(wl, qc, kc, vc, sc, out, lse)
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]


def test_translation_equivariance_sliding(na):
    # the same tokens seen through two grids shifted by d along W: interior
    # queries (windows unclamped in both) must agree
    H, W, w, d = 24, 40, 7, 5
    g = torch.Generator("cpu").manual_seed(95)
    X = [torch.randn((1, 1, H, W, 2, 64), generator=g).to(torch.bfloat16) for _ in range(3)]
    A = [x[:, :, :, : W - d].contiguous().cuda() for x in X]
    B = [x[:, :, :, d:].contiguous().cuda() for x in X]
    say("[special] translation equivariance")
    oa, _ = na.forward(*A, (1, w, w), (1, 1, 1), scale=0.125)
    ob, _ = na.forward(*B, (1, w, w), (1, 1, 1), scale=0.125)
    torch.cuda.synchronize()
    half = w // 2
    ia = oa[0, 0, half:H - half, half + d:W - d - half].float()
    ib = ob[0, 0, half:H - half, half:W - 2 * d - half].float()
    assert ia.numel() > 0
    assert float((ia - ib).abs().max()) <= 2 * TOL["bf16"][0]


def test_forced_mask_on_full_tiles_is_bit_identical(na, monkeypatch, path):
    # GNA page section 2.1: the mask is only needed on boundary tiles; applying
    # it to full tiles too must not change a single bit
    wl = WORKLOADS["video_block"].with_(grid=(20, 24, 32), heads=2, seed=96)
    say("[special] forced mask")
    qc, kc, vc, sc, q, k, v = inputs(wl)
    out1, lse1 = _run(na, wl, q, k, v)
    monkeypatch.setenv("NA_FORCE_MASK", "1")
    out2, lse2 = _run(na, wl, q, k, v)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_every_output_written(na, path):
    wl = WORKLOADS["video_sliding"].with_(grid=(3, 13, 21), window=(3, 5, 7), heads=3, seed=97)
    say("[special] poisoned outputs")
    qc, kc, vc, sc, q, k, v = inputs(wl)
    import gpu_util
    f = na.Forward(q, k, v, wl.window, wl.stride, scale=wl.scale, workspace=gpu_util.USE_WORKSPACE)
    f.out.fill_(float("nan"))
    f.lse.fill_(float("nan"))
    if f.workspace is not None:
        f.workspace.fill_(0xFF)   # NaN patterns in every tile-order buffer
    out, lse = f()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    eo, el = compare(wl, qc, kc, vc, sc, out, lse)
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]


def test_no_lse_and_empty_batch(na, path):
    wl = WORKLOADS["img64_sliding"].with_(heads=2, seed=98)
    qc, kc, vc, sc, q, k, v = inputs(wl)
    say("[special] lse = NULL, empty batch")
    import gpu_util
    ws = gpu_util.USE_WORKSPACE
    f = na.Forward(q, k, v, wl.window, wl.stride, scale=wl.scale, return_lse=False, workspace=ws)
    out, lse = f()
    torch.cuda.synchronize()
    assert lse is None
    f2 = na.Forward(q, k, v, wl.window, wl.stride, scale=wl.scale, workspace=ws)
    out2, _ = f2()
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    e = torch.empty((0, 1, 64, 64, 2, 64), dtype=torch.bfloat16, device="cuda")
    o, l = na.forward(e, e, e, (1, 17, 17), (1, 1, 1), workspace=ws)
    assert o.shape == e.shape and l.shape == e.shape[:-1]


def test_fp8_window_one_returns_scaled_v_exactly(na):
    # window 1: P = e4m3(64) exactly, l = 64, out = bf16(v8 * v_scale)
    wl = WORKLOADS["img256_block_fp8"].with_(grid=(2, 13, 24), window=(1, 1, 1), stride=(1, 1, 1), heads=2, seed=99)
    say("[special] fp8 window 1")
    qc, kc, vc, sc, q, k, v = inputs(wl)
    f = na.Forward(q, k, v, wl.window, wl.stride, scale=wl.scale, qkv_scale=sc)
    out, lse = f()
    torch.cuda.synchronize()
    ref = (vc.float() * sc[2]).to(torch.bfloat16)
    assert torch.equal(out.cpu(), ref)
    lref = wl.scale * sc[0] * sc[1] * (qc.double() * kc.double()).sum(-1)
    assert float((lse.cpu().double() - lref).abs().max()) <= TOL["fp8"][1]


@pytest.mark.parametrize("grid", [(20, 24, 40), (5, 19, 27)])
def test_three_forward_forms_agree(na, monkeypatch, grid):
    # the three forms feed the same tiles to the same arithmetic in the same
    # order: results are bit-identical (ragged grid: padding handled alike)
    wl = WORKLOADS["video_block"].with_(grid=grid, window=(3, 7, 9) if grid[0] == 5 else (18, 24, 24),
                                        stride=(1, 2, 3) if grid[0] == 5 else (16, 8, 8), heads=2, seed=100)
    say(f"[special] three forms agree grid={grid}")
    qc, kc, vc, sc, q, k, v = inputs(wl)
    res = {}
    for form in ("qo", "grid", "tiled"):
        with monkeypatch.context() as m:
            set_path(m, form)
            res[form] = _run(na, wl, q, k, v)
    for form in ("grid", "tiled"):
        assert torch.equal(res["qo"][0], res[form][0]) and torch.equal(res["qo"][1], res[form][1]), form


def test_offsets_beyond_32_bits_match_the_small_problem(na, path):
    # The video workload with every (batch, head) repeated: batch 2 x 168
    # heads puts element offsets of q, k, v, out and of the tile-order copies
    # above 2^32.  Each (b, h) is computed independently in one fixed order, so
    # every copy must equal the 24-head original bit for bit (the original is
    # the problem the full-size parity test checks against the oracle).
    import gpu_util
    wl = WORKLOADS["video_block"]
    say(f"[special] 2 x 168 heads of the video workload ({path})")
    _, _, _, _, q, k, v = inputs(wl)
    ws = gpu_util.USE_WORKSPACE
    f = na.Forward(q, k, v, wl.window, wl.stride, scale=wl.scale, workspace=ws)
    out, lse = f()
    torch.cuda.synchronize()
    out, lse = out.clone(), lse.clone()
    del f
    rep = (2, 1, 1, 1, 7, 1)
    qb, kb, vb = q.repeat(*rep), k.repeat(*rep), v.repeat(*rep)
    assert qb.numel() > 2 ** 32
    fb = na.Forward(qb, kb, vb, wl.window, wl.stride, scale=wl.scale, workspace=ws)
    ob, lb = fb()
    torch.cuda.synchronize()
    for b, h in [(1, 167), (1, 150), (0, 161), (1, 0), (0, 71)]:
        assert torch.equal(ob[b, ..., h, :], out[0, ..., h % wl.heads, :]), (b, h)
        assert torch.equal(lb[b, ..., h], lse[0, ..., h % wl.heads]), (b, h)
    del fb, qb, kb, vb, ob, lb
    torch.cuda.empty_cache()


def test_forward_replays_in_a_hip_graph(na, path):
    # After a first call has built the plan, na_forward only enqueues kernels,
    # so it can be captured in a HIP graph.  Each replay must equal the eager
    # result bit for bit; the outputs are poisoned by eager work in between.
    import gpu_util
    wl = WORKLOADS["video_block"].with_(grid=(8, 16, 24), window=(6, 8, 8), stride=(4, 4, 4), heads=2, seed=311)
    say(f"[special] graph replay ({path})")
    _, _, _, _, q, k, v = inputs(wl)
    f = na.Forward(q, k, v, wl.window, wl.stride, scale=wl.scale, workspace=gpu_util.USE_WORKSPACE)
    out_e, lse_e = f()
    torch.cuda.synchronize()
    out_e, lse_e = out_e.clone(), lse_e.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f()
    for _ in range(3):
        f.out.fill_(float("nan"))
        f.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(f.out, out_e) and torch.equal(f.lse, lse_e)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_rising_scores_rescale_every_block(na, path, dtype):
    # Scores that grow block by block along the key sequence (a 1-D grid,
    # window = grid): each 32-key block's scores sit 16 (in log2 units) above
    # the previous block's, far more than the lazy-rescale threshold, so the
    # rescale branch runs on every block; inside a block they are nearly
    # flat, so the softmax spreads over the last block's keys.  out and lse
    # must still match the oracle.
    from synth import quantize_e4m3
    if dtype == "fp8" and path != "qo":
        pytest.skip("fp8 runs form 1 only")
    D = 64 if dtype == "bf16" else 128
    wl = WORKLOADS["img64_sliding" if dtype == "bf16" else "img256_block_fp8"].with_(
        name="rising", batch=1, heads=2, grid=(1, 1, 2048), window=(1, 1, 2048), stride=(1, 1, 1), head_dim=D,
        seed=4242)
    say(f"[special] rising scores {dtype} ({path})")
    n = 2048
    g = torch.Generator("cpu").manual_seed(wl.seed)
    # q . k_j * scale * log2(e) = 16 * (j // 32) plus a little noise
    step = 16.0 / math.log2(math.e) / (wl.scale * D)
    q = torch.ones((1, 1, 1, n, 2, D))
    lev = (torch.arange(n) // 32).to(torch.float32) * step
    k = lev.reshape(1, 1, 1, n, 1, 1).expand(1, 1, 1, n, 2, D).clone()
    k = k + 0.01 * torch.randn(k.shape, generator=g)
    v = torch.randn((1, 1, 1, n, 2, D), generator=g)
    if dtype == "bf16":
        qc, kc, vc = (x.to(torch.bfloat16) for x in (q, k, v))
        sc = (1.0, 1.0, 1.0)
    else:
        (qc, s0), (kc, s1), (vc, s2) = (quantize_e4m3(x) for x in (q, k, v))
        sc = (s0, s1, s2)
    out, lse, _ = run_hip(na, wl, qc.cuda(), kc.cuda(), vc.cuda(), sc)
    eo, el = compare(wl, qc, kc, vc, sc, out, lse)
    say(f"  max|out-oracle|={eo:.3e} max|lse-oracle|={el:.3e}")
    to, tl = TOL[dtype]
    assert eo <= to and el <= tl


@pytest.mark.parametrize("name", ["video_block", "img256_block_fp8"])
def test_full_size_forward_is_deterministic(na, path, name):
    # The kernels use no atomics and a fixed visiting order, so repeated calls
    # on the full workload must agree bit for bit; a race on the LDS double
    # buffer or the tile-map reads would show up as a difference.  Outputs
    # are poisoned between the calls.
    import gpu_util
    wl = WORKLOADS[name]
    if wl.dtype == "fp8" and path != "qo":
        pytest.skip("fp8 runs form 1 only")
    say(f"[special] determinism {name} ({path})")
    qc, kc, vc, sc, q, k, v = inputs(wl)
    f = na.Forward(q, k, v, wl.window, wl.stride, scale=wl.scale,
                   qkv_scale=sc if wl.dtype == "fp8" else None,
                   workspace=gpu_util.USE_WORKSPACE or wl.dtype != "bf16")
    out0, lse0 = f()
    torch.cuda.synchronize()
    out0, lse0 = out0.clone(), lse0.clone()
    for _ in range(3):
        f.out.fill_(float("nan"))
        f.lse.fill_(float("nan"))
        f()
        torch.cuda.synchronize()
        assert torch.equal(f.out, out0) and torch.equal(f.lse, lse0)
    del f, q, k, v, out0, lse0
    torch.cuda.empty_cache()


@pytest.mark.parametrize("grid", [(1, 1, 1), (1, 1, 5), (1, 3, 1), (2, 1, 1), (3, 2, 1), (1, 1, 9)])
@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8"])
def test_tiny_grids(na, path, grid, dtype):
    # grids of one to nine tokens: tiles mostly padding, every query sees
    # every token (window = grid).  bf16 and fp32 are held to the workload
    # tolerances.  fp8 stores each weight as e4m3(64 p), 4 significant bits
    # (relative error up to 2^-4 per weight); a window of a few keys does not
    # average that out, so windows below FP8_FEW_KEYS keys are held to the
    # bound it implies instead: the normalised weights move by at most
    # 2u / (1 - u) in total, out by that times max |v| (u = 2^-4)
    if path != "qo" and dtype != "bf16":
        pytest.skip("the other forms are bf16 only")
    base = {"bf16": WORKLOADS["img64_block"], "f32": WORKLOADS["img16_f32"], "fp8": WORKLOADS["img256_block_fp8"]}[dtype]
    wl = base.with_(batch=2, heads=3, grid=grid, window=grid, stride=(1, 1, 1), seed=400 + sum(grid))
    qc, kc, vc, sc, q, k, v = inputs(wl)
    out, lse, _ = run_hip(na, wl, q, k, v, sc)
    eo, el = compare(wl, qc, kc, vc, sc, out, lse)
    to, tl = TOL[wl.dtype]
    if dtype == "fp8" and math.prod(grid) < FP8_FEW_KEYS:
        u = 2.0 ** -4
        to = max(to, 2 * u / (1 - u) * float(vc.float().abs().max()) * sc[2])
    say(f"[special] tiny grid {grid} {dtype} ({path}): max|out-oracle|={eo:.3e} (bound {to:.3e}) "
        f"max|lse-oracle|={el:.3e} (bound {tl:.3e})")
    assert eo <= to and el <= tl


# windows with fewer keys than this are the few-key fp8 cases above
FP8_FEW_KEYS = 16


@pytest.mark.parametrize("w", [2, 3, 4, 6, 9, 12, 16, 24, 32, 64, 128])
def test_fp8_error_against_window_size(na, w):
    # 1-D sequence, sliding window of w keys: the e4m3 weights' rounding
    # averages out as the window grows.  From FP8_FEW_KEYS keys on, out must
    # meet the fp8 workload tolerance; below, the few-key bound.
    wl = WORKLOADS["img256_block_fp8"].with_(name="fp8w", batch=1, heads=4, grid=(1, 1, 1024), window=(1, 1, w),
                                             stride=(1, 1, 1), seed=5000 + w)
    qc, kc, vc, sc, q, k, v = inputs(wl)
    out, lse, _ = run_hip(na, wl, q, k, v, sc)
    eo, el = compare(wl, qc, kc, vc, sc, out, lse)
    to, tl = TOL["fp8"]
    if w < FP8_FEW_KEYS:
        u = 2.0 ** -4
        to = max(to, 2 * u / (1 - u) * float(vc.float().abs().max()) * sc[2])
    say(f"[special] fp8 window {w}: max|out-oracle|={eo:.3e} (bound {to:.3e}) max|lse-oracle|={el:.3e}")
    assert eo <= to and el <= tl


def _random_permute_cases():
    cases = []
    for i in range(30):
        rng = np.random.default_rng(3000 + i)
        nd = int(rng.integers(1, 4))
        grid = [1, 1, int(rng.integers(1, 40))]
        if nd >= 2:
            grid[1] = int(rng.integers(1, 24))
        if nd == 3:
            grid[0] = int(rng.integers(1, 9))
        dtype = [torch.bfloat16, torch.float32, torch.float8_e4m3fn][i % 3]
        D = int(rng.choice([32, 64, 128]))
        tt_lg = int(rng.integers(0, 9))            # 1 .. 256 tokens per tile
        a = int(rng.integers(0, tt_lg + 1))
        b = int(rng.integers(0, tt_lg - a + 1))
        tile = (1 << a, 1 << b, 1 << (tt_lg - a - b))
        eb = torch.tensor([], dtype=dtype).element_size()
        transpose = bool(rng.random() < 0.6) and (1 << tt_lg) * eb % 16 == 0 and dtype != torch.float32
        cases.append((f"p{i}", tuple(grid), tile, dtype, D, int(rng.integers(1, 3)), int(rng.integers(1, 14)),
                      transpose))
    return cases


RANDOM_PERMUTE = _random_permute_cases()


@pytest.mark.parametrize("name,grid,tile,dtype,D,batch,heads,transpose", RANDOM_PERMUTE,
                         ids=[c[0] for c in RANDOM_PERMUTE])
def test_permute_random_shapes(na, name, grid, tile, dtype, D, batch, heads, transpose):
    # seeded random grids, power-of-two tiles of 1 .. 256 tokens, head dims,
    # head counts and element sizes: the tile layout bit for bit against the
    # NumPy index computation, and the round trip
    say(f"[permute] random {name} grid={grid} tile={tile} {dtype} D={D} B={batch} heads={heads} "
        f"transpose={transpose}")
    g = torch.Generator("cpu").manual_seed(3100 + int(name[1:]))
    x = torch.randn((batch, *grid, heads, D), generator=g).to(dtype)
    if transpose and math.prod(tile) * (D * x.element_size() + 4) > 65536:
        with pytest.raises(na.NAError):   # the staged tile would not fit in 64 KiB of LDS: refused on the host
            na.permute(x.cuda(), tile, transpose=True)
        return
    xt = na.permute(x.cuda(), tile, transpose=transpose)
    torch.cuda.synchronize()
    ib = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.float8_e4m3fn: torch.uint8}[dtype]
    ref = _ref_tile_order(x.view(ib).numpy(), tile, transpose)
    assert np.array_equal(xt.cpu().view(ib).numpy(), ref)
    if not transpose:
        back = na.unpermute(xt, grid, tile)
        torch.cuda.synchronize()
        assert torch.equal(back.cpu().view(ib), x.view(ib))


def test_calls_on_a_side_stream(na, path):
    # every call takes the caller's stream: the first call of a new geometry
    # (plan built and uploaded) and later ones on a non-default stream give
    # the default stream's results bit for bit, for the forward (each form),
    # and in form 1 for the backward and the top-k forward too
    import gpu_util
    wl = WORKLOADS["video_sliding"].with_(batch=2, heads=3, grid=(6, 13, 21), window=(3, 5, 9), stride=(1, 2, 4),
                                          seed=4242 + len(path))
    say(f"[special] side stream ({path})")
    _, _, _, _, q, k, v = inputs(wl)
    ws = gpu_util.USE_WORKSPACE
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o1, l1 = na.forward(q, k, v, wl.window, wl.stride, scale=wl.scale, stream=side, workspace=ws)
        o1b, l1b = na.forward(q, k, v, wl.window, wl.stride, scale=wl.scale, stream=side, workspace=ws)
    side.synchronize()
    o2, l2 = na.forward(q, k, v, wl.window, wl.stride, scale=wl.scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(o1b, o2) and torch.equal(l1b, l2)
    if path != "qo":
        return
    g = torch.Generator("cpu").manual_seed(4243)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16).cuda()
    with torch.cuda.stream(side):
        side.wait_stream(torch.cuda.default_stream())
        g1 = na.backward(q, k, v, o2, l2, do, wl.window, wl.stride, scale=wl.scale, stream=side)
        t1 = na.topk_forward(q, k, v, 3, scale=wl.scale, stream=side)
    side.synchronize()
    g2 = na.backward(q, k, v, o2, l2, do, wl.window, wl.stride, scale=wl.scale)
    t2 = na.topk_forward(q, k, v, 3, scale=wl.scale)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
    assert all(torch.equal(a, b) for a, b in zip(t1, t2))
