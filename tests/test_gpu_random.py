"""GPU parity on seeded random geometries: 1-, 2- and 3-D grids of ragged
extents, random windows and strides (1 <= s <= w <= L per axis), batch and
heads > 1, head_dim 64 / 128, so the tile chooser lands on many different
tile shapes and kernel instantiations.  Every output of every head is
compared with the oracle (one oracle pass per case, shared by the forms),
and a second call with scale 0 must count exactly prod(window) keys for
every query (lse = ln prod(window))."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, inputs, say, set_path
from synth import WORKLOADS, to_f64

pytestmark = pytest.mark.gpu

FP8_FEW_KEYS = 16     # below this many keys per query fp8 is held to the few-key bound (see test_gpu_special)


def _geometry(rng):
    ndim = int(rng.integers(1, 4))
    while True:
        if ndim == 1:
            grid = (1, 1, int(rng.integers(2, 1500)))
        elif ndim == 2:
            grid = (1, int(rng.integers(2, 40)), int(rng.integers(2, 60)))
        else:
            grid = (int(rng.integers(2, 9)), int(rng.integers(2, 20)), int(rng.integers(2, 30)))
        window = tuple(int(rng.integers(1, L + 1)) for L in grid)
        if math.prod(grid) <= 1500 and math.prod(window) <= 600:
            break
    stride = tuple(int(rng.integers(1, w + 1)) for w in window)
    return grid, window, stride


def _cases():
    out = []
    for i in range(48):
        rng = np.random.default_rng(7000 + i)
        grid, window, stride = _geometry(rng)
        dtype = "fp8" if i % 4 == 3 else ("f32" if i % 7 == 5 else "bf16")
        D = 128 if dtype == "fp8" else int(rng.choice([64, 128]))
        batch, heads = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        out.append((f"r{i}", dtype, grid, window, stride, D, batch, heads))
    return out


CASES = _cases()


@pytest.mark.parametrize("name,dtype,grid,window,stride,D,batch,heads", CASES, ids=[c[0] for c in CASES])
def test_random_geometry(na, monkeypatch, name, dtype, grid, window, stride, D, batch, heads):
    base = {"bf16": WORKLOADS["img64_sliding"], "f32": WORKLOADS["img16_f32"], "fp8": WORKLOADS["img256_block_fp8"]}
    wl = base[dtype].with_(name=name, batch=batch, heads=heads, grid=grid, window=window, stride=stride,
                           head_dim=D, seed=7100 + int(name[1:]))
    qc, kc, vc, sc, q, k, v = inputs(wl)
    N, W = wl.tokens, math.prod(window)
    ro = np.empty((batch, N, heads, D))
    rl = np.empty((batch, N, heads))
    for h in range(heads):
        o, l = oracle.attend(to_f64(qc[..., h:h + 1, :], sc[0]), to_f64(kc[..., h:h + 1, :], sc[1]),
                             to_f64(vc[..., h:h + 1, :], sc[2]), grid, window, stride, wl.scale)
        ro[:, :, h, :] = o[:, :, 0, :]
        rl[:, :, h] = l[:, :, 0]
    to, tl = TOL[dtype]
    if dtype == "fp8" and W < FP8_FEW_KEYS:
        u = 2.0 ** -4
        to = max(to, 2 * u / (1 - u) * float(vc.float().abs().max()) * sc[2])
    forms = ["qo", "grid", "tiled"] if dtype == "bf16" else ["qo"]
    for form in forms:
        with monkeypatch.context() as mp:
            set_path(mp, form)
            import gpu_util
            ws = gpu_util.USE_WORKSPACE or dtype != "bf16"
            say(f"[random] {name} {dtype} ({form}) batch={batch} heads={heads} grid={grid} w={window} "
                f"s={stride} D={D}")
            f = na.Forward(q, k, v, window, stride, scale=wl.scale, qkv_scale=sc if dtype == "fp8" else None,
                           workspace=ws)
            out, lse = f()
            torch.cuda.synchronize()
            go = out.to("cpu", torch.float64).reshape(batch, N, heads, D).numpy()
            gl = lse.to("cpu", torch.float64).reshape(batch, N, heads).numpy()
            assert np.isfinite(go).all() and np.isfinite(gl).all()
            eo, el = float(np.abs(go - ro).max()), float(np.abs(gl - rl).max())
            # exact key count: with scale 0 every weight is 1
            f0 = na.Forward(q, k, v, window, stride, scale=0.0, qkv_scale=sc if dtype == "fp8" else None,
                            workspace=ws)
            _, lse0 = f0()
            torch.cuda.synchronize()
            ek = float((lse0.to("cpu", torch.float64) - math.log(W)).abs().max())
            say(f"  max|out-oracle|={eo:.3e} (bound {to:.3e}) max|lse-oracle|={el:.3e} (bound {tl:.3e}) "
                f"max|lse(scale 0) - ln W|={ek:.3e} tiles {f.tile_q} / {f.tile_kv}")
            assert eo <= to and el <= tl
            assert ek <= 1.0 / (4 * W) + 1e-6
            del f, f0, out, lse, lse0


def _pow2_shape(rng, tokens, min_w):
    """A random power-of-two (T, H, W) shape with `tokens` tokens and W >= min_w."""
    bits = int(math.log2(tokens))
    while True:
        a = int(rng.integers(0, bits + 1))
        b = int(rng.integers(0, bits - a + 1))
        c = bits - a - b
        if (1 << c) >= min_w:
            return (1 << a, 1 << b, 1 << c)


def _forced_cases():
    out = []
    for i in range(24):
        rng = np.random.default_rng(7600 + i)
        grid, window, stride = _geometry(rng)
        dtype = "fp8" if i % 3 == 2 else "bf16"
        D = 128 if dtype == "fp8" else int(rng.choice([64, 128]))
        tq = _pow2_shape(rng, int(rng.choice([128, 256])), 1)
        tk = _pow2_shape(rng, int(rng.choice([64, 128])), 8)
        out.append((f"f{i}", dtype, grid, window, stride, D, tq, tk))
    return out


FORCED = _forced_cases()


@pytest.mark.parametrize("name,dtype,grid,window,stride,D,tq,tk", FORCED, ids=[c[0] for c in FORCED])
def test_random_geometry_forced_tiles(na, monkeypatch, name, dtype, grid, window, stride, D, tq, tk):
    # random geometries with random (Q, KV) tile shapes forced through the
    # host hook, so tile / geometry pairs the chooser would not pick run too:
    # every output against the oracle and the exact key count
    base = {"bf16": WORKLOADS["img64_sliding"], "fp8": WORKLOADS["img256_block_fp8"]}
    wl = base[dtype].with_(name=name, batch=1, heads=2, grid=grid, window=window, stride=stride, head_dim=D,
                           seed=7700 + int(name[1:]))
    qc, kc, vc, sc, q, k, v = inputs(wl)
    N, W = wl.tokens, math.prod(window)
    ro = np.empty((1, N, 2, D))
    rl = np.empty((1, N, 2))
    for h in range(2):
        o, l = oracle.attend(to_f64(qc[..., h:h + 1, :], sc[0]), to_f64(kc[..., h:h + 1, :], sc[1]),
                             to_f64(vc[..., h:h + 1, :], sc[2]), grid, window, stride, wl.scale)
        ro[:, :, h, :] = o[:, :, 0, :]
        rl[:, :, h] = l[:, :, 0]
    to, tl = TOL[dtype]
    if dtype == "fp8" and W < FP8_FEW_KEYS:
        u = 2.0 ** -4
        to = max(to, 2 * u / (1 - u) * float(vc.float().abs().max()) * sc[2])
    monkeypatch.setenv("NA_TILE_Q", ",".join(map(str, tq)))
    monkeypatch.setenv("NA_TILE_KV", ",".join(map(str, tk)))
    forms = ["qo", "grid", "tiled"] if dtype == "bf16" else ["qo"]
    for form in forms:
        with monkeypatch.context() as mp:
            set_path(mp, form)
            import gpu_util
            ws = gpu_util.USE_WORKSPACE or dtype != "bf16"
            say(f"[random] forced {name} {dtype} ({form}) grid={grid} w={window} s={stride} D={D} tiles {tq} / {tk}")
            f = na.Forward(q, k, v, window, stride, scale=wl.scale, qkv_scale=sc if dtype == "fp8" else None,
                           workspace=ws)
            assert tuple(f.tile_q) == tq and tuple(f.tile_kv) == tk
            out, lse = f()
            f0 = na.Forward(q, k, v, window, stride, scale=0.0, qkv_scale=sc if dtype == "fp8" else None,
                            workspace=ws)
            _, lse0 = f0()
            torch.cuda.synchronize()
            go = out.to("cpu", torch.float64).reshape(1, N, 2, D).numpy()
            gl = lse.to("cpu", torch.float64).reshape(1, N, 2).numpy()
            eo, el = float(np.abs(go - ro).max()), float(np.abs(gl - rl).max())
            ek = float((lse0.to("cpu", torch.float64) - math.log(W)).abs().max())
            say(f"  max|out-oracle|={eo:.3e} (bound {to:.3e}) max|lse-oracle|={el:.3e} "
                f"max|lse(scale 0) - ln W|={ek:.3e}")
            assert np.isfinite(go).all() and np.isfinite(gl).all()
            assert eo <= to and el <= tl
            assert ek <= 1.0 / (4 * W) + 1e-6
            del f, f0, out, lse, lse0
