"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
compare it with the CPU oracle on the same seeded inputs."""

import math
import sys

import numpy as np
import torch

import oracle
from synth import make_qkv, to_f64

# max-abs tolerances on N(0,1) inputs.  out: the workload specification's
# bounds.  lse: l sums the weights exactly as the PV product uses them,
# rounded to the product's type (bf16: 8 significant bits, relative error at
# most 2^-8 each; e4m3: 4 bits, 2^-4), so |d lse| <= ln(1 + 2^-8) = 3.90e-3 for
# bf16 and ln(1 + 2^-4) = 0.0606 for fp8, plus fp32 rounding of the
# statistics (2e-5 / 1e-4 of slack); fp32 from its fp32 statistics alone.
# Large windows average the rounding out (measured ~1e-3 for bf16); windows of
# a few keys can approach the bound.
TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-2, math.log1p(2.0 ** -8) + 2e-5), "fp8": (6e-2, 6.1e-2)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# whether run_hip passes a workspace to na_forward (bf16: False selects the
# form that permutes nothing); the `path` fixtures switch it
USE_WORKSPACE = True


def run_hip(na, wl, q, k, v, sc, window=None, stride=None):
    f = na.Forward(q, k, v, window or wl.window, stride or wl.stride, scale=wl.scale,
                   qkv_scale=sc if wl.dtype == "fp8" else None,
                   workspace=USE_WORKSPACE or wl.dtype != "bf16" or q.shape[-1] not in (64, 128))
    out, lse = f()
    torch.cuda.synchronize()
    return out, lse, f


def compare(wl, qc, kc, vc, sc, out, lse, queries=None, heads=None, window=None, stride=None):
    """Max-abs errors of (out, lse) against the oracle on the given queries
    (linear indices, default all) and heads (default all)."""
    B, H = wl.batch, wl.heads
    N = wl.tokens
    D = wl.head_dim
    heads = range(H) if heads is None else heads
    o_all = out.detach().to("cpu").to(torch.float64).reshape(B, N, H, D)
    l_all = lse.detach().to("cpu").to(torch.float64).reshape(B, N, H)
    eo = el = 0.0
    qi = np.arange(N) if queries is None else np.asarray(queries)
    for h in heads:
        qh = to_f64(qc[..., h:h + 1, :], sc[0])
        kh = to_f64(kc[..., h:h + 1, :], sc[1])
        vh = to_f64(vc[..., h:h + 1, :], sc[2])
        ro, rl = oracle.attend(qh, kh, vh, wl.grid, window or wl.window, stride or wl.stride, wl.scale,
                               queries=None if queries is None else qi)
        go = o_all[:, qi, h, :].numpy()
        gl = l_all[:, qi, h].numpy()
        assert np.isfinite(go).all() and np.isfinite(gl).all()
        eo = max(eo, float(np.abs(go - ro[:, :, 0, :]).max()))
        el = max(el, float(np.abs(gl - rl[:, :, 0]).max()))
    return eo, el


def set_path(monkeypatch, path):
    """Selects the form of na_forward: "qo" (default: k, v permuted; q, out,
    lse in grid order), "grid" (no permutation, no workspace) or "tiled"
    (q, k, v permuted, out / lse unpermuted)."""
    import gpu_util
    if path == "tiled":
        monkeypatch.setenv("NA_NO_FUSED", "1")
    if path == "grid":
        monkeypatch.setattr(gpu_util, "USE_WORKSPACE", False)


def inputs(wl):
    qc, kc, vc, sc = make_qkv(wl, device="cpu")
    return qc, kc, vc, sc, qc.cuda(), kc.cuda(), vc.cuda()
