"""Seeded synthetic inputs and the workload table.

This module draws random numbers and casts them; it holds none of the
attention method's arithmetic.  Both the HIP path (tests, bench) and the
CPU oracle consume exactly the tensors made here.

Recipe (the same for every workload): a CPU ``torch.Generator`` seeded with
the workload's seed draws q, k, v in that order as fp32 N(0, 1) tensors of
shape [batch, T, H, W, heads, head_dim].  They are then cast to the run
dtype: bf16 by round-to-nearest-even; fp8 by per-tensor quantisation to OCP
e4m3fn with scale = amax / 448 (the stored value is round(x / scale),
saturated to +-448, and x ~ value * scale).  The real activations of the
video and image models the pages measure (HunyuanVideo latents of 30x48x80
tokens, FLUX-1.dev 4K latents of 256x256 tokens) are not available; N(0, 1)
tensors of the same shapes stand in for them.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    grid: tuple          # (T, H, W)
    head_dim: int
    window: tuple        # (T, H, W)
    stride: tuple        # (T, H, W)
    dtype: str           # "f32" | "bf16" | "fp8"
    seed: int
    note: str = ""

    @property
    def tokens(self) -> int:
        return math.prod(self.grid)

    @property
    def keys_per_query(self) -> int:
        return math.prod(self.window)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def effective_flops(self) -> float:
        """4 * b * h * N * prod(w) * D: unmasked QK^T + PV FLOPs."""
        return 4.0 * self.batch * self.heads * self.tokens * self.keys_per_query * self.head_dim

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


VIDEO = (30, 48, 80)

WORKLOADS = {
    # 2-D neighborhood attention in fp32, the small exact case.
    "img16_f32": Workload("img16_f32", 1, 1, (1, 16, 16), 32, (1, 5, 5), (1, 1, 1), "f32", 101),
    # 2-D image attention in bf16, sliding and block mode.
    "img64_sliding": Workload("img64_sliding", 2, 8, (1, 64, 64), 64, (1, 17, 17), (1, 1, 1), "bf16", 201),
    "img64_block": Workload("img64_block", 2, 8, (1, 64, 64), 64, (1, 16, 16), (1, 8, 8), "bf16", 202),
    # 3-D video attention, HunyuanVideo latent shape (GNA page section 3.1).
    "video_sliding": Workload("video_sliding", 1, 24, VIDEO, 128, (30, 40, 40), (1, 1, 1), "bf16", 301,
                              "58.3% sparse, GNA(s1x1x1)"),
    "video_block": Workload("video_block", 1, 24, VIDEO, 128, (18, 24, 24), (16, 8, 8), "bf16", 401,
                            "91.0% sparse, GNA(s16x8x8)"),
    "video_dense": Workload("video_dense", 1, 24, VIDEO, 128, VIDEO, (1, 1, 1), "bf16", 401,
                            "window = grid: dense speed-up reference"),
    # 2-D 4K-image latent attention (GNA page section 3.2 / 4.1).
    "img256_block": Workload("img256_block", 1, 24, (1, 256, 256), 128, (1, 64, 64), (1, 16, 16), "bf16", 501),
    "img256_block_fp8": Workload("img256_block_fp8", 1, 24, (1, 256, 256), 128, (1, 64, 64), (1, 16, 16), "fp8", 501),
}


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor e4m3fn quantisation: returns (x8, scale) with x ~ x8 * scale."""
    amax = float(x.abs().max())
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    x8 = (x / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return x8, scale


def make_qkv(wl: Workload, device="cpu", seed=None):
    """Draw q, k, v for a workload.  Returns (q, k, v, qkv_scale) where the
    tensors are [B, T, H, W, heads, D] in the run dtype on ``device`` and
    qkv_scale is (1, 1, 1) except for fp8."""
    g = torch.Generator("cpu").manual_seed(wl.seed if seed is None else seed)
    shape = (wl.batch, *wl.grid, wl.heads, wl.head_dim)
    t = [torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(3)]
    if wl.dtype == "f32":
        out, sc = t, (1.0, 1.0, 1.0)
    elif wl.dtype == "bf16":
        out, sc = [x.to(torch.bfloat16) for x in t], (1.0, 1.0, 1.0)
    elif wl.dtype == "fp8":
        qs = [quantize_e4m3(x) for x in t]
        out, sc = [a for a, _ in qs], tuple(b for _, b in qs)
    else:
        raise ValueError(wl.dtype)
    return (*[x.to(device) for x in out], sc)


def to_f64(x: torch.Tensor, scale: float = 1.0):
    """Exact upcast of a (possibly quantised) tensor to a float64 numpy array."""
    a = x.detach().to("cpu").to(torch.float64)
    if scale != 1.0:
        a = a * scale
    return a.numpy()


def sample_queries(wl: Workload, tile_q, n_random=1024, seed_offset=7):
    """Seeded query sample for parity at full size: every query of the 8
    corner query tiles and of 4 edge-midpoint tiles, plus ``n_random``
    uniformly drawn queries.  Returns sorted unique linear query indices."""
    import numpy as np
    grid = wl.grid
    nt = [-(-L // t) for L, t in zip(grid, tile_q)]
    picks = set()
    corners = [(a, b, c) for a in (0, nt[0] - 1) for b in (0, nt[1] - 1) for c in (0, nt[2] - 1)]
    mids = [(nt[0] // 2, 0, nt[2] // 2), (nt[0] // 2, nt[1] - 1, nt[2] // 2),
            (nt[0] // 2, nt[1] // 2, 0), (nt[0] // 2, nt[1] // 2, nt[2] - 1)]
    for tc in corners + mids:
        for dt in range(tile_q[0]):
            for dh in range(tile_q[1]):
                for dw in range(tile_q[2]):
                    t = tc[0] * tile_q[0] + dt
                    h = tc[1] * tile_q[1] + dh
                    w = tc[2] * tile_q[2] + dw
                    if t < grid[0] and h < grid[1] and w < grid[2]:
                        picks.add((t * grid[1] + h) * grid[2] + w)
    rng = np.random.default_rng(wl.seed + seed_offset)
    picks.update(rng.integers(0, wl.tokens, size=n_random).tolist())
    return np.array(sorted(picks), dtype=np.int64)
