"""Python binding of libna.so, the MI355X GNA forward library.

The functions named ``na_*`` mirror the C ABI in ``include/na.h`` one to one
(argument marshalling only).  ``forward`` and friends are thin conveniences
that take torch tensors, allocate outputs and workspace with torch and call
those entry points on the current stream.  Every step of the computation
runs in the library's HIP kernels; there is no Python or CPU fallback: if
the library is missing, ``load()`` raises.
"""

from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# NA_LIB may name another build of the same library (e.g. to compare builds)
LIB_PATH = os.environ.get("NA_LIB") or os.path.join(HERE, "libna.so")

NA_OK, NA_ERR_INVALID_ARG, NA_ERR_UNSUPPORTED, NA_ERR_WORKSPACE, NA_ERR_HIP = 0, -1, -2, -3, -4
NA_F32, NA_BF16, NA_FP8_E4M3 = 0, 1, 2

SYMBOLS = (
    "na_choose_tiles", "na_build_tile_map", "na_simulate", "na_tile_candidates", "na_workspace_bytes",
    "na_forward_mode", "na_last_error",
    "na_release_cache", "na_forward", "na_permute", "na_unpermute", "na_unpermute_lse", "na_attend_tiled",
    "na_attend_kv_tiled", "na_backward_workspace_bytes", "na_backward", "na_topk_tiles",
    "na_topk_workspace_bytes", "na_topk_select", "na_topk_forward", "na_forward_noalloc",
)

# NA_NOALLOC_SCRATCH_BYTES of na.h: the fixed per-GPU device buffer of
# na_forward_noalloc
NOALLOC_SCRATCH_BYTES = 16 << 20


class NAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"na status {status}: {msg}")
        self.status = status


class TileMapStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n_q_tiles", "n_kv_tiles", "nnz", "n_full", "n_boundary", "computed_slots", "effective_slots")]


class SimResult(ctypes.Structure):
    _fields_ = [("tile_q", ctypes.c_int32 * 3), ("tile_kv", ctypes.c_int32 * 3), ("stats", TileMapStats),
                ("tile_efficiency", ctypes.c_double), ("flop_ratio_vs_dense", ctypes.c_double),
                ("speedup_bound", ctypes.c_double), ("perfectly_block_sparse", ctypes.c_int32),
                ("form", ctypes.c_int32), ("cost", ctypes.c_double), ("predicted_kernel_ms", ctypes.c_double),
                ("predicted_forward_ms", ctypes.c_double)]

    def as_dict(self):
        d = {n: getattr(self, n) for n, _ in self._fields_}
        d["tile_q"], d["tile_kv"] = tuple(self.tile_q), tuple(self.tile_kv)
        d["stats"] = {n: getattr(self.stats, n) for n, _ in TileMapStats._fields_}
        d["perfectly_block_sparse"] = bool(self.perfectly_block_sparse)
        return d


_lib = None
I3 = ctypes.c_int * 3
_p = ctypes.c_void_p
_i = ctypes.c_int
_fp = ctypes.POINTER(ctypes.c_float)


def load():
    """Loads libna.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python -m sparse_attention_tile_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "na_choose_tiles": ([I3, I3, I3, _i, _i, I3, I3], _i),
        "na_build_tile_map": ([I3, I3, I3, I3, I3, _p, _p, _p, ctypes.c_int64,
                               ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(TileMapStats)], _i),
        "na_workspace_bytes": ([_i, _i, _i, I3, I3, I3, _i], ctypes.c_size_t),
        "na_forward_mode": ([_i, _i, _i], _i),
        "na_simulate": ([_i, _i, _i, I3, I3, I3, _i, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                         ctypes.POINTER(SimResult)], _i),
        "na_tile_candidates": ([_i, _i, _i, I3, I3, I3, _i, ctypes.POINTER(SimResult), _i], _i),
        "na_last_error": ([], ctypes.c_char_p),
        "na_release_cache": ([], None),
        "na_forward": ([_p, _p, _p, _p, _p, _i, _i, _i, I3, I3, I3, ctypes.c_float, _i, _fp, _p,
                        ctypes.c_size_t, _p], _i),
        "na_permute": ([_p, _p, _i, _i, _i, I3, I3, _i, _i, _p], _i),
        "na_unpermute": ([_p, _p, _i, _i, _i, I3, I3, _i, _p], _i),
        "na_unpermute_lse": ([_p, _p, _i, _i, I3, I3, _p], _i),
        "na_attend_tiled": ([_p, _p, _p, _p, _p, _i, _i, _i, I3, I3, I3, I3, I3, ctypes.c_float, _i, _fp,
                             _p], _i),
        "na_attend_kv_tiled": ([_p, _p, _p, _p, _p, _i, _i, _i, I3, I3, I3, I3, ctypes.c_float, _i, _fp, _p], _i),
        "na_backward_workspace_bytes": ([_i, _i, _i, I3, I3, I3, _i], ctypes.c_size_t),
        "na_topk_tiles": ([I3, _i, _i, I3, I3], _i),
        "na_topk_workspace_bytes": ([_i, _i, _i, I3, _i, _i], ctypes.c_size_t),
        "na_topk_select": ([_p, _p, _i, _i, _i, I3, _i, _i, _p, _p, _p, ctypes.c_size_t, _p], _i),
        "na_topk_forward": ([_p, _p, _p, _p, _p, _i, _i, _i, I3, _i, ctypes.c_float, _i, _p, ctypes.c_size_t, _p],
                            _i),
        "na_backward": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, I3, I3, I3, ctypes.c_float, _i, _p,
                         ctypes.c_size_t, _p], _i),
        "na_forward_noalloc": ([_p, _p, _p, _p, _p, _i, _i, _i, I3, I3, I3, ctypes.c_float, _i, _p], _i),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(status: int):
    if status != NA_OK:
        raise NAError(status, na_last_error())


def _i3(x):
    return I3(*[int(v) for v in x])


# ---------------------------------------------------------------------------
# one-to-one wrappers of the C ABI
# ---------------------------------------------------------------------------

def na_last_error() -> str:
    return load().na_last_error().decode()


def na_release_cache() -> None:
    load().na_release_cache()


def na_choose_tiles(grid, window, stride, head_dim, dtype):
    tq, tk = I3(), I3()
    _check(load().na_choose_tiles(_i3(grid), _i3(window), _i3(stride), head_dim, dtype, tq, tk))
    return tuple(tq), tuple(tk)


def na_build_tile_map(grid, window, stride, tile_q, tile_kv):
    """Host tile map: returns (qptr, kv_idx, n_full) as numpy int32 arrays
    and the stats as a dict."""
    import numpy as np
    lib = load()
    nnz = ctypes.c_int64()
    st = TileMapStats()
    _check(lib.na_build_tile_map(_i3(grid), _i3(window), _i3(stride), _i3(tile_q), _i3(tile_kv),
                                 None, None, None, 0, ctypes.byref(nnz), ctypes.byref(st)))
    nq = st.n_q_tiles
    qptr = np.empty(nq + 1, dtype=np.int32)
    kv = np.empty(max(1, nnz.value), dtype=np.int32)
    nf = np.empty(nq, dtype=np.int32)
    _check(lib.na_build_tile_map(_i3(grid), _i3(window), _i3(stride), _i3(tile_q), _i3(tile_kv),
                                 qptr.ctypes.data, kv.ctypes.data, nf.ctypes.data, kv.size,
                                 ctypes.byref(nnz), ctypes.byref(st)))
    stats = {n: getattr(st, n) for n, _ in TileMapStats._fields_}
    return qptr, kv[: nnz.value], nf, stats


def na_simulate(batch, heads, head_dim, grid, window, stride, dtype, tile_q=None, tile_kv=None) -> dict:
    """Analytic model of one problem (see na.h): tile statistics, speedup
    bound over dense, perfectly-block-sparse flag, predicted MI355X ms."""
    r = SimResult()
    tq = _i3(tile_q) if tile_q is not None else None
    tk = _i3(tile_kv) if tile_kv is not None else None
    _check(load().na_simulate(batch, heads, head_dim, _i3(grid), _i3(window), _i3(stride), dtype, tq, tk,
                              ctypes.byref(r)))
    return r.as_dict()


def na_tile_candidates(batch, heads, head_dim, grid, window, stride, dtype) -> list:
    """Every tile-shape pair the chooser considers, sorted by cost (first =
    chosen), each as na_simulate reports it."""
    lib = load()
    n = lib.na_tile_candidates(batch, heads, head_dim, _i3(grid), _i3(window), _i3(stride), dtype, None, 0)
    if n < 0:
        _check(n)
    arr = (SimResult * max(1, n))()
    m = lib.na_tile_candidates(batch, heads, head_dim, _i3(grid), _i3(window), _i3(stride), dtype, arr, n)
    if m < 0:
        _check(m)
    return [arr[i].as_dict() for i in range(n)]


def na_forward_mode(dtype, head_dim, with_workspace=True) -> int:
    """Form of na_forward: 0 permute q, k, v (+ unpermute), 1 permute k, v only,
    2 no permutation (bf16 without a workspace)."""
    return int(load().na_forward_mode(dtype, head_dim, int(bool(with_workspace))))


def na_workspace_bytes(batch, heads, head_dim, grid, window, stride, dtype) -> int:
    n = load().na_workspace_bytes(batch, heads, head_dim, _i3(grid), _i3(window), _i3(stride), dtype)
    if n == 0 and na_last_error():
        raise NAError(NA_ERR_INVALID_ARG, na_last_error())
    return int(n)


def na_forward(q, k, v, out, lse, batch, heads, head_dim, grid, window, stride, scale, dtype,
               qkv_scale, workspace, workspace_bytes, stream):
    qs = (ctypes.c_float * 3)(*qkv_scale) if qkv_scale is not None else None
    _check(load().na_forward(q, k, v, out, lse, batch, heads, head_dim, _i3(grid), _i3(window), _i3(stride),
                             scale, dtype, qs, workspace, workspace_bytes, stream))


def na_forward_noalloc(q, k, v, out, lse, batch, heads, head_dim, grid, window, stride, scale, dtype, stream):
    _check(load().na_forward_noalloc(q, k, v, out, lse, batch, heads, head_dim, _i3(grid), _i3(window),
                                     _i3(stride), scale, dtype, stream))


def na_permute(x, xt, batch, heads, head_dim, grid, tile, elem_bytes, transpose, stream):
    _check(load().na_permute(x, xt, batch, heads, head_dim, _i3(grid), _i3(tile), elem_bytes, transpose, stream))


def na_unpermute(xt, x, batch, heads, head_dim, grid, tile, elem_bytes, stream):
    _check(load().na_unpermute(xt, x, batch, heads, head_dim, _i3(grid), _i3(tile), elem_bytes, stream))


def na_unpermute_lse(lse_t, lse, batch, heads, grid, tile, stream):
    _check(load().na_unpermute_lse(lse_t, lse, batch, heads, _i3(grid), _i3(tile), stream))


def na_attend_tiled(qt, kt, vt, ot, lse_t, batch, heads, head_dim, grid, window, stride, tile_q, tile_kv,
                    scale, dtype, qkv_scale, stream):
    qs = (ctypes.c_float * 3)(*qkv_scale) if qkv_scale is not None else None
    _check(load().na_attend_tiled(qt, kt, vt, ot, lse_t, batch, heads, head_dim, _i3(grid), _i3(window),
                                  _i3(stride), _i3(tile_q), _i3(tile_kv), scale, dtype, qs, stream))


def na_attend_kv_tiled(q, kt, vt, out, lse, batch, heads, head_dim, grid, window, stride, tile_kv, scale, dtype,
                       stream, qkv_scale=None):
    qs = (ctypes.c_float * 3)(*qkv_scale) if qkv_scale is not None else None
    _check(load().na_attend_kv_tiled(q, kt, vt, out, lse, batch, heads, head_dim, _i3(grid), _i3(window),
                                     _i3(stride), _i3(tile_kv), scale, dtype, qs, stream))


def na_backward_workspace_bytes(batch, heads, head_dim, grid, window, stride, dtype) -> int:
    n = load().na_backward_workspace_bytes(batch, heads, head_dim, _i3(grid), _i3(window), _i3(stride), dtype)
    if n == 0 and batch > 0 and heads > 0:
        raise NAError(NA_ERR_INVALID_ARG, na_last_error())
    return n


def na_backward(q, k, v, out, dout, lse, dq, dk, dv, batch, heads, head_dim, grid, window, stride, scale, dtype,
                workspace, workspace_bytes, stream):
    _check(load().na_backward(q, k, v, out, dout, lse, dq, dk, dv, batch, heads, head_dim, _i3(grid),
                              _i3(window), _i3(stride), scale, dtype, workspace, workspace_bytes, stream))


# ---------------------------------------------------------------------------
# torch conveniences (marshalling only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: NA_F32, torch.bfloat16: NA_BF16, torch.float8_e4m3fn: NA_FP8_E4M3}
    if t not in codes:
        raise NAError(NA_ERR_UNSUPPORTED, f"dtype {t} not supported")
    return codes[t]


def grid_of(q):
    """(T, H, W) of a [B, T, H, W, heads, D] / [B, H, W, heads, D] / [B, L, heads, D] tensor."""
    sp = tuple(q.shape[1:-2])
    if not 1 <= len(sp) <= 3:
        raise NAError(NA_ERR_INVALID_ARG, "q must be [B, *grid(1-3 dims), heads, D]")
    return (1,) * (3 - len(sp)) + sp


def _pad3(x, grid_rank):
    x = tuple(int(v) for v in (x if hasattr(x, "__len__") else [x] * grid_rank))
    if len(x) != grid_rank:
        raise NAError(NA_ERR_INVALID_ARG, "window/stride rank must match the grid")
    return (1,) * (3 - len(x)) + x


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Forward:
    """A prepared GNA forward call: validates once, owns the workspace and the
    outputs, and enqueues na_forward on each call (no allocation per call)."""

    def __init__(self, q, k, v, window, stride=1, scale=None, qkv_scale=None, return_lse=True, workspace=True):
        torch = _torch()
        load()
        for t in (q, k, v):
            if not t.is_cuda or not t.is_contiguous():
                raise NAError(NA_ERR_INVALID_ARG, "q, k, v must be contiguous device tensors")
        if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
            raise NAError(NA_ERR_INVALID_ARG, "q, k, v must have one shape and dtype")
        rank = q.dim() - 3
        self.grid = grid_of(q)
        self.window = _pad3(window, rank)
        self.stride = _pad3(stride, rank)
        self.batch, self.heads, self.head_dim = q.shape[0], q.shape[-2], q.shape[-1]
        self.dtype = dtype_code(q.dtype)
        self.scale = float(scale) if scale is not None else 1.0 / math.sqrt(self.head_dim)
        self.qkv_scale = tuple(qkv_scale) if qkv_scale is not None else None
        out_dtype = torch.float32 if self.dtype == NA_F32 else torch.bfloat16
        self.out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
        self.lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device) if return_lse else None
        if workspace:
            self.ws_bytes = na_workspace_bytes(self.batch, self.heads, self.head_dim, self.grid, self.window,
                                               self.stride, self.dtype)
            self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=q.device)
        else:   # permutation-free form (bf16, head_dim 64 / 128); else na_forward fails
            self.ws_bytes, self.workspace = 0, None
        self.mode = na_forward_mode(self.dtype, self.head_dim, workspace)
        self.tile_q, self.tile_kv = na_choose_tiles(self.grid, self.window, self.stride, self.head_dim, self.dtype)
        self.q, self.k, self.v = q, k, v

    def __call__(self, stream=None):
        na_forward(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.out.data_ptr(),
                   self.lse.data_ptr() if self.lse is not None else None, self.batch, self.heads, self.head_dim,
                   self.grid, self.window, self.stride, self.scale, self.dtype, self.qkv_scale,
                   self.workspace.data_ptr() if self.workspace is not None else None, self.ws_bytes,
                   _stream_ptr(stream))
        return self.out, self.lse


def forward(q, k, v, window, stride=1, scale=None, qkv_scale=None, return_lse=True, stream=None, workspace=True):
    """GNA forward of device tensors q, k, v ([B, *grid, heads, D]).

    Returns (out, lse): out has q's shape (bf16 for fp8 input), lse is
    [B, *grid, heads] fp32 (None if return_lse is False)."""
    f = Forward(q, k, v, window, stride, scale, qkv_scale, return_lse, workspace)
    return f(stream)


def na_topk_tiles(grid, head_dim, dtype):
    tq, tk = I3(), I3()
    _check(load().na_topk_tiles(_i3(grid), head_dim, dtype, tq, tk))
    return tuple(tq), tuple(tk)


def na_topk_workspace_bytes(batch, heads, head_dim, grid, keep, dtype) -> int:
    n = load().na_topk_workspace_bytes(batch, heads, head_dim, _i3(grid), keep, dtype)
    if n == 0 and batch > 0 and heads > 0:
        raise NAError(NA_ERR_INVALID_ARG, na_last_error())
    return n


def topk_select(q, k, keep, stream=None):
    """Content-selected tile map of q, k (bf16 device tensors [B, *grid,
    heads, D]): (kv_idx [B*heads, nQ, keep], n_full [B*heads, nQ]) int32."""
    torch = _torch()
    grid = grid_of(q)
    B, heads, D = q.shape[0], q.shape[-2], q.shape[-1]
    dt = dtype_code(q.dtype)
    tq, tk = na_topk_tiles(grid, D, dt)
    nq = math.prod(-(-L // t) for L, t in zip(grid, tq))
    nb = na_topk_workspace_bytes(B, heads, D, grid, keep, dt)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
    idx = torch.empty((B * heads, nq, keep), dtype=torch.int32, device=q.device)
    nf = torch.empty((B * heads, nq), dtype=torch.int32, device=q.device)
    _check(load().na_topk_select(q.data_ptr(), k.data_ptr(), B, heads, D, _i3(grid), keep, dt, idx.data_ptr(),
                                 nf.data_ptr(), ws.data_ptr(), nb, _stream_ptr(stream)))
    return idx, nf


def topk_forward(q, k, v, keep, scale=None, return_lse=True, stream=None):
    """Attention of every query over the `keep` KV tiles its Q tile selects
    (block-mean scores): (out, lse) like ``forward``."""
    torch = _torch()
    grid = grid_of(q)
    B, heads, D = q.shape[0], q.shape[-2], q.shape[-1]
    dt = dtype_code(q.dtype)
    scale = float(scale) if scale is not None else 1.0 / math.sqrt(D)
    nb = na_topk_workspace_bytes(B, heads, D, grid, keep, dt)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device) if return_lse else None
    _check(load().na_topk_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr() if lse is not None else None, B, heads, D, _i3(grid), keep, scale,
                                  dt, ws.data_ptr(), nb, _stream_ptr(stream)))
    return out, lse


def backward(q, k, v, out, lse, dout, window, stride=1, scale=None, stream=None):
    """Gradients (dq, dk, dv) of ``forward`` for the loss sum(dout * out), bf16
    device tensors in q's layout; ``out`` and ``lse`` are the forward's
    outputs for the same q, k, v."""
    torch = _torch()
    load()
    for t in (q, k, v, out, dout, lse):
        if not t.is_cuda or not t.is_contiguous():
            raise NAError(NA_ERR_INVALID_ARG, "inputs must be contiguous device tensors")
    rank = q.dim() - 3
    grid = grid_of(q)
    window, stride = _pad3(window, rank), _pad3(stride, rank)
    B, heads, D = q.shape[0], q.shape[-2], q.shape[-1]
    dtype = dtype_code(q.dtype)
    scale = float(scale) if scale is not None else 1.0 / math.sqrt(D)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    nb = na_backward_workspace_bytes(B, heads, D, grid, window, stride, dtype)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
    na_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, heads, D, grid, window, stride, scale, dtype,
                ws.data_ptr(), nb, _stream_ptr(stream))
    return dq, dk, dv


def permute(x, tile, transpose=False, stream=None):
    """Grid order [B, *grid, heads, D] -> tile order [B, heads, tiles, tokens, D]
    (or [.., D, tokens] with transpose) as a new device tensor."""
    torch = _torch()
    grid = grid_of(x)
    tile = _pad3(tile, 3)
    B, heads, D = x.shape[0], x.shape[-2], x.shape[-1]
    nt = [-(-L // t) for L, t in zip(grid, tile)]
    tt = math.prod(tile)
    shape = (B, heads, math.prod(nt), D, tt) if transpose else (B, heads, math.prod(nt), tt, D)
    xt = torch.empty(shape, dtype=x.dtype, device=x.device)
    na_permute(x.data_ptr(), xt.data_ptr(), B, heads, D, grid, tile, x.element_size(), int(bool(transpose)),
               _stream_ptr(stream))
    return xt


def unpermute(xt, grid, tile, stream=None):
    """Tile order [B, heads, tiles, tokens, D] -> grid order [B, T, H, W, heads, D]."""
    torch = _torch()
    B, heads, D = xt.shape[0], xt.shape[1], xt.shape[-1]
    x = torch.empty((B, *grid, heads, D), dtype=xt.dtype, device=xt.device)
    na_unpermute(xt.data_ptr(), x.data_ptr(), B, heads, D, grid, _pad3(tile, 3), xt.element_size(),
                 _stream_ptr(stream))
    return x
