"""Oracle of content-selected block sparsity (top-k KV blocks per Q block).

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

The tutorial ("Video-generation inference speed-up: sparse attention
configuration tutorial", section 6, the data flow of sparse attention)
splits the sequence into blocks, scores block importance (its example: the
block mean), keeps the most important blocks by a keep ratio and skips the
rest whole, then runs block-wise attention with accumulated normalisation
over the kept blocks.  The overview page ("Sparse attention: the key
technology for more efficient AI models", section 2.2) lists top-k selection
among the content-based schemes.  Readings:

* blocks are the multi-dimensional tiles of the grid (Q tiles for queries,
  KV tiles for keys) -- the same tiles the GNA kernels use;
* score(a, c) = <mean of q over the real tokens of Q tile a, mean of k over
  the real tokens of KV tile c> (a positive softmax scale does not change the
  ranking and is left out);
* each Q tile keeps its ``keep`` highest-scoring KV tiles (equal scores: the
  lower tile index first); every query of the Q tile attends to every real
  key of the kept tiles, with an exact softmax over that union.

The selection is an integer decision taken from floating-point scores, so
the oracle evaluates the scores in float32 in one fixed order, the order the
kernel uses: block sums accumulate token by token in in-tile row-major order,
the mean is that sum divided by the real-token count (IEEE division), and a
score accumulates product by product over the head dimension (each product
and each sum rounded to float32, no fused multiply-add).  The attention
itself is float64.
"""

from __future__ import annotations

import math

import numpy as np


def _tile_tokens(grid, tile, index):
    """Linear grid indices of the real tokens of tile ``index`` (row-major
    tile order), in in-tile row-major order."""
    nt = [-(-L // t) for L, t in zip(grid, tile)]
    a0, rem = divmod(index, nt[1] * nt[2])
    a1, a2 = divmod(rem, nt[2])
    out = []
    for dt in range(tile[0]):
        for dy in range(tile[1]):
            for dx in range(tile[2]):
                t, y, x = a0 * tile[0] + dt, a1 * tile[1] + dy, a2 * tile[2] + dx
                if t < grid[0] and y < grid[1] and x < grid[2]:
                    out.append((t * grid[1] + y) * grid[2] + x)
    return np.array(out, dtype=np.int64)


def block_means_f32(x, grid, tile):
    """[B, nTiles, heads, D] float32 means of x ([B, N, heads, D], any real
    dtype) over each tile's real tokens: sequential float32 sums in in-tile
    row-major order, divided by the count."""
    x = np.asarray(x, dtype=np.float32)
    B, heads, D = x.shape[0], x.shape[-2], x.shape[-1]
    x = x.reshape(B, -1, heads, D)
    nt = math.prod(-(-L // t) for L, t in zip(grid, tile))
    out = np.zeros((B, nt, heads, D), dtype=np.float32)
    for a in range(nt):
        toks = _tile_tokens(grid, tile, a)
        acc = np.zeros((B, heads, D), dtype=np.float32)
        for tok in toks:
            acc = (acc + x[:, tok]).astype(np.float32)
        out[:, a] = (acc / np.float32(len(toks))).astype(np.float32)
    return out


def block_scores_f32(qm, km):
    """[B, heads, nQ, nK] float32 scores <qm_a, km_c>, accumulated over the
    head dimension in order, each product and sum rounded to float32."""
    B, nQ, heads, D = qm.shape
    nK = km.shape[1]
    s = np.zeros((B, heads, nQ, nK), dtype=np.float32)
    qh = np.transpose(qm, (0, 2, 1, 3))          # [B, h, nQ, D]
    kh = np.transpose(km, (0, 2, 1, 3))          # [B, h, nK, D]
    for d in range(D):
        prod = (qh[:, :, :, None, d] * kh[:, :, None, :, d]).astype(np.float32)
        s = (s + prod).astype(np.float32)
    return s


def select_blocks(scores, keep, kv_full):
    """Per row of ``scores`` [..., nQ, nK]: the ``keep`` best KV tiles (score
    descending, index ascending on ties), listed as the kernels want them --
    tiles without padding slots (``kv_full[c]``) first, then the others, each
    ascending.  Returns (kv_idx [..., nQ, keep] int32, n_full [..., nQ])."""
    lead = scores.shape[:-1]
    nK = scores.shape[-1]
    flat = scores.reshape(-1, nK)
    idx = np.empty((flat.shape[0], keep), dtype=np.int32)
    nf = np.empty(flat.shape[0], dtype=np.int32)
    order_key = np.arange(nK)
    for r in range(flat.shape[0]):
        # lexsort: last key is primary -> sort by -score, then index
        best = np.lexsort((order_key, -flat[r].astype(np.float64)))[:keep]
        full = sorted(int(c) for c in best if kv_full[c])
        part = sorted(int(c) for c in best if not kv_full[c])
        idx[r] = full + part
        nf[r] = len(full)
    return idx.reshape(*lead, keep), nf.reshape(lead)


def kv_tile_is_full(grid, tile_kv):
    """True for KV tiles with no padding slot (every slot a real token)."""
    nt = math.prod(-(-L // t) for L, t in zip(grid, tile_kv))
    per = math.prod(tile_kv)
    return np.array([len(_tile_tokens(grid, tile_kv, c)) == per for c in range(nt)])


def topk_select(q, k, grid, tile_q, tile_kv, keep):
    """The selection: (kv_idx [B, heads, nQ, keep], n_full [B, heads, nQ])."""
    qm = block_means_f32(q, grid, tile_q)
    km = block_means_f32(k, grid, tile_kv)
    s = block_scores_f32(qm, km)
    return select_blocks(s, keep, kv_tile_is_full(grid, tile_kv))


def topk_attend(q, k, v, grid, tile_q, tile_kv, keep, scale, queries=None):
    """Attention over the selected blocks, float64: (out [B, nq, heads, D],
    lse [B, nq, heads]) for the linear query indices ``queries`` (default
    all)."""
    kv_idx, _ = topk_select(q, k, grid, tile_q, tile_kv, keep)
    q64 = np.asarray(q, dtype=np.float64)
    B, heads, D = q64.shape[0], q64.shape[-2], q64.shape[-1]
    N = math.prod(grid)
    q64 = q64.reshape(B, N, heads, D)
    k64 = np.asarray(k, dtype=np.float64).reshape(B, N, heads, D)
    v64 = np.asarray(v, dtype=np.float64).reshape(B, N, heads, D)
    qs = np.arange(N) if queries is None else np.asarray(queries, dtype=np.int64)
    coords = np.unravel_index(qs, grid)
    nt_q = [-(-L // t) for L, t in zip(grid, tile_q)]
    qtile = ((coords[0] // tile_q[0]) * nt_q[1] + coords[1] // tile_q[1]) * nt_q[2] + coords[2] // tile_q[2]
    nK = math.prod(-(-L // t) for L, t in zip(grid, tile_kv))
    tok_of = [_tile_tokens(grid, tile_kv, c) for c in range(nK)]
    out = np.empty((B, len(qs), heads, D))
    lse = np.empty((B, len(qs), heads))
    for b in range(B):
        for h in range(heads):
            for n, (i, a) in enumerate(zip(qs, qtile)):
                keys = np.concatenate([tok_of[c] for c in kv_idx[b, h, a]])
                s = scale * k64[b, keys, h, :] @ q64[b, i, h, :]
                m = s.max()
                p = np.exp(s - m)
                l = p.sum()
                out[b, n, h] = p @ v64[b, keys, h, :] / l
                lse[b, n, h] = m + math.log(l)
    return out, lse
