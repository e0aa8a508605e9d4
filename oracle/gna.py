"""Plain float64 oracle of Generalized Neighborhood Attention (GNA), forward.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

Page citations use the pages' titles:

* GNA page   -- "GNA Sparse Attention Mechanism: Vision-Transformer Compute
                Optimisation in Practice" (coreui.cn article 2627473).
* tutorial   -- "Video-generation inference speed-up: sparse attention
                configuration tutorial" (developer.baidu.com article 9729325).
* SLA page   -- "Sparse attention in video and image generation: optimisation
                practice" (ijyty.com news 926702).

Conventions.  A token grid has three extents (T, H, W); a 2-D problem has
T = 1 and a 1-D problem T = H = 1.  Tokens are numbered row-major over
(T, H, W).  Tensors are token-major with heads next and the feature
dimension last: q, k, v are [B, T, H, W, heads, D] (or [B, N, heads, D]).

Readings of points the pages leave open (each one is listed, with its
reason, in the design notes of the repository):

* window placement for even w: the window starts floor(w/2) keys before
  its centre query, so it holds floor(w/2) keys before and w - floor(w/2) - 1
  keys after it;
* borders: the window is shifted (clamped) to stay inside the grid, so every
  query sees exactly prod(w) keys ("fixed window around the query", GNA page
  section 1.1);
* stride: queries are grouped as floor(i / s); every query of a group uses
  the window of the group's leader, the group's centre g*s + floor(s/2)
  (clamped to L - 1).  s = 1 is plain sliding-window neighborhood attention;
  s > 1 makes the window move in jumps and gives the block pattern (GNA page
  section 1.1);
* no dilation, no causal mask, equal head counts for q and k/v.
"""

from __future__ import annotations

import itertools
import math

import numpy as np


# ----------------------------------------------------------------------------
# geometry
# ----------------------------------------------------------------------------

def validate_geometry(grid, window, stride):
    """Return (grid, window, stride) as int tuples; raise on an invalid one.

    The pages only describe 1 <= stride <= window <= extent (a stride larger
    than the window would leave keys no query sees; a window larger than the
    grid cannot be "fixed size").  Anything else is rejected.
    """
    grid = tuple(int(x) for x in grid)
    window = tuple(int(x) for x in window)
    stride = tuple(int(x) for x in stride)
    if not (len(grid) == len(window) == len(stride)) or not 1 <= len(grid) <= 3:
        raise ValueError("grid, window and stride need the same rank, 1 to 3")
    for L, w, s in zip(grid, window, stride):
        if not (1 <= s <= w <= L):
            raise ValueError(f"need 1 <= stride <= window <= extent, got s={s} w={w} L={L}")
    return grid, window, stride


def window_start(i: int, L: int, w: int, s: int) -> int:
    """First key coordinate of the window of query coordinate ``i`` on one axis.

    GNA page, section 1.1: each query attends to a fixed-size window around
    it; with stride s > 1 the window moves in jumps, i.e. all queries of one
    stride group share the window of the group's leader.
    """
    g = i // s                              # stride group of the query
    lead = min(g * s + s // 2, L - 1)       # leader: centre of the group
    start = lead - w // 2                   # floor(w/2) keys before the leader
    return min(max(start, 0), L - w)        # keep the whole window inside the grid


def window_starts(L: int, w: int, s: int) -> np.ndarray:
    """``window_start`` for every coordinate 0..L-1 of one axis."""
    return np.array([window_start(i, L, w, s) for i in range(L)], dtype=np.int64)


def key_set(coord, grid, window, stride) -> np.ndarray:
    """Sorted linear indices of the keys the query at ``coord`` attends to.

    The key set is the product over axes of the per-axis windows (GNA page,
    section 1.1, multi-dimensional neighborhoods); it has prod(window)
    members.
    """
    grid, window, stride = validate_geometry(grid, window, stride)
    axes = []
    for c, L, w, s in zip(coord, grid, window, stride):
        a = window_start(int(c), L, w, s)
        axes.append(range(a, a + w))
    keys = [int(np.ravel_multi_index(j, grid)) for j in itertools.product(*axes)]
    return np.array(sorted(keys), dtype=np.int64)


def key_index_table(grid, window, stride, queries=None) -> np.ndarray:
    """[nq, prod(window)] linear key indices of each query (ascending per row).

    ``queries`` are linear query indices (default: all tokens).  Each row is
    the same set as ``key_set`` of that query.
    """
    grid, window, stride = validate_geometry(grid, window, stride)
    N = math.prod(grid)
    if queries is None:
        queries = np.arange(N, dtype=np.int64)
    queries = np.asarray(queries, dtype=np.int64)
    coords = np.unravel_index(queries, grid)
    # per axis: absolute key coordinate for each (query, offset in window)
    per_axis = []
    for c, L, w, s in zip(coords, grid, window, stride):
        st = window_starts(L, w, s)[c]                      # [nq]
        per_axis.append(st[:, None] + np.arange(w)[None])   # [nq, w]
    # row-major product over axes -> linear index, ascending because each
    # axis' coordinates ascend and the product is taken row-major
    idx = np.zeros((len(queries), 1), dtype=np.int64)
    for ax, L in zip(per_axis, grid):
        idx = (idx[:, :, None] * L + ax[:, None, :]).reshape(len(queries), -1)
    return idx


def sparsity(grid, window) -> float:
    """Fraction of query-key pairs skipped: 1 - prod(w)/prod(L)."""
    return 1.0 - math.prod(window) / math.prod(grid)


def effective_flops(batch, heads, grid, window, head_dim) -> float:
    """Unmasked QK^T + PV FLOPs of one forward: 4 * b * h * N * prod(w) * D.

    GNA page, section 1.2: cost O(n k) with k the keys per query; one
    multiply-add counts as two FLOPs, softmax is not counted.
    """
    return 4.0 * batch * heads * math.prod(grid) * math.prod(window) * head_dim


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def attend(q, k, v, grid, window, stride, scale, queries=None, chunk_bytes=1 << 27):
    """Exact GNA forward on the CPU in float64.

    q, k, v: arrays [B, N, heads, D] or [B, T, H, W, heads, D] (any real
    dtype; upcast exactly to float64).  ``queries``: optional linear query
    indices to evaluate (default all).  Returns (out [B, nq, heads, D],
    lse [B, nq, heads]) in float64, lse in natural log.

    For each query i with key set K(i):
        s_ij   = scale * <q_i, k_j>
        m_i    = max_j s_ij,  l_i = sum_j exp(s_ij - m_i)
        out_i  = sum_j exp(s_ij - m_i) v_j / l_i,   lse_i = m_i + ln l_i
    (tutorial section 3.3: softmax over the kept connections only; SLA page
    section 3.1: softmax in FP32 or wider -- here float64.)
    """
    grid, window, stride = validate_geometry(grid, window, stride)
    N = math.prod(grid)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, heads, D = q.shape[0], q.shape[-2], q.shape[-1]
    q = q.reshape(B, N, heads, D)
    k = k.reshape(B, N, heads, D)
    v = v.reshape(B, N, heads, D)
    keys = key_index_table(grid, window, stride, queries)       # [nq, W]
    nq, W = keys.shape
    qi = np.arange(N) if queries is None else np.asarray(queries, dtype=np.int64)
    out = np.empty((B, nq, heads, D), dtype=np.float64)
    lse = np.empty((B, nq, heads), dtype=np.float64)
    step = max(1, int(chunk_bytes // (W * D * 8 * 2)))
    for b in range(B):
        for h in range(heads):
            for c0 in range(0, nq, step):
                c1 = min(nq, c0 + step)
                kk = keys[c0:c1]                                  # [n, W]
                Kg = k[b, kk, h, :]                               # [n, W, D]
                Vg = v[b, kk, h, :]
                qq = q[b, qi[c0:c1], h, :]                        # [n, D]
                s = scale * np.einsum("nd,nwd->nw", qq, Kg)
                m = s.max(axis=1)
                p = np.exp(s - m[:, None])
                l = p.sum(axis=1)
                out[b, c0:c1, h, :] = np.einsum("nw,nwd->nd", p, Vg) / l[:, None]
                lse[b, c0:c1, h] = m + np.log(l)
    return out, lse


# ----------------------------------------------------------------------------
# tile map
# ----------------------------------------------------------------------------

def _ceil_div(a, b):
    return -(-a // b)


def tile_pairs_1d(L, w, s, tq, tkv):
    """Brute-force per-axis pair counts between query tiles and key tiles.

    Returns (pairs [nQ, nK], valid_q [nQ], valid_k [nK]) where
    pairs[a, c] = #{(i, j): i // tq == a, j // tkv == c, j in window(i)},
    counting only real (non-padding) coordinates.
    """
    nQ, nK = _ceil_div(L, tq), _ceil_div(L, tkv)
    pairs = np.zeros((nQ, nK), dtype=np.int64)
    st = window_starts(L, w, s)
    for i in range(L):
        for j in range(L):
            if st[i] <= j < st[i] + w:
                pairs[i // tq, j // tkv] += 1
    valid_q = np.array([min(tq, L - a * tq) for a in range(nQ)], dtype=np.int64)
    valid_k = np.array([min(tkv, L - c * tkv) for c in range(nK)], dtype=np.int64)
    return pairs, valid_q, valid_k


def tile_map(grid, window, stride, tile_q, tile_kv, return_pairs=False):
    """CSR list of key tiles per query tile, full tiles first.

    GNA page section 1.1: the grid is cut into fixed-size multi-dimensional
    Q and KV tiles and the stride decides which KV tiles each Q tile visits;
    section 2.1: a fine-grained mask is needed only on a KV tile that is not
    fully inside the window.

    A KV tile c is listed under Q tile a iff some (query of a, key of c)
    pair is attended.  It is *full* iff every real query of a attends every
    slot of c (so c has no padding slot), else *boundary*.  Q tiles are in
    row-major tile order; inside a row: full tiles, then boundary tiles,
    each ascending in row-major KV-tile index.

    The key set of a query is a box (product of per-axis windows) and tiles
    are boxes, so pair counts factor over axes: pairs(a, c) = prod_d
    pairs_d(a_d, c_d).  (The test-suite checks this against brute force over
    all N-D pairs on small grids.)

    Returns (qptr int32 [nQ+1], kv_idx int32 [nnz], n_full int32 [nQ]) and,
    with ``return_pairs``, the pair count of each listed entry (int64).
    """
    grid, window, stride = validate_geometry(grid, window, stride)
    tile_q = tuple(int(x) for x in tile_q)
    tile_kv = tuple(int(x) for x in tile_kv)
    per = [tile_pairs_1d(L, w, s, a, b)
           for L, w, s, a, b in zip(grid, window, stride, tile_q, tile_kv)]
    nQ = [p[0].shape[0] for p in per]
    nK = [p[0].shape[1] for p in per]
    kv_slots = math.prod(tile_kv)
    qptr = [0]
    kv_idx, n_full, pair_list = [], [], []
    for a in itertools.product(*[range(n) for n in nQ]):
        # pairs with every KV tile (row-major over KV tiles)
        pr = np.ones((1,), dtype=np.int64)
        vq = 1
        for d in range(len(grid)):
            pr = np.multiply.outer(pr, per[d][0][a[d]]).reshape(-1)
            vq *= int(per[d][1][a[d]])
        listed = np.nonzero(pr > 0)[0]
        full = listed[pr[listed] == vq * kv_slots]
        bnd = listed[pr[listed] != vq * kv_slots]
        row = np.concatenate([full, bnd])
        kv_idx.extend(row.tolist())
        pair_list.extend(pr[row].tolist())
        n_full.append(len(full))
        qptr.append(len(kv_idx))
    res = (np.array(qptr, dtype=np.int32), np.array(kv_idx, dtype=np.int32),
           np.array(n_full, dtype=np.int32))
    if return_pairs:
        return res + (np.array(pair_list, dtype=np.int64),)
    return res


def tile_map_stats(grid, window, stride, tile_q, tile_kv):
    """Counts derived from ``tile_map``: tiles, full/boundary entries and the
    ratio of effective (attended) to computed (tile-area) query-key slots."""
    qptr, kv_idx, n_full, pairs = tile_map(grid, window, stride, tile_q, tile_kv,
                                           return_pairs=True)
    nQ = len(qptr) - 1
    nnz = int(qptr[-1])
    computed = nnz * math.prod(tile_q) * math.prod(tile_kv)
    effective = math.prod(grid) * math.prod(window)
    return {
        "n_q_tiles": nQ,
        "nnz": nnz,
        "n_full": int(n_full.sum()),
        "n_boundary": nnz - int(n_full.sum()),
        "kv_tiles_per_q_tile": nnz / nQ,
        "pairs_total": int(pairs.sum()),
        "computed_slots": computed,
        "effective_slots": effective,
        "efficiency": effective / computed,
    }
