"""Plain float64 oracle of the GNA backward pass (gradients of the forward).

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

The pages name training with GNA as the next step ("GNA Sparse Attention
Mechanism: Vision-Transformer Compute Optimisation in Practice", section 5:
integrate the sparse pattern into training) and keep the softmax statistics
in FP32 or wider ("Sparse attention in video and image generation:
optimisation practice", section 3.1).  They give no backward formulas; the
gradients here are the plain derivatives of the forward ``gna.attend`` for
the scalar loss  L = sum_i <dout_i, out_i>  (no gradient flows into lse):

    s_ij  = scale <q_i, k_j>,   p_ij = exp(s_ij - lse_i)      (j in K(i))
    D_i   = <dout_i, out_i> = sum_j p_ij <dout_i, v_j>
    dP_ij = <dout_i, v_j>,      dS_ij = p_ij (dP_ij - D_i)
    dq_i  = scale sum_{j in K(i)}  dS_ij k_j
    dk_j  = scale sum_{i : j in K(i)} dS_ij q_i
    dv_j  =       sum_{i : j in K(i)} p_ij dout_i

The sums over keys use the forward's key table; the sums over queries use
the inverse table (the queries whose window holds a key), built from the
same per-axis window starts.
"""

from __future__ import annotations

import math

import numpy as np

from .gna import attend, key_index_table, validate_geometry, window_starts


def query_index_lists(grid, window, stride, keys):
    """For each linear key index in ``keys``: the ascending linear indices of
    the queries whose key set contains it.

    Per axis the queries whose window holds coordinate c are those i with
    start(i) <= c < start(i) + w; the set for a key is the product over axes.
    """
    grid, window, stride = validate_geometry(grid, window, stride)
    starts = [window_starts(L, w, s) for L, w, s in zip(grid, window, stride)]
    out = []
    for key in np.asarray(keys, dtype=np.int64):
        coord = np.unravel_index(int(key), grid)
        per_axis = []
        for c, st, w in zip(coord, starts, window):
            per_axis.append(np.nonzero((st <= c) & (c < st + w))[0])
        idx = np.zeros(1, dtype=np.int64)
        for ax, L in zip(per_axis, grid):
            idx = (idx[:, None] * L + ax[None, :]).reshape(-1)
        out.append(idx)
    return out


def attend_backward(q, k, v, dout, grid, window, stride, scale, queries=None, keys=None):
    """Gradients of ``gna.attend`` for the loss sum <dout, out>, in float64.

    q, k, v, dout: [B, N, heads, D] or [B, T, H, W, heads, D].  ``queries``
    (default all) selects the rows of dq that are computed, ``keys`` (default
    all) the rows of dk and dv.  Returns (dq [B, nq, heads, D],
    dk [B, nk, heads, D], dv [B, nk, heads, D]).
    """
    grid, window, stride = validate_geometry(grid, window, stride)
    N = math.prod(grid)
    q = np.asarray(q, dtype=np.float64)
    B, heads, D = q.shape[0], q.shape[-2], q.shape[-1]
    q = q.reshape(B, N, heads, D)
    k = np.asarray(k, dtype=np.float64).reshape(B, N, heads, D)
    v = np.asarray(v, dtype=np.float64).reshape(B, N, heads, D)
    dout = np.asarray(dout, dtype=np.float64).reshape(B, N, heads, D)
    qsel = np.arange(N) if queries is None else np.asarray(queries, dtype=np.int64)
    ksel = np.arange(N) if keys is None else np.asarray(keys, dtype=np.int64)

    # ---- dq: one query at a time over its key set
    dq = np.zeros((B, len(qsel), heads, D))
    if len(qsel):
        out_q, lse_q = attend(q, k, v, grid, window, stride, scale, queries=qsel)
        ktab = key_index_table(grid, window, stride, qsel)          # [nq, W]
        for b in range(B):
            for h in range(heads):
                Kg = k[b, ktab, h, :]                                 # [nq, W, D]
                Vg = v[b, ktab, h, :]
                s = scale * np.einsum("nd,nwd->nw", q[b, qsel, h, :], Kg)
                p = np.exp(s - lse_q[b, :, h][:, None])
                do = dout[b, qsel, h, :]
                Di = np.einsum("nd,nd->n", do, out_q[b, :, h, :])
                dP = np.einsum("nd,nwd->nw", do, Vg)
                dS = p * (dP - Di[:, None])
                dq[b, :, h, :] = scale * np.einsum("nw,nwd->nd", dS, Kg)

    # ---- dk, dv: one key at a time over the queries that attend it
    dk = np.zeros((B, len(ksel), heads, D))
    dv = np.zeros((B, len(ksel), heads, D))
    if len(ksel):
        qlists = query_index_lists(grid, window, stride, ksel)
        needed = np.unique(np.concatenate(qlists))
        out_n, lse_n = attend(q, k, v, grid, window, stride, scale, queries=needed)
        pos = {int(t): r for r, t in enumerate(needed)}
        for kk, (key, ql) in enumerate(zip(ksel, qlists)):
            rows = np.array([pos[int(t)] for t in ql], dtype=np.int64)
            for b in range(B):
                for h in range(heads):
                    qq = q[b, ql, h, :]                                 # [m, D]
                    do = dout[b, ql, h, :]
                    s = scale * qq @ k[b, key, h, :]
                    p = np.exp(s - lse_n[b, rows, h])
                    Di = np.einsum("md,md->m", do, out_n[b, rows, h, :])
                    dP = do @ v[b, key, h, :]
                    dS = p * (dP - Di)
                    dk[b, kk, h, :] = scale * dS @ qq
                    dv[b, kk, h, :] = p @ do
    return dq, dk, dv
