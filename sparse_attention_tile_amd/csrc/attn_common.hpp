// Device-side pieces shared by the GNA attention kernels: the kernel
// argument block, the work-item decode (with the XCD-aware remap) and the
// per-query window test used on boundary tiles.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.hpp"

namespace na {

struct KParams {
  const void* qt;
  const void* kt;
  const void* vt;
  void* ot;
  float* lse_t;
  const int32_t* qptr;
  const int32_t* kv_idx;
  const int32_t* n_full;
  int nQ;               // Q tiles per (batch, head)
  int nK;               // KV tiles per (batch, head)
  int num_wg;           // batch * heads * nQ
  int L0, L1, L2;       // grid
  int w0, w1, w2;       // window
  int s0, s1, s2;       // stride
  int lq0, lq1, lq2;    // log2 of the Q tile extents
  int lk0, lk1, lk2;    // log2 of the KV tile extents
  int nq0, nq1, nq2;    // Q tiles per axis
  int nk1, nk2;         // KV tiles along H and W
  float scale;          // multiplies q.k
  float c2;             // scale * log2(e)
  float v_scale;        // multiplies the output (fp8), else 1
  int heads;            // heads (grid-order addressing)
  int64_t map_bh_kv;    // per-(batch, head) tile maps: kv_idx offset per bh
  int map_bh_nf;        // and n_full offset per bh (0: one shared map)
};

// Backward kernels' argument block (see BwdArgs).
struct BwdParams {
  KParams kp;
  const void* q;          // grid-order q (dq kernel reading grid order)
  const void* dot;
  const void* out;
  const void* dout;
  const float* lse;
  float* lse2_t;
  float* d_t;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* tqptr;
  const int32_t* tq_idx;
  const int32_t* tn_full;
};

inline int host_lg2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

inline KParams make_kparams(const AttnArgs& a) {
  KParams p;
  p.qt = a.qt;
  p.kt = a.kt;
  p.vt = a.vt;
  p.ot = a.ot;
  p.lse_t = a.lse_t;
  p.qptr = a.qptr;
  p.kv_idx = a.kv_idx;
  p.n_full = a.n_full;
  p.nQ = a.nq[0] * a.nq[1] * a.nq[2];
  p.nK = a.nk[0] * a.nk[1] * a.nk[2];
  p.num_wg = a.batch * a.heads * p.nQ;
  p.L0 = a.L[0]; p.L1 = a.L[1]; p.L2 = a.L[2];
  p.w0 = a.w[0]; p.w1 = a.w[1]; p.w2 = a.w[2];
  p.s0 = a.s[0]; p.s1 = a.s[1]; p.s2 = a.s[2];
  p.lq0 = host_lg2(a.tq[0]); p.lq1 = host_lg2(a.tq[1]); p.lq2 = host_lg2(a.tq[2]);
  p.lk0 = host_lg2(a.tkv[0]); p.lk1 = host_lg2(a.tkv[1]); p.lk2 = host_lg2(a.tkv[2]);
  p.nq0 = a.nq[0]; p.nq1 = a.nq[1]; p.nq2 = a.nq[2];
  p.nk1 = a.nk[1]; p.nk2 = a.nk[2];
  p.scale = a.scale;
  // scale * log2(e), kept >= 1e-30 so that a masked score (-inf) times c2
  // stays -inf when scale is 0 (finite scores times 1e-30 still round to 0
  // in exp2)
  p.c2 = fmaxf(a.scale * 1.4426950408889634f, 1e-30f);
  p.v_scale = a.v_scale;
  p.heads = a.heads;
  p.map_bh_kv = a.map_bh_kv;
  p.map_bh_nf = a.map_bh_nf;
  return p;
}

// Window start of query coordinate i on one axis (GNA page, "GNA Sparse
// Attention Mechanism: Vision-Transformer Compute Optimisation in Practice",
// section 1.1): queries of a stride group share the window of the group's
// centre; the window holds floor(w/2) keys before it and stays in the grid.
__device__ __forceinline__ int dev_window_start(int i, int L, int w, int s) {
  int lead = (i / s) * s + (s >> 1);
  lead = lead < L - 1 ? lead : L - 1;
  int st = lead - (w >> 1);
  st = st > 0 ? st : 0;
  return st < L - w ? st : L - w;
}

// Maps the hardware workgroup id to a work item.  Workgroups are dealt to the
// 8 XCDs round-robin (id % 8); each XCD has its own L2.  The remap gives
// every XCD one contiguous range of work items, and inside a (batch, head)
// the Q tiles are ordered with T fastest, so Q tiles that share the same KV
// tiles (stride groups along T) run side by side on one XCD.
struct WorkItem {
  int bh;      // batch * heads + head
  int qrow;    // row of the tile map (row-major Q tile index)
  int a0, a1, a2;  // Q tile coordinates
};

__device__ __forceinline__ WorkItem decode_work(const KParams& p, int bid) {
  const int nx = 8;
  const int q = p.num_wg / nx, r = p.num_wg % nx;
  const int x = bid % nx, loc = bid / nx;
  // Window maps: each XCD takes one contiguous range, so Q tiles with the
  // same KV list share an L2.  Per-(batch, head) content-selected maps have
  // no such locality: there consecutive workgroups go to different XCDs, so
  // the whole chip works on one head at a time and its K / V stay in the
  // Infinity Cache (measured 2-4 % faster for top-k).
  const int logical = p.map_bh_kv ? bid : (x < r ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc);
  WorkItem w;
  w.bh = logical / p.nQ;
  const int t = logical % p.nQ;
  w.a0 = t % p.nq0;
  const int rest = t / p.nq0;
  w.a2 = rest % p.nq2;
  w.a1 = rest / p.nq2;
  w.qrow = (w.a0 * p.nq1 + w.a1) * p.nq2 + w.a2;
  return w;
}

}  // namespace na
