// bf16 GNA attention backward on gfx950 matrix cores.
//
// What it computes: the gradients of the forward (GNA page, "GNA Sparse
// Attention Mechanism: Vision-Transformer Compute Optimisation in Practice",
// sections 1.1 and 2.1; section 5 names training with the sparse pattern as
// the next step) for the loss sum <dO, O>, with the softmax statistics kept in
// fp32 (SLA page, "Sparse attention in video and image generation:
// optimisation practice", section 3.1):
//   p_ij = exp(scale q_i.k_j - lse_i),  D_i = <dO_i, O_i>
//   dS_ij = p_ij (<dO_i, v_j> - D_i)
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
//   dv_j = sum_i p_ij dO_i
// over exactly the (query, key) pairs of the forward's windows.
//
// Three kernels, no atomics (every output row is written by one workgroup):
//  * prep: D_i and lse_i log2(e) into tile order (padding rows 0);
//  * dq: one workgroup per Q tile, over the Q tile's KV tiles (the forward
//    tile map): S^T = K Q^T and dP^T = V dO^T with q and dO in registers,
//    dQ^T += K^T dS^T with K^T read by the transposing LDS load;
//  * dkdv: one workgroup per KV tile, over the Q tiles that list it (the
//    transposed tile map): S = Q K^T and dP = dO V^T with k and v in
//    registers, dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read by
//    the transposing LDS load.
// Inputs come in tile order as na_permute writes them (plain rows, v not
// transposed); dq, dk, dv are written in grid order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <type_traits>

#include "attn_common.hpp"
#include "attn_device.hpp"

namespace na {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// In-tile slot r of a tile with log2 extents (l0, l1, l2) -> grid coordinates
// of tile (a0, a1, a2).
struct Coord3 { int t, y, x; };
__device__ __forceinline__ Coord3 slot_coord(int r, int a0, int a1, int a2, int l0, int l1, int l2) {
  Coord3 c;
  c.x = (a2 << l2) + (r & ((1 << l2) - 1));
  c.y = (a1 << l1) + ((r >> l2) & ((1 << l1) - 1));
  c.t = (a0 << l0) + (r >> (l1 + l2));
  return c;
}

// ---------------------------------------------------------------------------
// prep: D = <dO, O> (fp32) and lse * log2(e) per query, in tile order.  LPR
// lanes share one (token, head) row, 8 dims each.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const KParams& k = p.kp;
  const int qtok = 1 << (k.lq0 + k.lq1 + k.lq2);
  const int64_t rows = (int64_t)k.num_wg * qtok;      // batch * heads * padded query slots
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  if (r >= rows) return;
  const int64_t bhq = r / qtok;                       // (b*heads + h) * nQ + tile
  const int in = (int)(r % qtok);
  const int tile = (int)(bhq % k.nQ);
  const int bh = (int)(bhq / k.nQ);
  const int a2 = tile % k.nq2, a1 = (tile / k.nq2) % k.nq1, a0 = tile / (k.nq2 * k.nq1);
  const Coord3 c = slot_coord(in, a0, a1, a2, k.lq0, k.lq1, k.lq2);
  const bool valid = c.t < k.L0 && c.y < k.L1 && c.x < k.L2;
  float dot = 0.f;
  float ls = 0.f;
  if (valid) {
    const int b = bh / k.heads, h = bh % k.heads;
    const int64_t tok = ((int64_t)c.t * k.L1 + c.y) * k.L2 + c.x;
    const int64_t gi = ((int64_t)b * k.L0 * k.L1 * k.L2 + tok) * k.heads + h;
    const bf16x8 o = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.out) + gi * D)[sub];
    const bf16x8 g = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.dout) + gi * D)[sub];
#pragma unroll
    for (int j = 0; j < 8; ++j) dot = fmaf((float)o[j], (float)g[j], dot);
    ls = p.lse[gi] * kLog2e;
  }
#pragma unroll
  for (int m = LPR / 2; m > 0; m >>= 1) dot += __shfl_xor(dot, m, LPR);
  if (sub == 0) {
    p.d_t[r] = valid ? dot : 0.f;
    p.lse2_t[r] = ls;
  }
}

// ---------------------------------------------------------------------------
// dq: Q tile of NW * 32 queries, KV tiles of KVT keys.  GQ: q, dout, out
// and lse are read in grid order and D_i is formed here from the dout and
// out rows (no prep data needed); else q, dout come in tile order with the
// prep kernel's lse2 / D.
template <int D, int NW, int KVT, bool GQ>
__global__ __launch_bounds__(NW * 64, 8 / NW) void bwd_dq_kernel(BwdParams bp) {
  const KParams& p = bp.kp;
  constexpr int QT = NW * 32;
  constexpr int DC = D / 16;
  constexpr int DB = D / 32;
  constexpr int KB = KVT / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = KVT * D * 2;
  constexpr int STAGE = 2 * TILEB;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
  lds_u8* lds = (lds_u8*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), hh = lane >> 5, lq = lane & 31;
  const WorkItem wi = decode_work(p, blockIdx.x);
  const size_t qtile = (size_t)wi.bh * p.nQ + wi.qrow;
  const int row = wv * 32 + lq;
  const size_t slot = qtile * QT + row;

  const Coord3 qc = slot_coord(row, wi.a0, wi.a1, wi.a2, p.lq0, p.lq1, p.lq2);
  const int st0 = dev_window_start(qc.t, p.L0, p.w0, p.s0);
  const int st1 = dev_window_start(qc.y, p.L1, p.w1, p.s1);
  const int st2 = dev_window_start(qc.x, p.L2, p.w2, p.s2);
  const bool q_valid = qc.t < p.L0 && qc.y < p.L1 && qc.x < p.L2;

  // q and dO rows of this lane's query (B operands), its statistics
  const int bb = wi.bh / p.heads, hd = wi.bh % p.heads;
  const size_t tok = ((size_t)min(qc.t, p.L0 - 1) * p.L1 + min(qc.y, p.L1 - 1)) * p.L2 + min(qc.x, p.L2 - 1);
  const size_t grow = ((size_t)bb * p.L0 * p.L1 * p.L2 + tok) * p.heads + hd;   // grid-order row (clamped)
  bf16x8 qr[DC], dr[DC];
  float lse2, dd;
  {
    const size_t r = GQ ? grow : slot;
    const bf16x8* qs = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(GQ ? bp.q : p.qt) + r * D);
    const bf16x8* ds = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(GQ ? bp.dout : bp.dot) + r * D);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      qr[c] = qs[2 * c + hh];
      dr[c] = ds[2 * c + hh];
    }
    if constexpr (GQ) {
      // D_i = <dout_i, out_i>: this lane half holds 64 (or 32) of the dims
      const bf16x8* os = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(bp.out) + r * D);
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 o = os[2 * c + hh];
#pragma unroll
        for (int j = 0; j < 8; ++j) part = fmaf((float)dr[c][j], (float)o[j], part);
      }
      dd = xhalf_sum(part);
      lse2 = bp.lse[r] * kLog2e;
    } else {
      lse2 = bp.lse2_t[slot];
      dd = bp.d_t[slot];
    }
  }
  const float c2 = p.c2;

  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x16{};

  typedef const __attribute__((address_space(4))) int32_t cint;
  cint* qptr = (cint*)p.qptr;
  cint* kv_idx = (cint*)p.kv_idx;
  const int qrow_u = __builtin_amdgcn_readfirstlane(wi.qrow);
  const int beg = __builtin_amdgcn_readfirstlane(qptr[qrow_u]);
  const int end = __builtin_amdgcn_readfirstlane(qptr[qrow_u + 1]);
  const int nfull = __builtin_amdgcn_readfirstlane(((cint*)p.n_full)[qrow_u]);
  const unsigned char* kbase = static_cast<const unsigned char*>(p.kt) + (size_t)wi.bh * p.nK * TILEB;
  const unsigned char* vbase = static_cast<const unsigned char*>(p.vt) + (size_t)wi.bh * p.nK * TILEB;
  const int km2 = (1 << p.lk2) - 1, km1 = (1 << p.lk1) - 1, ksh = p.lk1 + p.lk2;
  const unsigned koff = dma_lane_offset<ROWB, NW>(wv, lane);
  const int krow0 = kperm(lq);
  const int kswz = swz<ROWB / 16>(krow0);

  if (beg < end) {
    const int kv0 = kv_idx[beg];
    tile_to_lds<TILEB, NW>(kbase + (size_t)kv0 * TILEB, koff, lds, wv);
    tile_to_lds<TILEB, NW>(vbase + (size_t)kv0 * TILEB, koff, lds + TILEB, wv);
  }

  // The restrict qualifiers state that the stage read (Ks, Vs) and the stage
  // the next copy writes (nb) never overlap, so the compiler issues no wait on
  // the in-flight copy before the transposing reads of K.
  auto tile_body = [&](const unsigned char* __restrict__ Ks, const unsigned char* __restrict__ Vs,
                       lds_u8* __restrict__ nb, const unsigned char* nk, const unsigned char* nv, bool copy,
                       uint64_t vmask, auto bnd) {
    constexpr bool BOUNDARY = decltype(bnd)::value;
    if (copy) {
      tile_to_lds<TILEB, NW>(nk, koff, nb, wv);
      tile_to_lds<TILEB, NW>(nv, koff, nb + TILEB, wv);
    }
    // 8-wave tiles keep the block loop rolled: two waves per SIMD leave 256
    // registers, and unrolling hoists operand reads past that
#pragma unroll(GQ ? 1 : KB)
    for (int kb = 0; kb < KB; ++kb) {
      __builtin_amdgcn_iglp_opt(1);   // LLVM's single-wave MFMA / LDS-read interleaving
      f32x16 s = qk_block<D, ROWB>(Ks, kb, krow0, kswz, hh, qr);
      const f32x16 dp = qk_block<D, ROWB>(Vs, kb, krow0, kswz, hh, dr);
      if constexpr (BOUNDARY) apply_mask(s, vmask, kb);
      bf16x8 dsv[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lse2));
        dsv[i >> 3][i & 7] = (__bf16)(pr * (dp[i] - dd));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int d = 0; d < DB; ++d)
          acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand_tr<D>(Ks, 32 * kb + 16 * c, d, lane), dsv[c],
                                                           acc[d], 0, 0, 0);
    }
  };

  // One loop over the full tiles, then one over the boundary tiles, so each
  // keeps its own registers (a branch between the two inside one loop made
  // the compiler spill the values live across it on every tile).
  auto run_tile = [&](int j, auto bnd) {
    constexpr bool BOUNDARY = decltype(bnd)::value;
    const int stage = (j - beg) & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool copy = j + 1 < end;
    const int kvn = copy ? kv_idx[j + 1] : 0;
    const unsigned char* Ks = smem + stage * STAGE;
    lds_u8* nb = lds + (stage ^ 1) * STAGE;
    const unsigned char* nk = kbase + (size_t)kvn * TILEB;
    const unsigned char* nv = vbase + (size_t)kvn * TILEB;
    uint64_t vmask = 0;
    if constexpr (BOUNDARY) {
      const int kv = kv_idx[j];
      const int k2 = (kv % p.nk2) << p.lk2;
      const int k1 = ((kv / p.nk2) % p.nk1) << p.lk1;
      const int k0 = (kv / (p.nk2 * p.nk1)) << p.lk0;
      vmask = boundary_mask<KVT / 16>([&](int gg) { return 8 * (2 * gg + hh); }, k0, k1, k2, st0, st1, st2, p.w0,
                                      p.w1, p.w2, p.lk2, km1, km2, ksh);
    }
    tile_body(Ks, Ks + TILEB, nb, nk, nv, copy, vmask, bnd);
  };
  const int jfull = beg + nfull;
  for (int j = beg; j < jfull; ++j) run_tile(j, std::integral_constant<bool, false>{});
  for (int j = jfull; j < end; ++j) run_tile(j, std::integral_constant<bool, true>{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (!q_valid) return;
  __bf16* orow = static_cast<__bf16*>(bp.dq) + grow * D;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[d][4 * g + e] * p.scale);
      *reinterpret_cast<bf16x4*>(orow + d * 32 + 8 * g + 4 * hh) = v;
    }
}

// ---------------------------------------------------------------------------
// dkdv: KV tile of NW * 32 keys, Q tiles of QTT queries.

// Queries whose window holds coordinate c along one axis: [lo, lo + n) (the
// window start is non-decreasing in the query coordinate).
__device__ __forceinline__ void query_interval(int c, int L, int w, int s, int& lo, int& n) {
  // first query whose window ends after c
  int a = 0, b = L;
  while (a < b) {
    const int m = (a + b) >> 1;
    if (dev_window_start(m, L, w, s) + w - 1 >= c) b = m; else a = m + 1;
  }
  lo = a;
  // one past the last query whose window starts at or before c
  a = lo;
  b = L;
  while (a < b) {
    const int m = (a + b) >> 1;
    if (dev_window_start(m, L, w, s) <= c) a = m + 1; else b = m;
  }
  n = a - lo;
  if (n < 0) n = 0;
}

// What one wave of the dk/dv kernel does for its 32 keys: both gradients
// (one wave per 32 keys), or one of them (two waves per 32 keys on one SIMD).
// In the split the dV wave forms S and P = exp(S - lse) and passes P (bf16)
// to its dK partner through LDS, so S is computed once; the dK wave forms
// dP, dS = P (dP - D) and dK.  The split halves the registers a wave holds,
// so two waves share each SIMD, and pairs the dV wave's exponentials with
// the dK wave's dP product and the dK wave's dS arithmetic with the dV
// product.  dS is formed from the bf16 P the PV product uses in all forms.
enum DkdvRole { kBothKV = 0, kOnlyK = 1, kOnlyV = 2 };

// One wave's share of a dk/dv workgroup: the NW waves of the workgroup copy
// the Q-side tiles together; this wave owns keys kw * 32 .. kw * 32 + 31 of
// the KW * 32-key tile.  px: the split's P exchange, [2 slots][KW][2][64
// lanes] x 16 bytes.
template <int D, int NW, int KW, int QTT, int ROLE>
__device__ __forceinline__ void dkdv_wave(const BwdParams& bp, unsigned char* smem, unsigned char* px, int kw, int wv,
                                          int lane) {
  const KParams& p = bp.kp;
  constexpr bool DOK = ROLE != kOnlyV, DOV = ROLE != kOnlyK;
  constexpr bool NEED_K = ROLE != kOnlyK, NEED_V = ROLE != kOnlyV;   // k rows (for S), v rows (for dP)
  constexpr int KT = KW * 32;           // keys per workgroup (the KV tile)
  constexpr int DC = D / 16;
  constexpr int DB = D / 32;
  constexpr int QB = QTT / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = QTT * D * 2;    // one Q (or dO) tile
  constexpr int STATB = QTT * 4;        // lse or D of one Q tile
  constexpr int STAGE = 2 * TILEB + 2 * STATB;
  static_assert(QTT * 4 <= 64 * 16, "statistics copy is one wave instruction");
  lds_u8* lds = (lds_u8*)smem;
  const int hh = lane >> 5, lq = lane & 31;

  // work item: (batch * heads, KV tile), KV tiles with T fastest, XCD remap
  const int n_wg = p.num_wg;
  int bh, c0, c1, c2;
  {
    const int nx = 8;
    const int q = n_wg / nx, r = n_wg % nx;
    const int x = blockIdx.x % nx, loc = blockIdx.x / nx;
    const int logical = x < r ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
    bh = logical / p.nK;
    const int t = logical % p.nK;
    const int nk0 = p.nK / (p.nk1 * p.nk2);
    c0 = t % nk0;
    const int rest = t / nk0;
    c2 = rest % p.nk2;
    c1 = rest / p.nk2;
  }
  const int kvrow = (c0 * p.nk1 + c1) * p.nk2 + c2;
  const size_t ktile = (size_t)bh * p.nK + kvrow;
  const int row = kw * 32 + lq;
  const Coord3 kc = slot_coord(row, c0, c1, c2, p.lk0, p.lk1, p.lk2);
  const bool k_valid = kc.t < p.L0 && kc.y < p.L1 && kc.x < p.L2;
  int ql0 = 0, qn0 = 0, ql1 = 0, qn1 = 0, ql2 = 0, qn2 = 0;
  if constexpr (NEED_K) {   // the mask belongs to the wave that forms P
    query_interval(kc.t, p.L0, p.w0, p.s0, ql0, qn0);
    query_interval(kc.y, p.L1, p.w1, p.s1, ql1, qn1);
    query_interval(kc.x, p.L2, p.w2, p.s2, ql2, qn2);
  }

  bf16x8 kr[NEED_K ? DC : 1], vr[NEED_V ? DC : 1];
  {
    const size_t slot = ktile * KT + row;
    const bf16x8* ks = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.kt) + slot * D);
    const bf16x8* vs = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.vt) + slot * D);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      if constexpr (NEED_K) kr[c] = ks[2 * c + hh];
      if constexpr (NEED_V) vr[c] = vs[2 * c + hh];
    }
  }
  const float c2s = p.c2;

  f32x16 ak[DOK ? DB : 1], av[DOV ? DB : 1];
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    if constexpr (DOK) ak[d] = f32x16{};
    if constexpr (DOV) av[d] = f32x16{};
  }

  typedef const __attribute__((address_space(4))) int32_t cint;
  cint* tptr = (cint*)bp.tqptr;
  cint* tidx = (cint*)bp.tq_idx;
  const int krow_u = __builtin_amdgcn_readfirstlane(kvrow);
  const int beg = __builtin_amdgcn_readfirstlane(tptr[krow_u]);
  const int end = __builtin_amdgcn_readfirstlane(tptr[krow_u + 1]);
  const int nfull = __builtin_amdgcn_readfirstlane(((cint*)bp.tn_full)[krow_u]);
  const size_t qtiles_bh = (size_t)bh * p.nQ;
  const unsigned char* qbase = static_cast<const unsigned char*>(p.qt) + qtiles_bh * TILEB;
  const unsigned char* dbase = static_cast<const unsigned char*>(bp.dot) + qtiles_bh * TILEB;
  const unsigned char* lbase = reinterpret_cast<const unsigned char*>(bp.lse2_t) + qtiles_bh * STATB;
  const unsigned char* sbase = reinterpret_cast<const unsigned char*>(bp.d_t) + qtiles_bh * STATB;
  const int qm2 = (1 << p.lq2) - 1, qm1 = (1 << p.lq1) - 1, qsh = p.lq1 + p.lq2;
  const unsigned qoff = dma_lane_offset<ROWB, NW>(wv, lane);
  const int qrow0 = kperm(lq);
  const int qswz = swz<ROWB / 16>(qrow0);

  // copy of one Q tile's rows, dO rows and statistics into a stage (all NW
  // waves of the workgroup take part)
  auto copy_tile = [&](int a, lds_u8* st) {
    tile_to_lds<TILEB, NW>(qbase + (size_t)a * TILEB, qoff, st, wv);
    tile_to_lds<TILEB, NW>(dbase + (size_t)a * TILEB, qoff, st + TILEB, wv);
    if (wv < 2 && lane * 16 < STATB) {
      const unsigned char* src = (wv == 0 ? lbase : sbase) + (size_t)a * STATB + lane * 16;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(st + 2 * TILEB + wv * STATB), 16,
                                       0, 0);
    }
  };
  if (beg < end) copy_tile(tidx[beg], lds);

  auto tile_body = [&](const unsigned char* __restrict__ Qs, const unsigned char* __restrict__ Ds,
                       const float* __restrict__ Ls, const float* __restrict__ Ss, lds_u8* __restrict__ nb, int an,
                       bool copy, uint64_t vmask, auto bnd) {
    constexpr bool BOUNDARY = decltype(bnd)::value;
    if (copy) copy_tile(an, nb);
    // a split wave has half the registers: keep the query blocks rolled
#pragma unroll(ROLE == kBothKV ? QB : 1)
    for (int qb = 0; qb < QB; ++qb) {
      __builtin_amdgcn_iglp_opt(1);   // LLVM's single-wave MFMA / LDS-read interleaving (2.6 % faster)
      // this wave pair's P slot of the block: [c][lane], 16 bytes each
      bf16x8* pslot = reinterpret_cast<bf16x8*>(px + ((qb & 1) * KW + kw) * 2048) + lane;
      bf16x8 pv[2];
      f32x16 dp;
      if constexpr (DOK) dp = qk_block<D, ROWB>(Ds, qb, qrow0, qswz, hh, vr);
      if constexpr (NEED_K) {
        f32x16 s = qk_block<D, ROWB>(Qs, qb, qrow0, qswz, hh, kr);
        if constexpr (BOUNDARY) apply_mask(s, vmask, qb);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          // accumulators 8c .. 8c+7 hold queries 32 qb + 16 c + 8 hh + 0..7
          const int q0 = 32 * qb + 16 * c + 8 * hh;
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[c][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[8 * c + e], c2s, -Ls[q0 + e]));
        }
      }
      if constexpr (ROLE == kOnlyV) {
        pslot[0] = pv[0];
        pslot[64] = pv[1];
      }
      if constexpr (ROLE != kBothKV) __syncthreads();   // the pair's P of this block is in LDS
      if constexpr (ROLE == kOnlyK) {
        pv[0] = pslot[0];
        pv[1] = pslot[64];
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 dsv;
        if constexpr (DOK) {
          const int q0 = 32 * qb + 16 * c + 8 * hh;
#pragma unroll
          for (int e = 0; e < 8; ++e) dsv[e] = (__bf16)((float)pv[c][e] * (dp[8 * c + e] - Ss[q0 + e]));
        }
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          if constexpr (DOV)
            av[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand_tr<D>(Ds, 32 * qb + 16 * c, d, lane), pv[c],
                                                            av[d], 0, 0, 0);
          if constexpr (DOK)
            ak[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand_tr<D>(Qs, 32 * qb + 16 * c, d, lane), dsv,
                                                            ak[d], 0, 0, 0);
        }
      }
    }
  };

  for (int j = beg; j < end; ++j) {
    const int stage = (j - beg) & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool copy = j + 1 < end;
    const int an = copy ? tidx[j + 1] : 0;
    const int a = tidx[j];
    const unsigned char* Qs = smem + stage * STAGE;
    const float* Ls = reinterpret_cast<const float*>(Qs + 2 * TILEB);
    const float* Ss = Ls + QTT;
    lds_u8* nb = lds + (stage ^ 1) * STAGE;
    if (!NEED_K || j < beg + nfull) {   // the dK wave of a split takes masked P from its partner
      tile_body(Qs, Qs + TILEB, Ls, Ss, nb, an, copy, 0ull, std::integral_constant<bool, false>{});
    } else {
      const int a2 = a % p.nq2, a1 = (a / p.nq2) % p.nq1, a0 = a / (p.nq2 * p.nq1);
      const uint64_t vmask =
          boundary_mask<QTT / 16>([&](int gg) { return 8 * (2 * gg + hh); }, a0 << p.lq0, a1 << p.lq1, a2 << p.lq2, ql0,
                                  ql1, ql2, qn0, qn1, qn2, p.lq2, qm1, qm2, qsh);
      tile_body(Qs, Qs + TILEB, Ls, Ss, nb, an, copy, vmask, std::integral_constant<bool, true>{});
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (!k_valid) return;
  const int bb = bh / p.heads, hd = bh % p.heads;
  const size_t tok = ((size_t)kc.t * p.L1 + kc.y) * p.L2 + kc.x;
  const size_t goff = (((size_t)bb * p.L0 * p.L1 * p.L2 + tok) * p.heads + hd) * D;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (DOK) {
        bf16x4 kv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) kv4[e] = (__bf16)(ak[d][4 * g + e] * p.scale);
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(bp.dk) + goff + d * 32 + 8 * g + 4 * hh) = kv4;
      }
      if constexpr (DOV) {
        bf16x4 vv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) vv4[e] = (__bf16)av[d][4 * g + e];
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(bp.dv) + goff + d * 32 + 8 * g + 4 * hh) = vv4;
      }
    }
}

// SPLIT: 2 KW waves, one dK wave and one dV wave per 32 keys (waves w and
// w + KW share keys; the hardware places them on the same SIMD); else KW = NW
// waves doing both.
template <int D, int NW, int QTT, bool SPLIT>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv_kernel(BwdParams bp) {
  constexpr int KW = SPLIT ? NW / 2 : NW;
  constexpr int STAGE = 2 * (QTT * D * 2) + 2 * (QTT * 4);
  constexpr int PX = SPLIT ? 2 * KW * 2048 : 0;      // P exchange of the split
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE + PX];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (SPLIT) {
    if (wv < KW)
      dkdv_wave<D, NW, KW, QTT, kOnlyK>(bp, smem, smem + 2 * STAGE, wv, wv, lane);
    else
      dkdv_wave<D, NW, KW, QTT, kOnlyV>(bp, smem, smem + 2 * STAGE, wv - KW, wv, lane);
  } else {
    dkdv_wave<D, NW, KW, QTT, kBothKV>(bp, smem, nullptr, wv, wv, lane);
  }
}

}  // namespace

bool attn_bwd_supported(int head_dim, int q_tokens, int kv_tokens) {
  return (head_dim == 64 || head_dim == 128) && q_tokens == 128 && kv_tokens == 128;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
  const int qtok = a.attn.tq[0] * a.attn.tq[1] * a.attn.tq[2];
  const int ktok = a.attn.tkv[0] * a.attn.tkv[1] * a.attn.tkv[2];
  const int dq_q = a.dq_attn.tq[0] * a.dq_attn.tq[1] * a.dq_attn.tq[2];
  if (!attn_bwd_supported(a.attn.head_dim, qtok, ktok) || a.attn.tq[2] < 8 || a.attn.tkv[2] < 8 ||
      (dq_q != 128 && dq_q != 256))
    return hipErrorInvalidValue;
  for (int d = 0; d < 3; ++d)
    if (a.dq_attn.tkv[d] != a.attn.tkv[d] || (dq_q == 128 && a.dq_attn.tq[d] != a.attn.tq[d]))
      return hipErrorInvalidValue;   // the dq kernel shares the tile-order k, v (and, at 128, q, dout)
  BwdParams p;
  p.kp = make_kparams(a.attn);
  p.dot = a.dot;
  p.out = a.out;
  p.dout = a.dout;
  p.lse = a.lse;
  p.lse2_t = a.lse2_t;
  p.d_t = a.d_t;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.tqptr = a.tqptr;
  p.tq_idx = a.tq_idx;
  p.tn_full = a.tn_full;
  p.q = a.q;
  const int64_t rows = (int64_t)p.kp.num_wg * qtok;
  const bool d128 = a.attn.head_dim == 128;
  const int rpb = 256 / (a.attn.head_dim / 8);
  const unsigned prep_blocks = (unsigned)((rows + rpb - 1) / rpb);
  if (d128)
    bwd_prep_kernel<128><<<prep_blocks, 256, 0, st>>>(p);
  else
    bwd_prep_kernel<64><<<prep_blocks, 256, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dq: over its own tile map (dq_attn); 256-query tiles read grid order
  BwdParams pq = p;
  pq.kp = make_kparams(a.dq_attn);
  const int dq_qtok = a.dq_attn.tq[0] * a.dq_attn.tq[1] * a.dq_attn.tq[2];
  if (dq_qtok == 256) {
    if (d128)
      bwd_dq_kernel<128, 8, 128, true><<<pq.kp.num_wg, 512, 0, st>>>(pq);
    else
      bwd_dq_kernel<64, 8, 128, true><<<pq.kp.num_wg, 512, 0, st>>>(pq);
  } else {
    if (d128)
      bwd_dq_kernel<128, 4, 128, false><<<pq.kp.num_wg, 256, 0, st>>>(pq);
    else
      bwd_dq_kernel<64, 4, 128, false><<<pq.kp.num_wg, 256, 0, st>>>(pq);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  BwdParams pk = p;
  pk.kp.num_wg = a.attn.batch * a.attn.heads * p.kp.nK;
  const char* e_split = std::getenv("NA_DKDV_SPLIT");
  const bool split = !(e_split && e_split[0] == '0');
  if (split) {
    if (d128)
      bwd_dkdv_kernel<128, 8, 128, true><<<pk.kp.num_wg, 512, 0, st>>>(pk);
    else
      bwd_dkdv_kernel<64, 8, 128, true><<<pk.kp.num_wg, 512, 0, st>>>(pk);
  } else {
    if (d128)
      bwd_dkdv_kernel<128, 4, 128, false><<<pk.kp.num_wg, 256, 0, st>>>(pk);
    else
      bwd_dkdv_kernel<64, 4, 128, false><<<pk.kp.num_wg, 256, 0, st>>>(pk);
  }
  return hipGetLastError();
}

}  // namespace na
