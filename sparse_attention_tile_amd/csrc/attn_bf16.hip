// bf16 GNA attention forward on gfx950 matrix cores.
//
// What it computes (GNA page, "GNA Sparse Attention Mechanism:
// Vision-Transformer Compute Optimisation in Practice", sections 1.1 and
// 2.1): for every Q tile, loop over the KV tiles its tile-map row lists;
// S = scale * Q K^T on bf16 MFMA with fp32 accumulation; a fine-grained
// window mask only on boundary tiles; online softmax in fp32 (SLA page,
// "Sparse attention in video and image generation: optimisation practice",
// section 3.1 keeps softmax in FP32; tutorial "Video-generation inference
// speed-up: sparse attention configuration tutorial", section 3.3 the
// block-wise normalisation); O += P V on bf16 MFMA; out = O / l and
// lse = m + ln l.
//
// gfx950 mapping
// * Two wavefronts per SIMD, 32 queries per wavefront, NW wavefronts per
//   workgroup (Q tile = 32 NW queries).  While one wave of a SIMD runs its
//   softmax on the VALU, the other keeps the matrix core busy; each wave
//   holds its Q operand and its O accumulators in registers for the whole
//   kernel.
// * The transposed products are used: S^T = K Q^T and O^T = V^T P^T on
//   v_mfma_f32_32x32x16_bf16.  In the C layout of S^T a lane holds one query
//   and 16 keys: the lazy-rescale test compares each lane half's block
//   maximum with the running one, the cross-half exchange
//   (v_permlane32_swap) runs only when a rescale happens, and the row sum
//   stays in-lane.  K rows are fed to
//   the MFMA in a permuted order so that those 16 accumulators come out as
//   two runs of 8 consecutive keys, which is exactly the B-operand layout of
//   the P V product: P goes from registers to the next MFMA with no LDS trip.
// * V arrives transposed per tile ([D][tile tokens], done by the permutation
//   kernel), so the A operand of O^T is one 16-byte LDS read per lane.
// * K and V^T tiles stream HBM -> LDS with global_load_lds_dwordx4 (no
//   register staging) into a double buffer: tile j+1 is in flight while tile
//   j is multiplied.  A 16-byte-chunk XOR swizzle, applied through the
//   per-lane global addresses of those loads, keeps the MFMA operand reads
//   free of LDS bank conflicts.
// * Lazy rescaling: the running max only moves when a block max exceeds it
//   by more than 2^8 (after exp2), so O is rescaled almost never after the
//   first block; P stays <= 256.  Results equal exact-max softmax up to
//   rounding.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_common.hpp"
#include "attn_device.hpp"

namespace na {
namespace {

// Lazy rescaling: move the reference max m only when the block max exceeds
// it by more than thr (= 8 / c2, a factor 2^8 after exp2); then scale l and
// O by exp2((m_old - m_new) c2) and update the exponent offset nref = -m c2
// (kept with m rather than recomputed per block).  The branch is
// wave-uniform and rare.
template <int DB>
__device__ __forceinline__ void rescale_if_needed(const f32x16& s, float& m, float& nref, float& l, f32x16 (&o)[DB],
                                                  float c2, float thr) {
  // one serial chain of three-input maxima (v_max3_f32: 8 instructions)
  float bm = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) bm = fmaxf(fmaxf(bm, s[i]), s[i + 1]);
  bm = fmaxf(bm, s[15]);
  // m is the same in both lane halves (one query), so testing each half's
  // maximum decides the branch as the full row maximum would; the exchange
  // between the halves is only needed inside it
  if (__builtin_amdgcn_ballot_w64(bm > m + thr)) {
    bm = xhalf_max(bm);
    const float mn = fmaxf(m, bm);
    // alpha = 0 while nothing was accumulated (O and l are still 0)
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mn) * c2);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] *= alpha;
    m = mn;
    nref = mn == -INFINITY ? 0.f : -mn * c2;
  }
}

// Tensor layouts (IO mode, a template parameter of the kernel):
//  IO_TILE: q, k, v, out, lse in tile order (na_permute output; V transposed
//           per tile).
//  IO_QO:   q, out, lse are the caller's grid-order tensors (each query row is
//           read and written in place), k and v in tile order.
//  IO_GRID: all five in grid order; K / V tiles are gathered token by token
//           (the LDS-DMA takes one source address per lane), V stays [key][d]
//           in LDS and its PV operand is read with the transposing LDS load --
//           no permutation pass and no workspace at all.
// Copy step kb of a tile whose per-round source offsets (from base) are off[].
template <int TILEB, int NW, int KB, int ROUNDS>
__device__ __forceinline__ void tile_to_lds_step_off(const unsigned char* __restrict__ base,
                                                     const int64_t (&off)[ROUNDS], lds_u8* lds, int wv, int kb) {
  constexpr int ROUND = 1024 * NW;
  static_assert(TILEB / ROUND == ROUNDS, "one offset per copy round");
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i)
    if ((i * KB) / ROUNDS == kb)
      __builtin_amdgcn_global_load_lds(base + off[i],
                                       (__attribute__((address_space(3))) void*)(lds + i * ROUND + wv * 1024), 16, 0,
                                       0);
}

// PAIRED (k, v in tile order, 8 waves): the KV tiles in memory hold 64 keys
// and two consecutive entries of a tile-map row are copied into one 128-key
// LDS tile (K rows 0..63 from the first, 64..127 from the second; each V^T
// row's first and second halves likewise), so the 128-key pipeline runs with
// one barrier per 128 keys.  A pair is full when both of its tiles are; an
// odd row ends with a single tile whose second half is masked.
template <int D, int NW, int KVT, int IO, bool PAIRED>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_bf16_kernel(KParams p) {
  constexpr bool GQ = IO != IO_TILE;     // q, out, lse in grid order
  constexpr bool GKV = IO == IO_GRID;    // k, v in grid order
  static_assert(!PAIRED || (KVT == 128 && !GKV), "pairs of 64-key tiles in tile order make a 128-key LDS tile");
  constexpr int QT = NW * 32;            // queries per workgroup
  constexpr int DC = D / 16;             // k-steps of S^T
  constexpr int DB = D / 32;             // 32-row blocks of O^T
  constexpr int KB = KVT / 32;           // 32-key blocks per KV tile
  constexpr int KROW = D * 2;            // bytes per K row
  constexpr int VROW = GKV ? D * 2 : KVT * 2;    // bytes per V row (GKV) or V^T row
  constexpr int TILEB = KVT * D * 2;     // bytes of one K (or V) tile in LDS
  constexpr int MTILEB = PAIRED ? TILEB / 2 : TILEB;   // bytes of one K (or V^T) tile in memory
  constexpr int TSTEP = PAIRED ? 2 : 1;  // tile-map entries per LDS tile
  constexpr int ROUNDS = TILEB / (1024 * NW);    // copy rounds per tile
  constexpr int STAGE = 2 * TILEB;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
  lds_u8* lds = (lds_u8*)smem;

  const int tid = threadIdx.x;
  // wv is wave-uniform: keeping it in a scalar register lets the LDS-DMA
  // destination (M0) be computed with scalar arithmetic
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), hh = lane >> 5, lq = lane & 31;
  const WorkItem wi = decode_work(p, blockIdx.x);
  const size_t qtile = (size_t)wi.bh * p.nQ + wi.qrow;
  const int row = wv * 32 + lq;          // this lane's query inside the Q tile

  // this query's grid position and window on each axis (for boundary tiles),
  // and whether the wave holds any real query: a wave whose 32 slots are all
  // padding (ragged grid edge) skips the arithmetic and only helps with the
  // tile copies
  int st0, st1, st2;
  bool wave_active, q_valid;
  int q_tok;                             // grid token of the query (clamped inside the grid)
  {
    const int px = row & ((1 << p.lq2) - 1);
    const int py = (row >> p.lq2) & ((1 << p.lq1) - 1);
    const int pt = row >> (p.lq1 + p.lq2);
    const int gt = (wi.a0 << p.lq0) + pt, gy = (wi.a1 << p.lq1) + py, gx = (wi.a2 << p.lq2) + px;
    st0 = dev_window_start(gt, p.L0, p.w0, p.s0);
    st1 = dev_window_start(gy, p.L1, p.w1, p.s1);
    st2 = dev_window_start(gx, p.L2, p.w2, p.s2);
    q_valid = gt < p.L0 && gy < p.L1 && gx < p.L2;
    wave_active = __builtin_amdgcn_ballot_w64(q_valid) != 0;
    q_tok = (min(gt, p.L0 - 1) * p.L1 + min(gy, p.L1 - 1)) * p.L2 + min(gx, p.L2 - 1);
  }
  // grid-order element offset of token 0 of this (batch, head), and the
  // element stride between tokens
  const int bb = wi.bh / p.heads, hd = wi.bh % p.heads;
  const size_t grid_base = ((size_t)bb * p.L0 * p.L1 * p.L2 * p.heads + hd) * D;
  const size_t tok_stride = (size_t)p.heads * D;

  // ---- Q operand (B of S^T = K Q^T): query = lane % 32, 8 dims per lane
  bf16x8 qr[DC];
  {
    const __bf16* qrow = static_cast<const __bf16*>(p.qt) +
                         (GQ ? grid_base + (size_t)q_tok * tok_stride : (qtile * QT + row) * D);
    const bf16x8* src = reinterpret_cast<const bf16x8*>(qrow);
#pragma unroll
    for (int c = 0; c < DC; ++c) qr[c] = src[2 * c + hh];
  }

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x16{};
  float m = -INFINITY, l = 0.f;
  float nref = 0.f;   // -m c2 (0 while every key so far is masked: then p = 0)

  // The tile map is read-only for the whole launch: read it through the
  // constant address space so the loads are scalar (s_load, lgkmcnt) and never
  // wait on the vector-memory counter the K/V DMA uses.
  typedef const __attribute__((address_space(4))) int32_t cint;
  cint* qptr = (cint*)p.qptr;
  cint* kv_idx = (cint*)p.kv_idx;
  const int qrow_u = __builtin_amdgcn_readfirstlane(wi.qrow);
  const int bh_u = __builtin_amdgcn_readfirstlane(wi.bh);
  const int kvo = (int)(bh_u * p.map_bh_kv);     // per-(batch, head) maps (else 0)
  const int beg = __builtin_amdgcn_readfirstlane(qptr[qrow_u]) + kvo;
  const int end = __builtin_amdgcn_readfirstlane(qptr[qrow_u + 1]) + kvo;
  const int nfull = __builtin_amdgcn_readfirstlane(((cint*)p.n_full)[qrow_u + bh_u * p.map_bh_nf]);
  const unsigned char* kbase = static_cast<const unsigned char*>(p.kt) + (GKV ? grid_base * 2 : (size_t)wi.bh * p.nK * MTILEB);
  const unsigned char* vbase = static_cast<const unsigned char*>(p.vt) + (GKV ? grid_base * 2 : (size_t)wi.bh * p.nK * MTILEB);
  const float c2 = p.c2;
  const int km2 = (1 << p.lk2) - 1, km1 = (1 << p.lk1) - 1, ksh = p.lk1 + p.lk2;
  static_assert(KVT / 16 <= 8, "validity mask holds 64 bits");
  const int koff = dma_lane_offset<KROW, NW>(wv, lane);
  const int voff = dma_lane_offset<VROW, NW>(wv, lane);
  // the reference max moves only when a block max exceeds it by 8 / c2
  const float thr = c2 > 0.f ? 8.f / c2 : 3.0e38f;
  // K row this lane feeds to the MFMA, and its swizzle (same in every block)
  const int krow0 = kperm(lq);
  const int kswz = swz<KROW / 16>(krow0);
  const int vswz = swz<VROW / 16>(lq);

  // GKV: the token each lane copies in copy round i sits at in-tile slot
  // dslot[i]; its byte offset from the (batch, head) base depends on the tile
  // and is computed per tile in grid_offsets (padding slots are clamped to a
  // real token: finite data that the mask multiplies by zero).
  int dslot[ROUNDS > 0 ? ROUNDS : 1];
  int64_t goff[ROUNDS > 0 ? ROUNDS : 1];
  const int dchunk = (koff % KROW);      // byte offset of the lane's chunk inside its row
  if constexpr (GKV) {
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) dslot[i] = (i * 1024 * NW + koff) / KROW;
  }
  auto grid_offsets = [&](int kv) {
    const int o2 = (kv % p.nk2) << p.lk2;
    const int o1 = ((kv / p.nk2) % p.nk1) << p.lk1;
    const int o0 = (kv / (p.nk2 * p.nk1)) << p.lk0;
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      const int r = dslot[i];
      const int t = min(o0 + (r >> ksh), p.L0 - 1);
      const int y = min(o1 + ((r >> p.lk2) & km1), p.L1 - 1);
      const int x = min(o2 + (r & km2), p.L2 - 1);
      goff[i] = (int64_t)((t * p.L1 + y) * p.L2 + x) * (int64_t)(tok_stride * 2) + dchunk;
    }
  };

  // KV-tile indices live in scalar registers: kv_cur is tile j, kv_nxt tile
  // j+1; tile j+2's index is fetched one tile ahead so no wait on it ever
  // sits between a barrier and the next tile's DMA.
  int kv_cur = kv_idx[beg];
  int kv_nxt = beg + 1 < end ? kv_idx[beg + 1] : 0;
  // PAIRED: memory tiles of the pair being copied (nka, nva, nkb, nvb) and
  // the entries of the pair after it, fetched one pair ahead (pc0, pc1; an
  // odd row's last pair repeats its first tile, whose copy the mask drops)
  const unsigned char *nka = kbase, *nva = vbase, *nkb = kbase, *nvb = vbase;
  int pc0 = 0, pc1 = 0;
  if constexpr (PAIRED) {
    const int c1 = beg + 1 < end ? kv_nxt : kv_cur;
    nka = kbase + (size_t)kv_cur * MTILEB;
    nva = vbase + (size_t)kv_cur * MTILEB;
    nkb = kbase + (size_t)c1 * MTILEB;
    nvb = vbase + (size_t)c1 * MTILEB;
    pc0 = beg + 2 < end ? kv_idx[beg + 2] : kv_cur;
    pc1 = beg + 3 < end ? kv_idx[beg + 3] : pc0;
  }
  // PAIRED copy step kb: K rounds of the first half from tile a, the rest
  // from tile b; a V^T row's first VROW / 2 bytes from a, the rest from b
  const int vlc = (voff % VROW) / 16;    // the lane's logical V^T chunk (same every round)
  const int vrow0 = voff / VROW;
  auto pair_copy_step = [&](lds_u8* nb, int kb) {
    constexpr int ROUND = 1024 * NW;
    constexpr int HALF = VROW / 32;      // chunks per half V^T row
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      if ((i * KB) / ROUNDS != kb) continue;
      const unsigned char* ks = (i < ROUNDS / 2 ? nka : nkb) + (i % (ROUNDS / 2)) * ROUND + koff;
      const int r = vrow0 + i * (ROUND / VROW);
      const unsigned char* vs = (vlc < HALF ? nva : nvb) + r * (VROW / 2) + (vlc % HALF) * 16;
      __builtin_amdgcn_global_load_lds(ks, (__attribute__((address_space(3))) void*)(nb + i * ROUND + wv * 1024), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(
          vs, (__attribute__((address_space(3))) void*)(nb + TILEB + i * ROUND + wv * 1024), 16, 0, 0);
    }
  };
  if constexpr (GKV) {    // prologue: tile 0 in flight
    grid_offsets(kv_cur);
    for (int kb = 0; kb < KB; ++kb) {
      tile_to_lds_step_off<TILEB, NW, KB>(kbase, goff, lds, wv, kb);
      tile_to_lds_step_off<TILEB, NW, KB>(vbase, goff, lds + TILEB, wv, kb);
    }
  } else if constexpr (PAIRED) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) pair_copy_step(lds, kb);
  } else {
    tile_to_lds<TILEB, NW>(kbase + (size_t)kv_cur * TILEB, koff, lds, wv);
    tile_to_lds<TILEB, NW>(vbase + (size_t)kv_cur * TILEB, voff, lds + TILEB, wv);
  }

  // One KV tile from LDS: a software pipeline over its 32-key blocks.  S^T of
  // block kb+1 is issued before the exponentials of block kb, and the max /
  // rescale decision of block kb+1 comes after the P V product of block kb, so
  // each step offers the scheduler independent MFMA and VALU work.  BOUNDARY
  // tiles apply the key-validity mask; full tiles have no mask code at all.
  // copy of the next tile, issued step by step inside tile_body
  const unsigned char* nk = kbase;
  const unsigned char* nv = vbase;
  lds_u8* nbuf = lds;
  auto copy_step = [&](lds_u8* nb, int kb) {
    if constexpr (GKV) {
      tile_to_lds_step_off<TILEB, NW, KB>(kbase, goff, nb, wv, kb);
      tile_to_lds_step_off<TILEB, NW, KB>(vbase, goff, nb + TILEB, wv, kb);
    } else if constexpr (PAIRED) {
      pair_copy_step(nb, kb);
    } else {
      tile_to_lds_step<TILEB, NW, KB>(nk, koff, nb, wv, kb);
      tile_to_lds_step<TILEB, NW, KB>(nv, voff, nb + TILEB, wv, kb);
    }
  };
  // The restrict qualifiers state that the stage being read (Ks, Vs) and the
  // stage the next tile's copy writes (nb) never overlap; the compiler then
  // knows the in-flight copy cannot feed this tile's LDS reads and issues no
  // wait on it before them (it cannot see this for the transposing reads).
  // mask(s, kb) applies the window mask to block kb's scores (a no-op on
  // full tiles).
  auto tile_body = [&](const unsigned char* __restrict__ Ks, const unsigned char* __restrict__ Vs,
                       lds_u8* __restrict__ nb, auto&& mask) {
    f32x16 s = qk_block<D, KROW>(Ks, 0, krow0, kswz, hh, qr);
    mask(s, 0);
    rescale_if_needed(s, m, nref, l, o, c2, thr);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      // LLVM's single-wave MFMA / LDS-read interleaving strategy for this
      // scheduling region (measured 1.5 % faster than the default order)
      __builtin_amdgcn_iglp_opt(1);
      copy_step(nb, kb);
      f32x16 sn;
      if (kb + 1 < KB) sn = qk_block<D, KROW>(Ks, kb + 1, krow0, kswz, hh, qr);
      // ---- P = exp2(S c2 - m c2) in bf16; accumulator i <-> key 16*(i/8) + 8*hh + i%8
      bf16x8 pv[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) pv[i >> 3][i & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[i], c2, nref));
      // row sum of the bf16 weights the P V product uses (two dot2 chains)
      const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
      float ra = 0.f, rb = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ra = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pv[0][2 * q], pv[0][2 * q + 1]}, one2, ra, false);
        rb = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pv[1][2 * q], pv[1][2 * q + 1]}, one2, rb, false);
      }
      l += ra + rb;
      // ---- O^T += V^T P^T over the block's two 16-key halves
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          bf16x8 a;
          if constexpr (GKV) {
            a = v_operand_tr<D>(Vs, 32 * kb + 16 * c, d, lane);
          } else {
            a = *reinterpret_cast<const bf16x8*>(Vs + (d * 32 + lq) * VROW + (((4 * kb + 2 * c + hh) ^ vswz) * 16));
          }
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pv[c], o[d], 0, 0, 0);
        }
      }
      if (kb + 1 < KB) {
        mask(sn, kb + 1);
        rescale_if_needed(sn, m, nref, l, o, c2, thr);
        s = sn;
      }
    }
  };

  // Barrier for tile j and bookkeeping of the next tile's copy; returns the
  // LDS buffers holding tile j.
  auto begin_tile = [&](int j, const unsigned char*& Ks, const unsigned char*& Vs) {
    const int stage = ((j - beg) / TSTEP) & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    nbuf = lds + (stage ^ 1) * STAGE;
    int kv = kv_cur;
    if constexpr (PAIRED) {
      if (j + 2 < end) {                 // else the last pair re-copies itself (idle buffer)
        nka = kbase + (size_t)pc0 * MTILEB;
        nva = vbase + (size_t)pc0 * MTILEB;
        nkb = kbase + (size_t)pc1 * MTILEB;
        nvb = vbase + (size_t)pc1 * MTILEB;
        pc0 = j + 4 < end ? kv_idx[j + 4] : pc0;
        pc1 = j + 5 < end ? kv_idx[j + 5] : pc0;
      }
    } else {
      const int kv_copy = j + 1 < end ? kv_nxt : kv_cur;   // the last tile re-copies itself (idle buffer)
      if constexpr (GKV) {
        grid_offsets(kv_copy);
      } else {
        nk = kbase + (size_t)kv_copy * TILEB;
        nv = vbase + (size_t)kv_copy * TILEB;
      }
      kv_cur = kv_nxt;
      if (j + 2 < end) kv_nxt = kv_idx[j + 2];
    }
    Ks = smem + stage * STAGE;
    Vs = Ks + TILEB;
    return kv;
  };
  // validity mask of this lane's query over NG groups of KV tile kv (group
  // gg: keys 16 gg + 8 hh .. + 7 of the tile)
  auto kv_tile_mask = [&](int kv, auto ng) {
    constexpr int NG = decltype(ng)::value;
    const int k2 = (kv % p.nk2) << p.lk2;
    const int k1 = ((kv / p.nk2) % p.nk1) << p.lk1;
    const int k0 = (kv / (p.nk2 * p.nk1)) << p.lk0;
    return boundary_mask<NG>([&](int gg) { return 8 * (2 * gg + hh); }, k0, k1, k2, st0, st1, st2, p.w0, p.w1, p.w2,
                             p.lk2, km1, km2, ksh);
  };

  // Boundary tiles 8 or 16 keys wide along W (not paired): each 8-key group
  // a lane holds lies in one key row (t, y) of the tile, at an x offset that
  // is the same for both of the lane's groups and every block (0 for 8-wide
  // tiles, 8 hh for 16-wide ones).  So a key is inside the lane's window iff
  // its row is and its x is: the 8 x tests are made once per tile (lane
  // masks, kept in scalar registers), the row test once per group and block,
  // then one select per score.  Same masked set as boundary_mask / apply_mask.
  auto row_masker = [&](int kv) {
    const int k2 = (kv % p.nk2) << p.lk2;
    const int k1 = ((kv / p.nk2) % p.nk1) << p.lk1;
    const int k0 = (kv / (p.nk2 * p.nk1)) << p.lk0;
    const int x0 = k2 + (p.lk2 == 4 ? 8 * hh : 0) - st2;
    bool xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = (unsigned)(x0 + j) < (unsigned)p.w2;
    return [=, &p](f32x16& sc, int kb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = (32 * kb + 16 * c + 8 * hh) >> p.lk2;   // key row of accumulators 8 c .. 8 c + 7
        const bool rv = ((unsigned)(k0 + (row >> p.lk1) - st0) < (unsigned)p.w0) &
                        ((unsigned)(k1 + (row & km1) - st1) < (unsigned)p.w1);
#pragma unroll
        for (int j = 0; j < 8; ++j) sc[8 * c + j] = (rv && xv[j]) ? sc[8 * c + j] : -INFINITY;
      }
    };
  };

  // Three homogeneous loops (padding-only waves copy; full tiles; boundary
  // tiles), so the accumulators flow through simple loop phis.
  const unsigned char* Ks;
  const unsigned char* Vs;
  // LDS tiles before jfull have only full tile-map entries
  const int jfull = beg + (nfull / TSTEP) * TSTEP;
  if (!wave_active) {
    for (int j = beg; j < end; j += TSTEP) {
      begin_tile(j, Ks, Vs);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) copy_step(nbuf, kb);
    }
  } else {
    for (int j = beg; j < jfull; j += TSTEP) {
      begin_tile(j, Ks, Vs);
      tile_body(Ks, Vs, nbuf, [](f32x16&, int) {});
    }
    if (!PAIRED && !GKV && KVT == 128 && (p.lk2 == 3 || p.lk2 == 4)) {
      for (int j = jfull; j < end; j += TSTEP) {
        const int kv = begin_tile(j, Ks, Vs);
        tile_body(Ks, Vs, nbuf, row_masker(kv));
      }
    } else {
      for (int j = jfull; j < end; j += TSTEP) {
        const int kv = begin_tile(j, Ks, Vs);
        uint64_t vmask;
        if constexpr (PAIRED) {   // the two tiles' masks side by side (groups 0..3, 4..7)
          const uint64_t ma = kv_tile_mask(kv_idx[j], std::integral_constant<int, 4>{});
          const uint64_t mb = j + 1 < end ? kv_tile_mask(kv_idx[j + 1], std::integral_constant<int, 4>{}) : 0ull;
          vmask = ma | (mb << 32);
        } else {
          vmask = kv_tile_mask(kv, std::integral_constant<int, KVT / 16>{});
        }
        tile_body(Ks, Vs, nbuf, [vmask](f32x16& sc, int kb) { apply_mask(sc, vmask, kb); });
      }
    }
  }
  // the last step's copy must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: O / l in bf16, lse = m*scale + ln l
  // padding-only waves store zeros (finite, meaningless rows)
  const float lt = wave_active ? xhalf_sum(l) : 1.f;
  const float inv = 1.f / lt;
  __bf16* orow = static_cast<__bf16*>(p.ot) + (GQ ? grid_base + (size_t)q_tok * tok_stride : (qtile * QT + row) * D);
  if (GQ && !q_valid) return;            // padding rows have no place in grid order
#pragma unroll
  for (int d = 0; d < DB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v;
      v[0] = (__bf16)(o[d][4 * g + 0] * inv);
      v[1] = (__bf16)(o[d][4 * g + 1] * inv);
      v[2] = (__bf16)(o[d][4 * g + 2] * inv);
      v[3] = (__bf16)(o[d][4 * g + 3] * inv);
      *reinterpret_cast<bf16x4*>(orow + d * 32 + 8 * g + 4 * hh) = v;
    }
  }
  if (p.lse_t && hh == 0)
    p.lse_t[GQ ? (grid_base / D) + (size_t)q_tok * p.heads : qtile * QT + row] =
        (m == -INFINITY ? 0.f : m * p.scale) + logf(lt);
}

// 8-wave workgroups run 64-key tiles in tile order as pairs in a 128-key
// LDS tile (4-wave ones keep 64-key stages: two such workgroups share a CU)
template <int D, int NW, int KVT>
hipError_t launch_cfg(const KParams& p, int io, hipStream_t st) {
  constexpr bool PAIRED = KVT == 64 && NW == 8;
  constexpr int LKVT = PAIRED ? 128 : KVT;
  if (io == IO_GRID)
    attn_bf16_kernel<D, NW, KVT, IO_GRID, false><<<p.num_wg, NW * 64, 0, st>>>(p);
  else if (io == IO_QO)
    attn_bf16_kernel<D, NW, LKVT, IO_QO, PAIRED><<<p.num_wg, NW * 64, 0, st>>>(p);
  else
    attn_bf16_kernel<D, NW, LKVT, IO_TILE, PAIRED><<<p.num_wg, NW * 64, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

bool attn_bf16_supported(int head_dim, int q_tokens, int kv_tokens) {
  return (head_dim == 64 || head_dim == 128) && (q_tokens == 128 || q_tokens == 256) &&
         (kv_tokens == 64 || kv_tokens == 128);
}

// Extra shape rule of the boundary mask: the KV tile's W extent is >= 8.
bool attn_bf16_tile_ok(const int tile_kv[3]) { return tile_kv[2] >= 8; }

bool attn_bf16_grid_io_supported(int head_dim) { return head_dim == 64 || head_dim == 128; }

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st) {
  const KParams p = make_kparams(a);
  const int qtok = a.tq[0] * a.tq[1] * a.tq[2];
  const int ktok = a.tkv[0] * a.tkv[1] * a.tkv[2];
  if (!attn_bf16_supported(a.head_dim, qtok, ktok) || !attn_bf16_tile_ok(a.tkv)) return hipErrorInvalidValue;
  const int key = (a.head_dim == 128 ? 4 : 0) | (qtok == 256 ? 2 : 0) | (ktok == 128 ? 1 : 0);
  switch (key) {
    case 0: return launch_cfg<64, 4, 64>(p, a.io_mode, st);
    case 1: return launch_cfg<64, 4, 128>(p, a.io_mode, st);
    case 2: return launch_cfg<64, 8, 64>(p, a.io_mode, st);
    case 3: return launch_cfg<64, 8, 128>(p, a.io_mode, st);
    case 4: return launch_cfg<128, 4, 64>(p, a.io_mode, st);
    case 5: return launch_cfg<128, 4, 128>(p, a.io_mode, st);
    case 6: return launch_cfg<128, 8, 64>(p, a.io_mode, st);
    default: return launch_cfg<128, 8, 128>(p, a.io_mode, st);
  }
}

}  // namespace na
