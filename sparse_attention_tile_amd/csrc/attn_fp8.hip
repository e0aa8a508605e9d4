// fp8 (OCP e4m3fn) GNA attention forward on gfx950 matrix cores.
//
// Same method and workgroup structure as the bf16 kernel (GNA page, "GNA
// Sparse Attention Mechanism: Vision-Transformer Compute Optimisation in
// Practice", sections 1.1 and 2.1; the FP8 mode of section 2.1): q, k, v are
// e4m3 with per-tensor dequantisation factors (q and k factors folded into
// the softmax scale, the v factor into the epilogue); S and the softmax
// statistics are fp32 (SLA page, "Sparse attention in video and image
// generation: optimisation practice", section 3.1); the output is bf16.
//
// gfx950 mapping (differences from the bf16 kernel)
// * Both products use v_mfma_scale_f32_32x32x64_f8f6f4 with unit block
//   scales: S^T = K Q^T takes 64 head dims per instruction, O^T = V^T P^T 64
//   keys per instruction.  The k index of this instruction is any assignment
//   of (lane half, byte) to k that the A and B operands share, so each lane
//   half simply takes 32 consecutive dims (QK) or two runs of 16 consecutive
//   keys (PV).
// * K rows are fed to the QK instruction so that accumulator i of lane half h
//   is key 16 h + i of its 32-key block; two blocks then give a lane half the
//   32 P bytes its PV B operand needs, straight from registers.
// * P is stored as e4m3(64 p): the lazy-rescaling threshold is 2^2 here, so
//   64 p <= 256 stays inside e4m3's range (448) while small weights keep
//   precision.  l is computed by the matrix core from the same quantised P,
//   so O / l cancels the factor 64 exactly: a 16x16x128 product whose A
//   operand is e4m3 1.0 in the lane groups that hold the keys of the output
//   row's query and 0 elsewhere (output row r of lane group g belongs to
//   query 16 (r / 4 % 2) + column, and lane groups g and g + 2 hold the two
//   key halves of one query), so every output element of a lane is its
//   query's row sum.
// * The first conversion into each P dword takes that dword's previous
//   contents as the bytes it keeps (the second conversion overwrites them),
//   which saves zeroing it first.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_common.hpp"
#include "attn_device.hpp"

namespace na {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr float kPScaleLog2 = 6.f;   // P is stored as e4m3(2^6 p)
constexpr float kLazyLog2 = 2.f;     // reference max moves when a block max exceeds it by 2^2

// K row fed to MFMA row r of a 32-key block: r = 8 j + 4 h + t -> key
// 16 h + 4 j + t, so accumulator i of lane half h holds key 16 h + i.
__device__ __forceinline__ int kperm8(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

__device__ __forceinline__ i32x8 gload32(const unsigned char* p0, const unsigned char* p1) {
  const int4 a = *reinterpret_cast<const int4*>(p0);
  const int4 b = *reinterpret_cast<const int4*>(p1);
  return i32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // formats: 0 = e4m3 for A and B; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// GQ: q, out and lse in grid order (each lane reads and writes its query's
// row in place; padding rows read a clamped real token and store nothing),
// k and v in tile order; else all in tile order.
//
// PAIRED: the KV tiles in memory hold 64 keys, and two consecutive entries of
// a tile-map row are loaded as one 128-key LDS tile (keys 0..63 from the
// first, 64..127 from the second; a row with an odd count ends with a single
// tile whose second half is masked).  One barrier then serves 128 keys
// instead of 64.  A pair counts as full when both of its tiles are.
template <int D, int NW, int KVT, bool GQ, bool PAIRED>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_fp8_kernel(KParams p) {
  constexpr int QT = NW * 32;            // queries per workgroup
  constexpr int DS = D / 64;             // 64-dim k-steps of S^T
  constexpr int DB = D / 32;             // 32-row blocks of O^T
  constexpr int NSTEP = KVT / 64;        // 64-key steps per KV tile
  constexpr int KROW = D;                // bytes per K row
  constexpr int VROW = KVT;              // bytes per V^T row
  constexpr int TILEB = KVT * D;         // bytes of one K (or V^T) tile in LDS
  constexpr int MTILEB = PAIRED ? TILEB / 2 : TILEB;   // bytes of one K (or V^T) tile in memory
  constexpr int STAGE = 2 * TILEB;
  constexpr int KB = KVT / 32;           // copy steps per tile (one per 32-key block)
  static_assert(!PAIRED || KVT == 128, "pairs of 64-key tiles make a 128-key LDS tile");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
  lds_u8* lds = (lds_u8*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, hh = lane >> 5, lq = lane & 31;
  const WorkItem wi = decode_work(p, blockIdx.x);
  const size_t qtile = (size_t)wi.bh * p.nQ + wi.qrow;
  const int row = wv * 32 + lq;

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
  // grid-order element offset of token 0 of this (batch, head) and the
  // element stride between tokens (GQ)
  const int bb = wi.bh / p.heads, hd = wi.bh % p.heads;
  const size_t grid_base = ((size_t)bb * p.L0 * p.L1 * p.L2 * p.heads + hd) * D;
  const size_t tok_stride = (size_t)p.heads * D;

  // ---- Q operand (B of S^T): query lq, dims 64 s + 32 hh .. + 31
  i32x8 qr[DS];
  {
    const unsigned char* src = static_cast<const unsigned char*>(p.qt) +
                               (GQ ? grid_base + (size_t)q_tok * tok_stride : (qtile * QT + row) * D);
#pragma unroll
    for (int s = 0; s < DS; ++s) qr[s] = gload32(src + 64 * s + 32 * hh, src + 64 * s + 32 * hh + 16);
  }

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x16{};
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  f32x4_t osum = {};                      // every element: sum of the stored P of this lane's query
  float m = -INFINITY;
  // exponent offset of P: -m c2 + log2 of the P scale (the m term is 0 while
  // every key so far is masked); kept with m, updated when m moves
  float nref = kPScaleLog2;
  // A operand of the row-sum product (16x16x128): e4m3 1.0 where the lane
  // group holds the keys of the query this output row belongs to, else 0
  const int selv = (((lane >> 2) ^ (lane >> 4)) & 1) ? 0 : 0x38383838;
  const i32x8 sel = {selv, selv, selv, selv, selv, selv, selv, selv};
  i32x8 pb = {};

  typedef const __attribute__((address_space(4))) int32_t cint;
  const int qrow_u = __builtin_amdgcn_readfirstlane(wi.qrow);
  const int beg = __builtin_amdgcn_readfirstlane(((cint*)p.qptr)[qrow_u]);
  const int end = __builtin_amdgcn_readfirstlane(((cint*)p.qptr)[qrow_u + 1]);
  const int nfull = __builtin_amdgcn_readfirstlane(((cint*)p.n_full)[qrow_u]);
  cint* kv_idx = (cint*)p.kv_idx;
  const unsigned char* kbase = static_cast<const unsigned char*>(p.kt) + (size_t)wi.bh * p.nK * MTILEB;
  const unsigned char* vbase = static_cast<const unsigned char*>(p.vt) + (size_t)wi.bh * p.nK * MTILEB;
  const float c2 = p.c2;
  const int km2 = (1 << p.lk2) - 1, km1 = (1 << p.lk1) - 1, ksh = p.lk1 + p.lk2;
  const int koff = dma_lane_offset<KROW, NW>(wv, lane);
  const int voff = dma_lane_offset<VROW, NW>(wv, lane);
  const float thr = c2 > 0.f ? kLazyLog2 / c2 : 3.0e38f;
  const int krow0 = kperm8(lq);
  const int kswz = swz<KROW / 16>(krow0);
  const int vswz = swz<VROW / 16>(lq);

  // Copy of an LDS tile into the stage at nb, round by round; a round is
  // 1024 * NW bytes and step kb of KB issues its share.  In a pair the K
  // rounds of the first half come from tile ka, the rest from kb2; a V^T row
  // takes its first 64 bytes from va and its last 64 from vb2.
  constexpr int ROUND = 1024 * NW;
  constexpr int ROUNDS = TILEB / ROUND;
  const int vlc = (voff % VROW) / 16;                  // the lane's logical V^T chunk (same every round)
  const int vrow0 = voff / VROW;
  auto copy_step = [&](const unsigned char* ka, const unsigned char* va, const unsigned char* kb2,
                       const unsigned char* vb2, lds_u8* nb, int kb) {
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      if ((i * KB) / ROUNDS != kb) continue;
      const unsigned char* ks;
      const unsigned char* vs;
      if constexpr (PAIRED) {
        ks = (i < ROUNDS / 2 ? ka : kb2) + (i % (ROUNDS / 2)) * ROUND + koff;
        const int r = vrow0 + i * (ROUND / VROW);
        vs = (vlc < 4 ? va : vb2) + r * (VROW / 2) + (vlc & 3) * 16;
      } else {
        ks = ka + i * ROUND + koff;
        vs = va + i * ROUND + voff;
      }
      __builtin_amdgcn_global_load_lds(ks, (__attribute__((address_space(3))) void*)(nb + i * ROUND + wv * 1024), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(
          vs, (__attribute__((address_space(3))) void*)(nb + TILEB + i * ROUND + wv * 1024), 16, 0, 0);
    }
  };
  constexpr int TSTEP = PAIRED ? 2 : 1;                // tile-map entries per LDS tile
  // memory tiles of the LDS tile at entry j (a pair's second is its first
  // again at the end of an odd row: valid memory whose keys the mask drops)
  auto tile_ptrs = [&](int j, const unsigned char*& ka, const unsigned char*& va, const unsigned char*& kb2,
                       const unsigned char*& vb2) {
    const int c0 = kv_idx[j];
    const int c1 = PAIRED && j + 1 < end ? kv_idx[j + 1] : c0;
    ka = kbase + (size_t)c0 * MTILEB;
    va = vbase + (size_t)c0 * MTILEB;
    kb2 = kbase + (size_t)c1 * MTILEB;
    vb2 = vbase + (size_t)c1 * MTILEB;
  };
  const unsigned char *nka, *nva, *nkb, *nvb;
  tile_ptrs(beg, nka, nva, nkb, nvb);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) copy_step(nka, nva, nkb, nvb, lds, kb);
  lds_u8* nbuf = lds;

  // S^T of 32-key block blk of the K tile at Ks
  auto qk = [&](const unsigned char* Ks, int blk) {
    f32x16 s = f32x16{};
    const unsigned char* kr = Ks + (blk * 32 + krow0) * KROW;
#pragma unroll
    for (int t = 0; t < DS; ++t) {
      const int c0 = 4 * t + 2 * hh;
      const i32x8 a = gload32(kr + ((c0 ^ kswz) * 16), kr + (((c0 + 1) ^ kswz) * 16));
      s = mfma8(a, qr[t], s);
    }
    return s;
  };

  // lazy rescaling on the 64 keys (s0, s1) of one step: the reference max
  // moves only when their max exceeds it by 2^2 (after exp2)
  auto rescale = [&](const f32x16& s0, const f32x16& s1) {
    // one serial chain of three-input maxima (v_max3_f32)
    float bm = fmaxf(fmaxf(s0[0], s1[0]), s0[1]);
#pragma unroll
    for (int i = 1; i < 15; ++i) bm = fmaxf(fmaxf(bm, s1[i]), s0[i + 1]);
    bm = fmaxf(bm, s1[15]);
    // each lane half tests its own maximum (m is shared by the halves); the
    // full row maximum is formed only when the branch is taken
    if (__builtin_amdgcn_ballot_w64(bm > m + thr)) {   // rare after the first steps
      bm = xhalf_max(bm);
      const float mn = fmaxf(m, bm);
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mn) * c2);
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] *= alpha;
      osum *= alpha;
      m = mn;
      nref = (mn == -INFINITY ? 0.f : -mn * c2) + kPScaleLog2;
    }
  };

  // P = e4m3(64 exp2(S c2 - m c2)) of step st and O^T += V^T P^T over its 64
  // keys, with the row sums through the selector product
  auto softmax_pv = [&](const f32x16& s0, const f32x16& s1, const unsigned char* Vs, int st) {
    // P bytes: byte j < 16 is key 16 hh + j of block 2 st, byte 16 + j key 16 hh + j of block 2 st + 1
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(fmaf(s0[4 * q], c2, nref)),
                                               __builtin_amdgcn_exp2f(fmaf(s0[4 * q + 1], c2, nref)), pb[q], false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(fmaf(s0[4 * q + 2], c2, nref)),
                                           __builtin_amdgcn_exp2f(fmaf(s0[4 * q + 3], c2, nref)), w0, true);
      int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(fmaf(s1[4 * q], c2, nref)),
                                               __builtin_amdgcn_exp2f(fmaf(s1[4 * q + 1], c2, nref)), pb[4 + q], false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_exp2f(fmaf(s1[4 * q + 2], c2, nref)),
                                           __builtin_amdgcn_exp2f(fmaf(s1[4 * q + 3], c2, nref)), w1, true);
      pb[q] = w0;
      pb[4 + q] = w1;
    }
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const unsigned char* vr = Vs + (d * 32 + lq) * VROW;
      const int c0 = 4 * st + hh, c1 = 4 * st + 2 + hh;
      const i32x8 a = gload32(vr + ((c0 ^ vswz) * 16), vr + ((c1 ^ vswz) * 16));
      o[d] = mfma8(a, pb, o[d]);
    }
    osum = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, pb, osum, 0, 0, 0, 127, 0, 127);
  };

  // One LDS tile: a software pipeline over its 64-key steps -- S^T of step
  // st + 1 is issued before the exponentials of step st, so the wave has
  // matrix work beside them.  The restrict qualifiers state that the stage
  // being read (Ks, Vs) and the stage the next tile's copy writes (nb) never
  // overlap, so the compiler issues no wait on that in-flight copy before
  // this tile's LDS reads.
  auto tile_body = [&](const unsigned char* __restrict__ Ks, const unsigned char* __restrict__ Vs,
                       lds_u8* __restrict__ nb, uint64_t vmask, auto bnd) {
    constexpr bool BOUNDARY = decltype(bnd)::value;
    f32x16 s0 = qk(Ks, 0), s1 = qk(Ks, 1);
    if constexpr (BOUNDARY) {
      apply_mask(s0, vmask, 0);
      apply_mask(s1, vmask, 1);
    }
    rescale(s0, s1);
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      copy_step(nka, nva, nkb, nvb, nb, 2 * st);
      copy_step(nka, nva, nkb, nvb, nb, 2 * st + 1);
      f32x16 t0, t1;
      if (st + 1 < NSTEP) {
        t0 = qk(Ks, 2 * st + 2);
        t1 = qk(Ks, 2 * st + 3);
      }
      softmax_pv(s0, s1, Vs, st);
      if (st + 1 < NSTEP) {
        if constexpr (BOUNDARY) {
          apply_mask(t0, vmask, 2 * st + 2);
          apply_mask(t1, vmask, 2 * st + 3);
        }
        rescale(t0, t1);
        s0 = t0;
        s1 = t1;
      }
    }
  };

  // Barrier for the LDS tile at entry j and bookkeeping of the next one's
  // copy; sets the LDS buffers holding it.
  auto begin_tile = [&](int j, const unsigned char*& Ks, const unsigned char*& Vs) {
    const int stage = ((j - beg) / TSTEP) & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // the last LDS tile re-copies itself (into the idle buffer)
    tile_ptrs(j + TSTEP < end ? j + TSTEP : j, nka, nva, nkb, nvb);
    nbuf = lds + (stage ^ 1) * STAGE;
    Ks = smem + stage * STAGE;
    Vs = Ks + TILEB;
  };
  // validity mask of this lane's query over KV tile kv: NG groups of 8 keys,
  // group gg at tile slot slot0(gg), placed at bit 8 (gg + g0)
  auto kv_tile_mask = [&](int kv, auto ng, auto slot0) {
    constexpr int NG = decltype(ng)::value;
    const int k2 = (kv % p.nk2) << p.lk2;
    const int k1 = ((kv / p.nk2) % p.nk1) << p.lk1;
    const int k0 = (kv / (p.nk2 * p.nk1)) << p.lk0;
    return boundary_mask<NG>(slot0, k0, k1, k2, st0, st1, st2, p.w0, p.w1, p.w2, p.lk2, km1, km2, ksh);
  };
  // validity mask of the LDS tile at entry j (group gg holds keys
  // 32 (gg / 2) + 16 hh + 8 (gg % 2) .. + 7 of the LDS tile)
  auto lds_tile_mask = [&](int j) {
    if constexpr (PAIRED) {
      // groups 0..3 are keys 0..63 (the first tile), 4..7 keys 64..127 (the second)
      auto slot = [&](int gg) { return 32 * (gg >> 1) + 16 * hh + 8 * (gg & 1); };
      const uint64_t ma = kv_tile_mask(kv_idx[j], std::integral_constant<int, 4>{}, slot);
      const uint64_t mb = j + 1 < end ? kv_tile_mask(kv_idx[j + 1], std::integral_constant<int, 4>{}, slot) : 0ull;
      return ma | (mb << 32);
    } else {
      return kv_tile_mask(kv_idx[j], std::integral_constant<int, KVT / 16>{},
                          [&](int gg) { return 32 * (gg >> 1) + 16 * hh + 8 * (gg & 1); });
    }
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
      for (int kb = 0; kb < KB; ++kb) copy_step(nka, nva, nkb, nvb, nbuf, kb);
    }
  } else {
    for (int j = beg; j < jfull; j += TSTEP) {
      begin_tile(j, Ks, Vs);
      tile_body(Ks, Vs, nbuf, 0ull, std::integral_constant<bool, false>{});
    }
    for (int j = jfull; j < end; j += TSTEP) {
      begin_tile(j, Ks, Vs);
      tile_body(Ks, Vs, nbuf, lds_tile_mask(j), std::integral_constant<bool, true>{});
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: out = v_scale * O / l (the factor 64 of P cancels), bf16
  const float lt = wave_active ? osum[0] : 1.f;
  const float mult = p.v_scale / lt;
  __bf16* orow = static_cast<__bf16*>(p.ot) + (GQ ? grid_base + (size_t)q_tok * tok_stride : (qtile * QT + row) * D);
  if (GQ && !q_valid) return;            // padding rows have no place in grid order
#pragma unroll
  for (int d = 0; d < DB; ++d) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v;
      v[0] = (__bf16)(o[d][4 * g + 0] * mult);
      v[1] = (__bf16)(o[d][4 * g + 1] * mult);
      v[2] = (__bf16)(o[d][4 * g + 2] * mult);
      v[3] = (__bf16)(o[d][4 * g + 3] * mult);
      *reinterpret_cast<bf16x4*>(orow + d * 32 + 8 * g + 4 * hh) = v;
    }
  }
  if (p.lse_t && hh == 0)
    p.lse_t[GQ ? (grid_base / D) + (size_t)q_tok * p.heads : qtile * QT + row] =
        m == -INFINITY ? 0.f : m * p.scale + logf(lt) - kPScaleLog2 * 0.69314718055994531f;
}

// 64-key KV tiles run as pairs in the 128-key LDS tile
template <int NW, int KVT>
hipError_t launch_cfg(const KParams& p, int io, hipStream_t st) {
  constexpr bool PAIRED = KVT == 64;
  constexpr int LKVT = PAIRED ? 128 : KVT;
  if (io == IO_QO)
    attn_fp8_kernel<128, NW, LKVT, true, PAIRED><<<p.num_wg, NW * 64, 0, st>>>(p);
  else
    attn_fp8_kernel<128, NW, LKVT, false, PAIRED><<<p.num_wg, NW * 64, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

bool attn_fp8_supported(int head_dim, int q_tokens, int kv_tokens) {
  return head_dim == 128 && (q_tokens == 128 || q_tokens == 256) && (kv_tokens == 64 || kv_tokens == 128);
}

hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t st) {
  const KParams p = make_kparams(a);
  const int qtok = a.tq[0] * a.tq[1] * a.tq[2];
  const int ktok = a.tkv[0] * a.tkv[1] * a.tkv[2];
  if (!attn_fp8_supported(a.head_dim, qtok, ktok) || !attn_bf16_tile_ok(a.tkv) || a.io_mode == IO_GRID)
    return hipErrorInvalidValue;
  const int key = (qtok == 256 ? 2 : 0) | (ktok == 128 ? 1 : 0);
  switch (key) {
    case 0: return launch_cfg<4, 64>(p, a.io_mode, st);
    case 1: return launch_cfg<4, 128>(p, a.io_mode, st);
    case 2: return launch_cfg<8, 64>(p, a.io_mode, st);
    default: return launch_cfg<8, 128>(p, a.io_mode, st);
  }
}

}  // namespace na
