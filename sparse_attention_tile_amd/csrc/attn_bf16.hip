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
// * Workgroup = 4 wavefronts (one per SIMD), Q tile = 4 * QB * 32 queries;
//   each wave owns QB blocks of 32 queries and keeps its Q operand in
//   registers for the whole kernel.
// * The transposed products are used: S^T = K Q^T and O^T = V^T P^T on
//   v_mfma_f32_32x32x16_bf16.  In the C layout of S^T a lane holds one query
//   and 16 keys, so the row max needs one cross-half exchange
//   (v_permlane32_swap) and the row sum stays in-lane.  K rows are fed to
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
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_common.hpp"

namespace na {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// 16-byte chunk swizzle of a tile row with `cpr` chunks.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CPR >= 16) return row & 15;
  else return (row >> 1) & (CPR - 1);
}

// Row of K fed to MFMA row `r` of a 32-key block: quads 1 and 2 of each
// 16-row group swap places, so that accumulator i of lane half h holds key
// 16*(i/8) + 8*h + i%8 of the block.
__device__ __forceinline__ int kperm(int r) { return (((r >> 2) ^ (r >> 3)) & 1) ? (r ^ 12) : r; }

__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Copies one tile (ROWS rows of ROWB bytes) global -> LDS, swizzled.  Each
// wave moves 1 KiB per instruction: lane i fills LDS bytes [16 i, 16 i + 16)
// of the wave's segment, so its global address picks the chunk that belongs
// there.
template <int ROWB, int TILEB>
__device__ __forceinline__ void tile_to_lds(const unsigned char* __restrict__ g, lds_u8* lds, int wv, int lane) {
  constexpr int CPR = ROWB / 16;
  constexpr int SEGS = TILEB / 1024;
  static_assert(SEGS % 4 == 0, "tile must split evenly over 4 waves");
#pragma unroll
  for (int i = 0; i < SEGS / 4; ++i) {
    const int seg = i * 4 + wv;
    const int byte = seg * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int pc = (byte % ROWB) / 16;
    const int lc = pc ^ swz<CPR>(row);
    __builtin_amdgcn_global_load_lds(g + row * ROWB + lc * 16, (__attribute__((address_space(3))) void*)(lds + seg * 1024),
                                     16, 0, 0);
  }
}

template <int D, int QB, int KVT>
__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(KParams p) {
  constexpr int QT = 4 * QB * 32;        // queries per workgroup
  constexpr int DC = D / 16;             // k-steps of S^T
  constexpr int DB = D / 32;             // 32-row blocks of O^T
  constexpr int KB = KVT / 32;           // 32-key blocks per KV tile
  constexpr int KROW = D * 2;            // bytes per K row
  constexpr int VROW = KVT * 2;          // bytes per V^T row
  constexpr int TILEB = KVT * D * 2;     // bytes of one K (or V^T) tile
  constexpr int STAGE = 2 * TILEB;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
  lds_u8* lds = (lds_u8*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, hh = lane >> 5, lq = lane & 31;
  const WorkItem wi = decode_work(p, blockIdx.x);
  const size_t qtile = (size_t)wi.bh * p.nQ + wi.qrow;

  // ---- Q operand (B of S^T = K Q^T): query = lane % 32, 8 dims per lane
  const __bf16* qbase = static_cast<const __bf16*>(p.qt) + qtile * QT * D;
  bf16x8 qr[QB][DC];
  int st0[QB], st1[QB], st2[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int row = wv * QB * 32 + b * 32 + lq;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(qbase + (size_t)row * D);
#pragma unroll
    for (int c = 0; c < DC; ++c) qr[b][c] = src[2 * c + hh];
    const int px = row & ((1 << p.lq2) - 1);
    const int py = (row >> p.lq2) & ((1 << p.lq1) - 1);
    const int pt = row >> (p.lq1 + p.lq2);
    st0[b] = dev_window_start((wi.a0 << p.lq0) + pt, p.L0, p.w0, p.s0);
    st1[b] = dev_window_start((wi.a1 << p.lq1) + py, p.L1, p.w1, p.s1);
    st2[b] = dev_window_start((wi.a2 << p.lq2) + px, p.L2, p.w2, p.s2);
  }

  f32x16 o[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    m[b] = -INFINITY;
    l[b] = 0.f;
#pragma unroll
    for (int d = 0; d < DB; ++d) o[b][d] = f32x16{};
  }

  const int beg = p.qptr[wi.qrow], end = p.qptr[wi.qrow + 1];
  const int nfull = p.n_full[wi.qrow];
  const unsigned char* kbase = static_cast<const unsigned char*>(p.kt) + (size_t)wi.bh * p.nK * TILEB;
  const unsigned char* vbase = static_cast<const unsigned char*>(p.vt) + (size_t)wi.bh * p.nK * TILEB;
  const float c2 = p.c2;
  const int km2 = (1 << p.lk2) - 1, km1 = (1 << p.lk1) - 1, ksh = p.lk1 + p.lk2;

  {  // prologue: first tile in flight
    const int kv = p.kv_idx[beg];
    tile_to_lds<KROW, TILEB>(kbase + (size_t)kv * TILEB, lds, wv, lane);
    tile_to_lds<VROW, TILEB>(vbase + (size_t)kv * TILEB, lds + TILEB, wv, lane);
  }

  for (int j = beg; j < end; ++j) {
    const int stage = (j - beg) & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < end) {
      const int kv = p.kv_idx[j + 1];
      lds_u8* nb = lds + (stage ^ 1) * STAGE;
      tile_to_lds<KROW, TILEB>(kbase + (size_t)kv * TILEB, nb, wv, lane);
      tile_to_lds<VROW, TILEB>(vbase + (size_t)kv * TILEB, nb + TILEB, wv, lane);
    }
    const unsigned char* Ks = smem + stage * STAGE;
    const unsigned char* Vs = Ks + TILEB;
    const bool boundary = (j - beg) >= nfull;
    int k0 = 0, k1 = 0, k2 = 0;
    if (boundary) {
      const int kv = p.kv_idx[j];
      k2 = (kv % p.nk2) << p.lk2;
      k1 = ((kv / p.nk2) % p.nk1) << p.lk1;
      k0 = (kv / (p.nk2 * p.nk1)) << p.lk0;
    }

#pragma unroll 1
    for (int kb = 0; kb < KB; ++kb) {
      // ---- S^T block: 32 keys x 32 queries per query block
      f32x16 s[QB];
#pragma unroll
      for (int b = 0; b < QB; ++b) s[b] = f32x16{};
      const int krow = kb * 32 + kperm(lq);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const int pc = (2 * c + hh) ^ swz<KROW / 16>(krow);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + krow * KROW + pc * 16);
#pragma unroll
        for (int b = 0; b < QB; ++b) s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[b][c], s[b], 0, 0, 0);
      }

      // ---- online softmax (fp32); accumulator i <-> key 16*(i/8) + 8*hh + i%8
      bf16x8 pv[QB][2];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        if (boundary) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = kb * 32 + 16 * (i >> 3) + 8 * hh + (i & 7);
            const int kx = k2 + (r & km2);
            const int ky = k1 + ((r >> p.lk2) & km1);
            const int kt = k0 + (r >> ksh);
            const bool ok = (unsigned)(kt - st0[b]) < (unsigned)p.w0 &&
                            (unsigned)(ky - st1[b]) < (unsigned)p.w1 &&
                            (unsigned)(kx - st2[b]) < (unsigned)p.w2;
            if (!ok) s[b][i] = -INFINITY;
          }
        }
        float bm = s[b][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) bm = fmaxf(bm, s[b][i]);
        bm = xhalf_max(bm);
        const float mn = fmaxf(m[b], bm);
        const float ref = mn == -INFINITY ? 0.f : mn;  // every key so far masked
        const float alpha = __builtin_amdgcn_exp2f((m[b] - ref) * c2);
        const float nref = -ref * c2;
        float rs = 0.f;
        float pf[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pf[i] = __builtin_amdgcn_exp2f(fmaf(s[b][i], c2, nref));
          rs += pf[i];
        }
        l[b] = l[b] * alpha + rs;
        m[b] = mn;
#pragma unroll
        for (int d = 0; d < DB; ++d) o[b][d] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pv[b][0][i] = (__bf16)pf[i];
          pv[b][1][i] = (__bf16)pf[8 + i];
        }
      }

      // ---- O^T += V^T P^T over the block's two 16-key halves
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const int vr = d * 32 + lq;
          const int pc = (4 * kb + 2 * c + hh) ^ swz<VROW / 16>(vr);
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vs + vr * VROW + pc * 16);
#pragma unroll
          for (int b = 0; b < QB; ++b) o[b][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pv[b][c], o[b][d], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: O / l in bf16, lse = m*scale + ln l
  __bf16* obase = static_cast<__bf16*>(p.ot) + qtile * QT * D;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float lt = xhalf_sum(l[b]);
    const float inv = 1.f / lt;
    const int row = wv * QB * 32 + b * 32 + lq;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v;
        v[0] = (__bf16)(o[b][d][4 * g + 0] * inv);
        v[1] = (__bf16)(o[b][d][4 * g + 1] * inv);
        v[2] = (__bf16)(o[b][d][4 * g + 2] * inv);
        v[3] = (__bf16)(o[b][d][4 * g + 3] * inv);
        const int col = d * 32 + 8 * g + 4 * hh;
        *reinterpret_cast<bf16x4*>(obase + (size_t)row * D + col) = v;
      }
    }
    if (p.lse_t && hh == 0) p.lse_t[qtile * QT + row] = m[b] * p.scale + logf(lt);
  }
}

template <int D, int QB, int KVT>
hipError_t launch_cfg(const KParams& p, hipStream_t st) {
  attn_bf16_kernel<D, QB, KVT><<<p.num_wg, 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

bool attn_bf16_supported(int head_dim, int q_tokens, int kv_tokens) {
  return (head_dim == 64 || head_dim == 128) && (q_tokens == 128 || q_tokens == 256) &&
         (kv_tokens == 64 || kv_tokens == 128);
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st) {
  const KParams p = make_kparams(a);
  const int qtok = a.tq[0] * a.tq[1] * a.tq[2];
  const int ktok = a.tkv[0] * a.tkv[1] * a.tkv[2];
  const int key = (a.head_dim == 128 ? 4 : 0) | (qtok == 256 ? 2 : 0) | (ktok == 128 ? 1 : 0);
  if (!attn_bf16_supported(a.head_dim, qtok, ktok)) return hipErrorInvalidValue;
  switch (key) {
    case 0: return launch_cfg<64, 1, 64>(p, st);
    case 1: return launch_cfg<64, 1, 128>(p, st);
    case 2: return launch_cfg<64, 2, 64>(p, st);
    case 3: return launch_cfg<64, 2, 128>(p, st);
    case 4: return launch_cfg<128, 1, 64>(p, st);
    case 5: return launch_cfg<128, 1, 128>(p, st);
    case 6: return launch_cfg<128, 2, 64>(p, st);
    default: return launch_cfg<128, 2, 128>(p, st);
  }
}

}  // namespace na
