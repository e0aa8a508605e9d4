// Content-selected block sparsity: block-mean importance scores and the
// top-k KV tiles of every Q tile ("Video-generation inference speed-up:
// sparse attention configuration tutorial", section 6: score blocks, keep the
// most important ones by a keep ratio, skip the rest whole; "Sparse
// attention: the key technology for more efficient AI models", section 2.2:
// top-k selection).  The attention over the kept tiles is the bf16 GNA kernel
// with one tile map per (batch, head).
//
// The selection is an integer decision taken from floating-point scores; it
// is evaluated in one fixed float32 order (sequential sums with explicit
// round-to-nearest adds and multiplies, no fused multiply-add, IEEE
// division), so that it is reproducible bit for bit.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace na {
namespace {

// Mean over the real tokens of each tile of x (grid order [B, T, H, W,
// heads, D] bf16) in in-tile row-major order: one thread per (tile, 8 dims)
// of a (batch, head), one 16-byte load per token, each dim's sum sequential
// over the tokens; out [B*heads, n_tiles, D] fp32, or [B*heads, D, n_tiles]
// with `dim_major` (the layout the selection reads K means in).
__global__ __launch_bounds__(256) void block_mean_kernel(const __bf16* __restrict__ x, float* __restrict__ out,
                                                         TopkGeom g, int t0, int t1, int t2, int64_t n_items,
                                                         bool dim_major) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (bh, tile, 8-dim chunk)
  if (item >= n_items) return;
  const int chunks = g.head_dim / 8;
  const int ch = (int)(item % chunks);
  const int64_t bt = item / chunks;
  const int nt1 = (g.L[1] + t1 - 1) / t1, nt2 = (g.L[2] + t2 - 1) / t2;
  const int ntl = ((g.L[0] + t0 - 1) / t0) * nt1 * nt2;
  const int tile = (int)(bt % ntl);
  const int bh = (int)(bt / ntl);
  const int b = bh / g.heads, h = bh % g.heads;
  const int a2 = tile % nt2, a1 = (tile / nt2) % nt1, a0 = tile / (nt2 * nt1);
  const int64_t N = (int64_t)g.L[0] * g.L[1] * g.L[2];
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int cnt = 0;
  for (int dt = 0; dt < t0; ++dt) {
    const int t = a0 * t0 + dt;
    if (t >= g.L[0]) break;
    for (int dy = 0; dy < t1; ++dy) {
      const int y = a1 * t1 + dy;
      if (y >= g.L[1]) break;
      for (int dx = 0; dx < t2; ++dx) {
        const int xx = a2 * t2 + dx;
        if (xx >= g.L[2]) break;
        const int64_t tok = ((int64_t)t * g.L[1] + y) * g.L[2] + xx;
        const bf16x8_t v = reinterpret_cast<const bf16x8_t*>(x + ((b * N + tok) * g.heads + h) * g.head_dim)[ch];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __fadd_rn(acc[j], (float)v[j]);
        ++cnt;
      }
    }
  }
  const float fc = (float)cnt;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = ch * 8 + j;
    out[dim_major ? ((int64_t)bh * g.head_dim + d) * ntl + tile : bt * g.head_dim + d] = __fdiv_rn(acc[j], fc);
  }
}

// Order-preserving map of a float32 score to uint32 (larger float -> larger
// integer; callers turn -0 into +0 first so equal floats map equal).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k KV tiles of one Q tile of one (batch, head).  Scores go to LDS as
// 64-bit keys (ordered score bits, then the inverted tile index), sorted
// descending by a bitonic network of SORTN >= nk entries (padding keys 0),
// so the first `keep` keys are the kept tiles: larger score first, the lower
// index first among equal scores.  The kept tiles are written full tiles
// first (no padding slot), then the others, each ascending.  qptr (shared by
// all (batch, head)) is written by bh 0.
template <int SORTN>
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ qm, const float* __restrict__ km,
                                                     int32_t* __restrict__ kv_idx, int32_t* __restrict__ n_full,
                                                     int32_t* __restrict__ qptr, TopkGeom g, int nq, int nk,
                                                     int keep) {
  __shared__ uint64_t key[SORTN];
  __shared__ float qv[128];
  __shared__ unsigned char sel[SORTN];
  __shared__ int n_kept_full;
  const int row = blockIdx.x;                        // bh * nq + a
  const int bh = row / nq, a = row % nq;
  const int D = g.head_dim;
  for (int d = threadIdx.x; d < D; d += 256) qv[d] = qm[(int64_t)row * D + d];
  if (threadIdx.x == 0) n_kept_full = 0;
  __syncthreads();
  const float* kb = km + (int64_t)bh * nk * D;       // [D][nk]: lanes read consecutive tiles
  for (int c = threadIdx.x; c < SORTN; c += 256) {
    uint64_t kk = 0;
    if (c < nk) {
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = __fadd_rn(s, __fmul_rn(qv[d], kb[(int64_t)d * nk + c]));
      s = __fadd_rn(s, 0.f);   // -0 -> +0: equal floats get equal keys
      kk = ((uint64_t)ordered_bits(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)c);
    }
    key[c] = kk;
    sel[c] = 0;
  }
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= SORTN; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < SORTN / 2; i += 256) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = key[lo], y = key[hi];
        if ((x < y) == desc) {
          key[lo] = y;
          key[hi] = x;
        }
      }
      __syncthreads();
    }
  const int nt1 = (g.L[1] + g.tkv[1] - 1) / g.tkv[1], nt2 = (g.L[2] + g.tkv[2] - 1) / g.tkv[2];
  // sel[c]: bit 0 kept, bit 1 kept and full (no padding slot)
  for (int r = threadIdx.x; r < keep; r += 256) {
    const int c = (int)(0xFFFFFFFFu - (uint32_t)(key[r] & 0xFFFFFFFFu));
    const int c2 = c % nt2, c1 = (c / nt2) % nt1, c0 = c / (nt2 * nt1);
    const bool full =
        (c0 + 1) * g.tkv[0] <= g.L[0] && (c1 + 1) * g.tkv[1] <= g.L[1] && (c2 + 1) * g.tkv[2] <= g.L[2];
    sel[c] = full ? 3 : 1;
  }
  __syncthreads();
  // positions: full kept tiles first, then the others, each ascending --
  // an exclusive prefix count over c, each thread owning a run of SORTN/256
  constexpr int RUN = SORTN / 256;
  __shared__ int cnt_f[256], cnt_b[256];
  int nfr = 0, nbr = 0;
  const int c_lo = threadIdx.x * RUN;
#pragma unroll
  for (int e = 0; e < RUN; ++e) {
    const unsigned char v = sel[c_lo + e];
    nfr += v == 3;
    nbr += v == 1;
  }
  cnt_f[threadIdx.x] = nfr;
  cnt_b[threadIdx.x] = nbr;
  __syncthreads();
  if (threadIdx.x == 0) {   // 256-entry exclusive scan, one thread (cheap next to the sort)
    int sf = 0, sb = 0;
    for (int t = 0; t < 256; ++t) {
      const int f = cnt_f[t], b = cnt_b[t];
      cnt_f[t] = sf;
      cnt_b[t] = sb;
      sf += f;
      sb += b;
    }
    n_kept_full = sf;
  }
  __syncthreads();
  const int nf = n_kept_full;
  int32_t* out = kv_idx + (int64_t)row * keep;
  int pf = cnt_f[threadIdx.x], pb = nf + cnt_b[threadIdx.x];
#pragma unroll
  for (int e = 0; e < RUN; ++e) {
    const int c = c_lo + e;
    const unsigned char v = sel[c];
    if (v == 3) out[pf++] = c;
    else if (v == 1) out[pb++] = c;
  }
  if (threadIdx.x == 0) {
    n_full[row] = nf;
    if (bh == 0) {
      qptr[a] = a * keep;
      if (a == nq - 1) qptr[nq] = nq * keep;
    }
  }
}

}  // namespace

// Largest sortable tile count (the sort keys of a row live in LDS).
constexpr int kMaxSort = 4096;
bool topk_select_supported(int nk, int head_dim) { return nk <= kMaxSort && head_dim <= 128 && head_dim % 8 == 0; }

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t st) {
  const TopkGeom& g = a.geom;
  const int64_t bh = (int64_t)g.batch * g.heads;
  const int64_t nq_items = bh * a.nq * (g.head_dim / 8), nk_items = bh * a.nk * (g.head_dim / 8);
  block_mean_kernel<<<(unsigned)((nq_items + 255) / 256), 256, 0, st>>>(static_cast<const __bf16*>(a.q), a.qm, g,
                                                                          g.tq[0], g.tq[1], g.tq[2], nq_items, false);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  block_mean_kernel<<<(unsigned)((nk_items + 255) / 256), 256, 0, st>>>(static_cast<const __bf16*>(a.k), a.km, g,
                                                                          g.tkv[0], g.tkv[1], g.tkv[2], nk_items, true);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nb = (unsigned)(bh * a.nq);
  if (a.nk <= 1024)
    select_kernel<1024><<<nb, 256, 0, st>>>(a.qm, a.km, a.kv_idx, a.n_full, a.qptr, g, a.nq, a.nk, a.keep);
  else
    select_kernel<kMaxSort><<<nb, 256, 0, st>>>(a.qm, a.km, a.kv_idx, a.n_full, a.qptr, g, a.nq, a.nk, a.keep);
  return hipGetLastError();
}

}  // namespace na
