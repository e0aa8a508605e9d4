// fp32 GNA attention: fp32 inputs, products, softmax and accumulation, no
// reduced-precision matrix path.  It is the exact-arithmetic variant (small
// problems, head_dim 32/64/128); the bf16 and fp8 kernels are the fast ones.
//
// One wavefront per Q tile of 64 queries, one query per lane.  For each KV
// tile of the Q tile's row in the tile map (GNA page, "GNA Sparse Attention
// Mechanism: Vision-Transformer Compute Optimisation in Practice", section
// 1.1) the K and V tiles are staged in LDS; every lane computes its 64
// scores, masks them only on boundary tiles (section 2.1) and folds them into
// a running max / sum / output (block-wise softmax normalisation, tutorial
// "Video-generation inference speed-up: sparse attention configuration
// tutorial", section 3.3).
#include <hip/hip_runtime.h>

#include <cmath>

#include "attn_common.hpp"

namespace na {
namespace {

constexpr int kTile = 64;

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(KParams p) {
  __shared__ __attribute__((aligned(16))) float Ks[kTile * D];
  __shared__ __attribute__((aligned(16))) float Vs[kTile * D];
  const WorkItem wi = decode_work(p, blockIdx.x);
  const int lane = threadIdx.x;

  // this lane's query and its window on each axis
  const int px = lane & ((1 << p.lq2) - 1);
  const int py = (lane >> p.lq2) & ((1 << p.lq1) - 1);
  const int pt = lane >> (p.lq1 + p.lq2);
  const int st0 = dev_window_start((wi.a0 << p.lq0) + pt, p.L0, p.w0, p.s0);
  const int st1 = dev_window_start((wi.a1 << p.lq1) + py, p.L1, p.w1, p.s1);
  const int st2 = dev_window_start((wi.a2 << p.lq2) + px, p.L2, p.w2, p.s2);

  const size_t qtile = (size_t)wi.bh * p.nQ + wi.qrow;
  const float* qrow = static_cast<const float*>(p.qt) + (qtile * kTile + lane) * D;
  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qrow[d];
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int beg = p.qptr[wi.qrow], end = p.qptr[wi.qrow + 1];
  const int nf = p.n_full[wi.qrow];
  const float* kb = static_cast<const float*>(p.kt) + (size_t)wi.bh * p.nK * kTile * D;
  const float* vb = static_cast<const float*>(p.vt) + (size_t)wi.bh * p.nK * kTile * D;
  const int kmask2 = (1 << p.lk2) - 1, kmask1 = (1 << p.lk1) - 1;

  for (int j = beg; j < end; ++j) {
    const int kv = p.kv_idx[j];
    __syncthreads();
    const float4* ks = reinterpret_cast<const float4*>(kb + (size_t)kv * kTile * D);
    const float4* vs = reinterpret_cast<const float4*>(vb + (size_t)kv * kTile * D);
    for (int e = lane; e < kTile * D / 4; e += 64) {
      reinterpret_cast<float4*>(Ks)[e] = ks[e];
      reinterpret_cast<float4*>(Vs)[e] = vs[e];
    }
    __syncthreads();
    const bool boundary = (j - beg) >= nf;
    const int c2 = kv % p.nk2;
    const int c1 = (kv / p.nk2) % p.nk1;
    const int c0 = kv / (p.nk2 * p.nk1);
    float s[kTile];
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], Ks[r * D + d], acc);
      acc *= p.scale;
      if (boundary) {
        const int kx = (c2 << p.lk2) + (r & kmask2);
        const int ky = (c1 << p.lk1) + ((r >> p.lk2) & kmask1);
        const int kt = (c0 << p.lk0) + (r >> (p.lk1 + p.lk2));
        const bool ok = (unsigned)(kt - st0) < (unsigned)p.w0 && (unsigned)(ky - st1) < (unsigned)p.w1 &&
                        (unsigned)(kx - st2) < (unsigned)p.w2;
        if (!ok) acc = -INFINITY;
      }
      s[r] = acc;
      bm = fmaxf(bm, acc);
    }
    const float mn = fmaxf(m, bm);
    const float ref = mn == -INFINITY ? 0.f : mn;   // every key so far masked
    const float alpha = expf(m - ref);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int r = 0; r < kTile; ++r) {
      const float pr = expf(s[r] - ref);
      l += pr;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(pr, Vs[r * D + d], o[d]);
    }
    m = mn;
  }

  const float inv = 1.f / l;
  float4* orow = reinterpret_cast<float4*>(static_cast<float*>(p.ot) + (qtile * kTile + lane) * D);
#pragma unroll
  for (int d = 0; d < D; d += 4) orow[d / 4] = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
  if (p.lse_t) p.lse_t[qtile * kTile + lane] = m + logf(l);
}

}  // namespace

bool attn_f32_supported(int head_dim, int q_tokens, int kv_tokens) {
  return (head_dim == 32 || head_dim == 64 || head_dim == 128) && q_tokens == kTile && kv_tokens == kTile;
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st) {
  KParams p = make_kparams(a);
  switch (a.head_dim) {
    case 32: attn_f32_kernel<32><<<p.num_wg, 64, 0, st>>>(p); break;
    case 64: attn_f32_kernel<64><<<p.num_wg, 64, 0, st>>>(p); break;
    case 128: attn_f32_kernel<128><<<p.num_wg, 64, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace na
