// Token permutation between grid order and tile order (GNA page, "GNA
// Sparse Attention Mechanism: Vision-Transformer Compute Optimisation in
// Practice", section 2.2: the tokens are permuted into tile order before the
// attention kernel and back afterwards; the page plans a dedicated kernel
// that fuses the permutation with padding).
//
// Grid order: [B, T, H, W, heads, D].  Tile order: [B, heads, tiles, tile
// tokens, D] (or [.., D, tile tokens] for the transposed variant the
// attention kernel reads V from), tiles and in-tile tokens row-major over
// (T, H, W), each axis zero-padded to a whole number of tiles.
//
// These kernels are HBM-bound copies.  One workgroup moves one tile of one
// (batch, head): its rows are D * elem_bytes contiguous bytes on both sides,
// so every thread moves 16-byte chunks and both reads and writes stay
// coalesced.  The transposed variant stages the tile through LDS.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace na {
namespace {

struct TileGeom {
  int L0, L1, L2;      // grid extents
  int lg0, lg1, lg2;   // log2 tile extents
  int n1, n2;          // tiles along H and W
  int ntiles;          // tiles per (batch, head)
  int heads;
  int cpr_lg;          // log2 of 16-byte chunks per token row
};

// Work item of this workgroup: one tile of one (batch, head), heads fastest,
// so the workgroups in flight at once cover every head of a few tiles and
// together read (or write) whole grid-order token rows (heads x D) instead of
// one head's slice of many rows.  lin = (batch, head) x tiles + tile is the
// tile's slot in tile order.
struct TileBlock {
  int tile, bh;
  size_t lin;
};
__device__ inline TileBlock tile_block(const TileGeom& g) {
  const int nbh = gridDim.x / g.ntiles;
  TileBlock w;
  w.bh = blockIdx.x % nbh;
  w.tile = blockIdx.x / nbh;
  w.lin = (size_t)w.bh * g.ntiles + w.tile;
  return w;
}

__device__ inline void tile_origin(const TileGeom& g, int tile, int& t0, int& y0, int& x0) {
  const int a2 = tile % g.n2;
  const int rest = tile / g.n2;
  const int a1 = rest % g.n1;
  const int a0 = rest / g.n1;
  t0 = a0 << g.lg0;
  y0 = a1 << g.lg1;
  x0 = a2 << g.lg2;
}

// grid -> tile order, one 16-byte chunk per thread step
__global__ __launch_bounds__(256) void permute_rows_kernel(const uint4* __restrict__ x, uint4* __restrict__ xt,
                                                           TileGeom g) {
  const TileBlock wb = tile_block(g);
  const int tile = wb.tile;
  const int bh = wb.bh;
  const int b = bh / g.heads;
  const int h = bh % g.heads;
  int t0, y0, x0;
  tile_origin(g, tile, t0, y0, x0);
  const int ttok_lg = g.lg0 + g.lg1 + g.lg2;
  const int total = 1 << (ttok_lg + g.cpr_lg);
  const int cmask = (1 << g.cpr_lg) - 1;
  uint4* dst = xt + (wb.lin << (ttok_lg + g.cpr_lg));
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int p = e >> g.cpr_lg;
    const int c = e & cmask;
    const int px = p & ((1 << g.lg2) - 1);
    const int py = (p >> g.lg2) & ((1 << g.lg1) - 1);
    const int pt = p >> (g.lg1 + g.lg2);
    const int t = t0 + pt, y = y0 + py, xx = x0 + px;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < g.L0 && y < g.L1 && xx < g.L2) {
      const size_t row = ((((size_t)b * g.L0 + t) * g.L1 + y) * g.L2 + xx) * g.heads + h;
      v = x[(row << g.cpr_lg) + c];
    }
    dst[e] = v;
  }
}

// tile -> grid order (padding dropped)
__global__ __launch_bounds__(256) void unpermute_rows_kernel(const uint4* __restrict__ xt, uint4* __restrict__ x,
                                                             TileGeom g) {
  const TileBlock wb = tile_block(g);
  const int tile = wb.tile;
  const int bh = wb.bh;
  const int b = bh / g.heads;
  const int h = bh % g.heads;
  int t0, y0, x0;
  tile_origin(g, tile, t0, y0, x0);
  const int ttok_lg = g.lg0 + g.lg1 + g.lg2;
  const int total = 1 << (ttok_lg + g.cpr_lg);
  const int cmask = (1 << g.cpr_lg) - 1;
  const uint4* src = xt + (wb.lin << (ttok_lg + g.cpr_lg));
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int p = e >> g.cpr_lg;
    const int c = e & cmask;
    const int px = p & ((1 << g.lg2) - 1);
    const int py = (p >> g.lg2) & ((1 << g.lg1) - 1);
    const int pt = p >> (g.lg1 + g.lg2);
    const int t = t0 + pt, y = y0 + py, xx = x0 + px;
    if (t < g.L0 && y < g.L1 && xx < g.L2) {
      const size_t row = ((((size_t)b * g.L0 + t) * g.L1 + y) * g.L2 + xx) * g.heads + h;
      x[(row << g.cpr_lg) + c] = src[e];
    }
  }
}

// grid -> transposed tile order: each tile stored as [D][tile tokens].
// The tile is staged in LDS as [tokens][D] with a 4-byte row pad so the
// column reads of the transpose hit distinct banks.
template <typename T>
__global__ __launch_bounds__(256) void permute_transpose_kernel(const uint4* __restrict__ x, uint4* __restrict__ xt,
                                                                TileGeom g, int D) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
  const TileBlock wb = tile_block(g);
  const int tile = wb.tile;
  const int bh = wb.bh;
  const int b = bh / g.heads;
  const int h = bh % g.heads;
  int t0, y0, x0;
  tile_origin(g, tile, t0, y0, x0);
  const int ttok_lg = g.lg0 + g.lg1 + g.lg2;
  const int TT = 1 << ttok_lg;
  const int cpr = 1 << g.cpr_lg;
  const int row_bytes = D * (int)sizeof(T) + 4;
  // load [TT][D] into LDS
  for (int e = threadIdx.x; e < TT * cpr; e += blockDim.x) {
    const int p = e >> g.cpr_lg;
    const int c = e & (cpr - 1);
    const int px = p & ((1 << g.lg2) - 1);
    const int py = (p >> g.lg2) & ((1 << g.lg1) - 1);
    const int pt = p >> (g.lg1 + g.lg2);
    const int t = t0 + pt, y = y0 + py, xx = x0 + px;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < g.L0 && y < g.L1 && xx < g.L2) {
      const size_t row = ((((size_t)b * g.L0 + t) * g.L1 + y) * g.L2 + xx) * g.heads + h;
      v = x[(row << g.cpr_lg) + c];
    }
    // 4-byte stores (rows are only 4-byte aligned because of the pad)
    uint32_t* d32 = reinterpret_cast<uint32_t*>(lds_raw + p * row_bytes + c * 16);
    d32[0] = v.x;
    d32[1] = v.y;
    d32[2] = v.z;
    d32[3] = v.w;
  }
  __syncthreads();
  // store [D][TT]: chunk e covers tokens (e % (TT/E))*E .. +E-1 of row d
  const int cpd = TT / E;  // chunks per output row
  uint4* dst = xt + wb.lin * (size_t)(TT * cpr);
  for (int e = threadIdx.x; e < D * cpd; e += blockDim.x) {
    const int d = e / cpd;
    const int p0 = (e % cpd) * E;
    union {
      T el[E];
      uint4 v;
    } u;
#pragma unroll
    for (int j = 0; j < E; ++j) u.el[j] = *reinterpret_cast<const T*>(lds_raw + (p0 + j) * row_bytes + d * sizeof(T));
    dst[e] = u.v;
  }
}

// lse: [B, heads, tiles, TT] -> [B, T, H, W, heads]
__global__ __launch_bounds__(256) void unpermute_lse_kernel(const float* __restrict__ lt, float* __restrict__ l,
                                                            TileGeom g) {
  const TileBlock wb = tile_block(g);
  const int tile = wb.tile;
  const int bh = wb.bh;
  const int b = bh / g.heads;
  const int h = bh % g.heads;
  int t0, y0, x0;
  tile_origin(g, tile, t0, y0, x0);
  const int ttok_lg = g.lg0 + g.lg1 + g.lg2;
  const float* src = lt + (wb.lin << ttok_lg);
  for (int p = threadIdx.x; p < (1 << ttok_lg); p += blockDim.x) {
    const int px = p & ((1 << g.lg2) - 1);
    const int py = (p >> g.lg2) & ((1 << g.lg1) - 1);
    const int pt = p >> (g.lg1 + g.lg2);
    const int t = t0 + pt, y = y0 + py, xx = x0 + px;
    if (t < g.L0 && y < g.L1 && xx < g.L2) l[((((size_t)b * g.L0 + t) * g.L1 + y) * g.L2 + xx) * g.heads + h] = src[p];
  }
}

int lg2i(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

TileGeom make_geom(int batch, int heads, int head_dim, const int grid[3], const int tile[3], int eb, int* nblocks) {
  TileGeom g;
  g.L0 = grid[0];
  g.L1 = grid[1];
  g.L2 = grid[2];
  g.lg0 = lg2i(tile[0]);
  g.lg1 = lg2i(tile[1]);
  g.lg2 = lg2i(tile[2]);
  const int n0 = (grid[0] + tile[0] - 1) / tile[0];
  g.n1 = (grid[1] + tile[1] - 1) / tile[1];
  g.n2 = (grid[2] + tile[2] - 1) / tile[2];
  g.ntiles = n0 * g.n1 * g.n2;
  g.heads = heads;
  g.cpr_lg = lg2i(head_dim * eb / 16);
  *nblocks = batch * heads * g.ntiles;
  return g;
}

}  // namespace

size_t permute_transpose_lds_bytes(int head_dim, int tile_tokens, int elem_bytes) {
  return (size_t)tile_tokens * (size_t)(head_dim * elem_bytes + 4);
}

hipError_t launch_permute(const void* x, void* xt, int batch, int heads, int head_dim, const int grid[3],
                          const int tile[3], int elem_bytes, int transpose, hipStream_t st) {
  int nb = 0;
  TileGeom g = make_geom(batch, heads, head_dim, grid, tile, elem_bytes, &nb);
  if ((head_dim * elem_bytes) != (16 << g.cpr_lg)) return hipErrorInvalidValue;  // rows must be 2^k chunks
  if (!transpose) {
    permute_rows_kernel<<<nb, 256, 0, st>>>(static_cast<const uint4*>(x), static_cast<uint4*>(xt), g);
    return hipGetLastError();
  }
  const int tt = tile[0] * tile[1] * tile[2];
  const size_t lds = permute_transpose_lds_bytes(head_dim, tt, elem_bytes);
  if (lds > 65536) return hipErrorInvalidValue;
  switch (elem_bytes) {
    case 1:
      permute_transpose_kernel<uint8_t><<<nb, 256, lds, st>>>(static_cast<const uint4*>(x), static_cast<uint4*>(xt),
                                                              g, head_dim);
      break;
    case 2:
      permute_transpose_kernel<uint16_t><<<nb, 256, lds, st>>>(static_cast<const uint4*>(x),
                                                               static_cast<uint4*>(xt), g, head_dim);
      break;
    default:
      permute_transpose_kernel<uint32_t><<<nb, 256, lds, st>>>(static_cast<const uint4*>(x),
                                                               static_cast<uint4*>(xt), g, head_dim);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_unpermute(const void* xt, void* x, int batch, int heads, int head_dim, const int grid[3],
                            const int tile[3], int elem_bytes, hipStream_t st) {
  int nb = 0;
  TileGeom g = make_geom(batch, heads, head_dim, grid, tile, elem_bytes, &nb);
  if ((head_dim * elem_bytes) != (16 << g.cpr_lg)) return hipErrorInvalidValue;
  unpermute_rows_kernel<<<nb, 256, 0, st>>>(static_cast<const uint4*>(xt), static_cast<uint4*>(x), g);
  return hipGetLastError();
}

hipError_t launch_unpermute_lse(const float* lse_t, float* lse, int batch, int heads, const int grid[3],
                                const int tile[3], hipStream_t st) {
  int nb = 0;
  TileGeom g = make_geom(batch, heads, 4, grid, tile, 4, &nb);
  unpermute_lse_kernel<<<nb, 256, 0, st>>>(lse_t, lse, g);
  return hipGetLastError();
}

}  // namespace na
