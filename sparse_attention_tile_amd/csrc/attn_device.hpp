// Device helpers shared by the gfx950 attention kernels: LDS swizzle, the
// LDS-DMA tile copies, cross-half reductions and the boundary-tile masks.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace na {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// 16-byte chunk swizzle of a tile row with CPR chunks: chunk c of row r is
// stored at position c ^ swz(r).  The 64 LDS banks (4 bytes each) span 256
// bytes = 16 / CPR rows.  Two read shapes must be conflict-free:
//  * 16-byte reads down a column (16 consecutive rows, one chunk): needs
//    swz to be a bijection of the row's index within 16 rows (in units of
//    the 256-byte span) onto the span's 16 chunk slots;
//  * transposing 8-byte reads (4 consecutive rows x 4 consecutive chunks
//    each): needs the 4 rows to move the chunk quad to 4 different quads.
// For CPR = 16 the row's two low bits XOR the chunk's quad bits and the next
// two XOR the chunk within the quad; for CPR = 8 the same holds after the
// row pair (two rows share one span) is taken as the unit.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CPR >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else if constexpr (CPR == 8) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  else return (row / (16 / CPR)) & (CPR - 1);
}

__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Global -> LDS copy of one tile (rows of ROWB bytes), swizzled.  Each wave
// moves 1 KiB per instruction: lane i fills LDS bytes [16 i, 16 i + 16) of
// the wave's segment, so its global address picks the chunk that belongs
// there.  Wave wv copies segments wv, wv + NW, ...; segment NW i + wv starts
// 1024 NW i bytes after segment wv and the swizzle repeats within that
// distance, so a lane's source offset is lane_off + 1024 NW i with lane_off
// fixed for the whole kernel.
template <int ROWB, int NW>
__device__ __forceinline__ int dma_lane_offset(int wv, int lane) {
  constexpr int CPR = ROWB / 16;
  constexpr int ROUND = 1024 * NW;
  static_assert(ROUND % ROWB == 0, "rows must divide the copy round");
  static_assert((ROUND / ROWB) % 16 == 0, "swizzle period must divide the copy round");
  const int byte = wv * 1024 + lane * 16;
  const int row = byte / ROWB;
  const int pc = (byte % ROWB) / 16;
  return row * ROWB + ((pc ^ swz<CPR>(row)) * 16);
}

template <int TILEB, int NW>
__device__ __forceinline__ void tile_to_lds(const unsigned char* __restrict__ g, unsigned lane_off, lds_u8* lds, int wv) {
  constexpr int ROUND = 1024 * NW;
  static_assert(TILEB % ROUND == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < TILEB / ROUND; ++i)
    __builtin_amdgcn_global_load_lds(g + i * ROUND + lane_off,
                                     (__attribute__((address_space(3))) void*)(lds + i * ROUND + wv * 1024), 16, 0, 0);
}

// The rounds of a tile copy that belong to step kb of KB: the copy of the
// next tile is spread over the current tile's key blocks, so the CU's vector
// memory path sees a steady trickle instead of every wave's whole copy at
// the barrier (which would stall all waves until the address queue drains).
template <int TILEB, int NW, int KB>
__device__ __forceinline__ void tile_to_lds_step(const unsigned char* __restrict__ g, unsigned lane_off,
                                                 lds_u8* lds, int wv, int kb) {
  constexpr int ROUND = 1024 * NW;
  constexpr int ROUNDS = TILEB / ROUND;
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i)
    if ((i * KB) / ROUNDS == kb)
      __builtin_amdgcn_global_load_lds(g + i * ROUND + lane_off,
                                       (__attribute__((address_space(3))) void*)(lds + i * ROUND + wv * 1024), 16, 0,
                                       0);
}

// Boundary tiles: accumulator i of 32-key block kb has validity bit 16 kb + i
// of the lane's mask.
__device__ __forceinline__ void apply_mask(f32x16& s, uint64_t vmask, int kb) {
  const unsigned mb = (unsigned)(vmask >> (16 * kb)) & 0xFFFFu;
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = ((mb >> i) & 1u) ? s[i] : -INFINITY;
}

// Validity bits of the key slots one lane holds in a boundary KV tile.  The
// lane's slots come in NG groups of 8 consecutive slots; group gg starts at
// slot slot0(gg) and its bits go to bits 8 gg .. 8 gg + 7.  The KV tile's W
// extent is >= 8 and a power of two, so a group shares its (T, H) position
// and covers 8 consecutive W positions: a query at window starts (st0, st1,
// st2) sees slot 8-run W positions [st2, st2 + w2) intersected with the group.
template <int NG, typename SlotFn>
__device__ __forceinline__ uint64_t boundary_mask(SlotFn slot0, int k0, int k1, int k2, int st0, int st1, int st2,
                                                  int w0, int w1, int w2, int lk2, int km1, int km2, int ksh) {
  static_assert(NG <= 8, "validity mask holds 64 bits");
  uint64_t vmask = 0;
#pragma unroll 1
  for (int gg = 0; gg < NG; ++gg) {
    const int r0 = slot0(gg);
    const int lo = min(max(st2 - k2 - (r0 & km2), 0), 8);
    const int hi = min(max(st2 + w2 - k2 - (r0 & km2), 0), 8);
    const unsigned bits = ((1u << hi) - 1u) & ~((1u << lo) - 1u);
    const bool th = ((unsigned)(k0 + (r0 >> ksh) - st0) < (unsigned)w0) &
                    ((unsigned)(k1 + ((r0 >> lk2) & km1) - st1) < (unsigned)w1);
    vmask |= (uint64_t)(th ? bits : 0u) << (8 * gg);
  }
  return vmask;
}

// ---- bf16 MFMA operand helpers shared by the forward and backward kernels

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Row of an LDS tile fed to MFMA row `r` of a 32-row block: quads 1 and 2 of
// each 16-row group swap places, so that accumulator i of lane half h holds
// row 16*(i/8) + 8*h + i%8 of the block (two runs of 8 consecutive rows, the
// k order of a B operand).
__device__ __forceinline__ int kperm(int r) { return (((r >> 2) ^ (r >> 3)) & 1) ? (r ^ 12) : r; }

// 32 rows (block kb) of an LDS tile of [row][D] bf16 rows times the register
// operand br (B: D x 32 columns, lane n holds 8 consecutive dims of column n
// per 16-dim step): a 32 x 32 fp32 block, lane = column, accumulator i = row
// 16*(i/8) + 8*h + i%8.  With K rows and Q columns this is S^T = K Q^T.
template <int D, int ROWB>
__device__ __forceinline__ f32x16 qk_block(const unsigned char* Ts, int kb, int row0, int rswz, int hh,
                                           const bf16x8* br) {
  f32x16 s = f32x16{};
  const unsigned char* rowp = Ts + (kb * 32 + row0) * ROWB;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(rowp + (((2 * c + hh) ^ rswz) * 16));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, br[c], s, 0, 0, 0);
  }
  return s;
}

// A operand of O^T = V^T P^T (32 head dims x 16 keys: keys key0 .. key0+15 of
// the tile, dims 32 db .. 32 db + 31) from a tile stored [key][d] (rows of
// 2 D bytes, the chunk swizzle above), with two transposing LDS reads.  Any
// [row][d] tile works the same way (the backward reads K^T, Q^T, dO^T so).  Within each
// group of 16 lanes the read hands lane 4 a + b element b of the 8-byte chunks
// addressed by lanes a, a + 4, a + 8, a + 12; so lane i of group g addresses
// key key0 + 8 (g / 2) + 4 r + i / 4 at dims 32 db + 16 (g % 2) + 4 (i % 4),
// and lane l then holds dim 32 db + l % 32 for keys key0 + 8 (l / 32) + 0..7,
// the order of the P operand.
template <int D>
__device__ __forceinline__ bf16x8 v_operand_tr(const unsigned char* Vs, int key0, int db, int lane) {
  constexpr int ROWB = D * 2;
  const int g = lane >> 4, i = lane & 15;
  const int dcol = 32 * db + 16 * (g & 1) + 4 * (i & 3);          // first of 4 dims
  const int chunk = (dcol * 2) >> 4, sub = (dcol * 2) & 15;
  bf16x4 h[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int key = key0 + 8 * (g >> 1) + 4 * r + (i >> 2);
    const unsigned char* a = Vs + key * ROWB + ((chunk ^ swz<ROWB / 16>(key)) * 16) + sub;
    h[r] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)a);
  }
  return bf16x8{h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
}

}  // namespace na
