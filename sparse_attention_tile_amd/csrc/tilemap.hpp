// Host tile-map builder for GNA (pure C++17; no HIP dependency).
//
// GNA page ("GNA Sparse Attention Mechanism: Vision-Transformer Compute
// Optimisation in Practice"), section 1.1: the token grid is cut into
// fixed-size multi-dimensional Q and KV tiles, and the stride fixes the range
// of KV tiles each Q tile must visit; section 2.1: the fine-grained mask is
// only needed on KV tiles that are not fully inside the attention window.
//
// Everything here is integer interval arithmetic per axis.  On one axis the
// window start of a query is monotone in the query coordinate and moves by at
// most the stride (<= window) between neighbours, so over a Q tile
//   union        = [start(first), start(last) + w)     (contiguous)
//   intersection = [start(last),  start(first) + w)
// A KV tile is listed iff it meets the union on every axis, and is full iff
// on every axis it lies inside the intersection and holds no padding slot.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace na {

struct Geometry {
  int L[3];  // grid extents (T, H, W)
  int w[3];  // window
  int s[3];  // stride
};

// First key coordinate of the window of query coordinate i on one axis.
int window_start(int i, int L, int w, int s);

// Returns "" if the geometry is valid, else a message.
std::string check_geometry(const Geometry& g);
// Returns "" if every tile extent is a power of two in [1, 1024].
std::string check_tile(const int t[3]);

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int ilog2(int x) { int r = 0; while ((1 << r) < x) ++r; return r; }

// Per-axis KV-tile ranges of one Q tile (inclusive bounds; full range may
// be empty, then full_lo > full_hi).
struct AxisRange {
  int lo, hi;
  int full_lo, full_hi;
};

// Ranges for every Q tile of one axis.
std::vector<AxisRange> axis_ranges(int L, int w, int s, int tq, int tkv);

struct TileCounts {
  int64_t n_q_tiles = 0, n_kv_tiles = 0, nnz = 0, n_full = 0;
  int64_t computed_slots = 0, effective_slots = 0;
};

// Counts without materialising the map (they factor over axes).
TileCounts count_tiles(const Geometry& g, const int tq[3], const int tkv[3]);

struct TileMap {
  int nq[3] = {0, 0, 0};   // Q tiles per axis
  int nk[3] = {0, 0, 0};   // KV tiles per axis
  std::vector<int32_t> qptr;    // [nQ + 1]
  std::vector<int32_t> kv_idx;  // [nnz] row-major linear KV-tile index
  std::vector<int32_t> n_full;  // [nQ]
  TileCounts counts;
};

// Builds the CSR map: Q tiles in row-major order; in each row the full
// tiles (ascending), then the boundary tiles (ascending).
TileMap build_tile_map(const Geometry& g, const int tq[3], const int tkv[3]);

// The transpose of a tile map: for each KV tile (row-major index), the Q
// tiles whose rows list it -- full ones first, then boundary ones, each
// ascending (the backward's dK/dV kernel walks these rows).
struct TransposedMap {
  std::vector<int32_t> kptr;    // [nK + 1]
  std::vector<int32_t> q_idx;   // [nnz] row-major linear Q-tile index
  std::vector<int32_t> n_full;  // [nK]
};
TransposedMap transpose_tile_map(const TileMap& m);

// Kernel families the library has (tile token counts they take).
enum class Family { F32, MFMA16, FP8 };

// Chooses (tile_q, tile_kv) for a family by minimising a cost model over
// power-of-two tile shapes.  Returns false if the family has no kernel for
// head_dim.
bool choose_tiles(const Geometry& g, int head_dim, Family fam, int tq[3], int tkv[3]);

// One tile-shape candidate of a family, with its counts and relative cost.
struct Candidate {
  int tq[3], tkv[3];
  TileCounts c;
  double cost;
};

// Every candidate the chooser considers, sorted by cost (the first one is
// what choose_tiles returns).  Empty if the family has no kernel for head_dim.
// min_q_w: the smallest Q tile extent along W (the backward's dk/dv kernel
// needs 8; a narrower grid is then padded along W).
std::vector<Candidate> tile_candidates(const Geometry& g, int head_dim, Family fam, int min_q_w = 1);

// Predicted attention-kernel time (ms) on one MI355X: a per-CU serial model
// calibrated on the measured kernels (see the constants in tilemap.cpp).
double predict_kernel_ms(const Geometry& g, int batch, int heads, int head_dim, Family fam, const int tq[3],
                         const int tkv[3], const TileCounts& c);

}  // namespace na
