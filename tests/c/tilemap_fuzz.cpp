// The host tile-map builder, chooser and time model on random geometries,
// built with AddressSanitizer and UndefinedBehaviorSanitizer (host code
// only): internal consistency of every map, and no memory or UB errors.
// Usage: tilemap_fuzz [iterations]
#include <cstdio>
#include <cstdlib>
#include <random>
#include "tilemap.hpp"
using namespace na;
int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 300;
  std::mt19937 rng(7);
  long checked = 0;
  for (int it = 0; it < iters; ++it) {
    Geometry g;
    for (int d = 0; d < 3; ++d) {
      g.L[d] = 1 + rng() % 40;
      g.w[d] = 1 + rng() % g.L[d];
      g.s[d] = 1 + rng() % g.w[d];
    }
    if (!check_geometry(g).empty()) { std::printf("bad geometry rejected?\n"); return 1; }
    int tq[3], tk[3];
    for (int d = 0; d < 3; ++d) { tq[d] = 1 << (rng() % 5); tk[d] = 1 << (rng() % 5); }
    TileMap m = build_tile_map(g, tq, tk);
    TileCounts c = count_tiles(g, tq, tk);
    const size_t nq = m.n_full.size();
    if (m.qptr.size() != nq + 1 || (int64_t)m.kv_idx.size() != c.nnz || c.n_q_tiles != (int64_t)nq) {
      std::printf("size mismatch at %d\n", it); return 1;
    }
    int64_t nf = 0;
    for (size_t r = 0; r < nq; ++r) {
      if (m.qptr[r] > m.qptr[r + 1] || m.n_full[r] > m.qptr[r + 1] - m.qptr[r]) { std::printf("row %zu bad\n", r); return 1; }
      nf += m.n_full[r];
      for (int32_t j = m.qptr[r]; j < m.qptr[r + 1]; ++j)
        if (m.kv_idx[j] < 0 || m.kv_idx[j] >= c.n_kv_tiles) { std::printf("kv out of range\n"); return 1; }
    }
    if (nf != c.n_full) { std::printf("n_full mismatch\n"); return 1; }
    TransposedMap t = transpose_tile_map(m);
    if ((int64_t)t.q_idx.size() != c.nnz || (int64_t)t.n_full.size() != c.n_kv_tiles) { std::printf("transpose size\n"); return 1; }
    for (int fam = 0; fam < 3; ++fam) {
      int a[3], b[3];
      const Family f = fam == 0 ? Family::F32 : fam == 1 ? Family::MFMA16 : Family::FP8;
      const int D = fam == 0 ? 32 : 128;
      if (choose_tiles(g, D, f, a, b)) {
        TileCounts cc = count_tiles(g, a, b);
        (void)predict_kernel_ms(g, 2, 3, D, f, a, b, cc);
      }
      (void)tile_candidates(g, D, f);
    }
    ++checked;
  }
  std::printf("ok %ld geometries\n", checked);
  return 0;
}
