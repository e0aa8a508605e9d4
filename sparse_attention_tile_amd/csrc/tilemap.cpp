// Host tile-map builder for GNA.  See tilemap.hpp for the interval rules.
#include "tilemap.hpp"

#include <algorithm>
#include <cmath>
#include <array>
#include <limits>

namespace na {

int window_start(int i, int L, int w, int s) {
  // GNA page section 1.1: stride groups share the window of their leader,
  // the centre of the group; the window holds floor(w/2) keys before the
  // leader and is shifted to stay inside the grid.
  const int g = i / s;
  int lead = g * s + s / 2;
  if (lead > L - 1) lead = L - 1;
  int st = lead - w / 2;
  if (st < 0) st = 0;
  if (st > L - w) st = L - w;
  return st;
}

std::string check_geometry(const Geometry& g) {
  for (int d = 0; d < 3; ++d) {
    if (g.L[d] < 1 || g.w[d] < 1 || g.s[d] < 1)
      return "grid, window and stride must be >= 1 on every axis";
    if (g.s[d] > g.w[d]) return "stride larger than window on axis " + std::to_string(d);
    if (g.w[d] > g.L[d]) return "window larger than grid on axis " + std::to_string(d);
  }
  return "";
}

std::string check_tile(const int t[3]) {
  for (int d = 0; d < 3; ++d) {
    if (t[d] < 1 || t[d] > 1024 || (t[d] & (t[d] - 1)) != 0)
      return "tile extents must be powers of two in [1, 1024]";
  }
  return "";
}

std::vector<AxisRange> axis_ranges(int L, int w, int s, int tq, int tkv) {
  const int nq = ceil_div(L, tq);
  std::vector<AxisRange> r(nq);
  for (int a = 0; a < nq; ++a) {
    const int first = a * tq;
    const int last = std::min(L, (a + 1) * tq) - 1;
    const int sf = window_start(first, L, w, s);
    const int sl = window_start(last, L, w, s);
    AxisRange x;
    x.lo = sf / tkv;
    x.hi = (sl + w - 1) / tkv;
    // full: c*tkv >= sl, (c+1)*tkv <= sf + w, (c+1)*tkv <= L
    x.full_lo = ceil_div(sl, tkv);
    const int top = std::min(sf + w, L);
    x.full_hi = top / tkv - 1;
    if (x.full_lo < x.lo) x.full_lo = x.lo;
    if (x.full_hi > x.hi) x.full_hi = x.hi;
    r[a] = x;
  }
  return r;
}

TileCounts count_tiles(const Geometry& g, const int tq[3], const int tkv[3]) {
  TileCounts c;
  int64_t listed = 1, full = 1, nqt = 1, nkt = 1;
  for (int d = 0; d < 3; ++d) {
    auto r = axis_ranges(g.L[d], g.w[d], g.s[d], tq[d], tkv[d]);
    int64_t sl = 0, sf = 0;
    for (const auto& x : r) {
      sl += x.hi - x.lo + 1;
      sf += std::max(0, x.full_hi - x.full_lo + 1);
    }
    listed *= sl;
    full *= sf;
    nqt *= (int64_t)r.size();
    nkt *= ceil_div(g.L[d], tkv[d]);
  }
  c.n_q_tiles = nqt;
  c.n_kv_tiles = nkt;
  c.nnz = listed;
  c.n_full = full;
  const int64_t qtok = (int64_t)tq[0] * tq[1] * tq[2];
  const int64_t ktok = (int64_t)tkv[0] * tkv[1] * tkv[2];
  c.computed_slots = listed * qtok * ktok;
  c.effective_slots = (int64_t)g.L[0] * g.L[1] * g.L[2] * ((int64_t)g.w[0] * g.w[1] * g.w[2]);
  return c;
}

TileMap build_tile_map(const Geometry& g, const int tq[3], const int tkv[3]) {
  TileMap m;
  std::vector<AxisRange> r[3];
  for (int d = 0; d < 3; ++d) {
    r[d] = axis_ranges(g.L[d], g.w[d], g.s[d], tq[d], tkv[d]);
    m.nq[d] = (int)r[d].size();
    m.nk[d] = ceil_div(g.L[d], tkv[d]);
  }
  m.counts = count_tiles(g, tq, tkv);
  const int64_t nQ = (int64_t)m.nq[0] * m.nq[1] * m.nq[2];
  m.qptr.reserve(nQ + 1);
  m.n_full.reserve(nQ);
  m.kv_idx.reserve(m.counts.nnz);
  m.qptr.push_back(0);
  for (int a0 = 0; a0 < m.nq[0]; ++a0)
    for (int a1 = 0; a1 < m.nq[1]; ++a1)
      for (int a2 = 0; a2 < m.nq[2]; ++a2) {
        const AxisRange& x0 = r[0][a0];
        const AxisRange& x1 = r[1][a1];
        const AxisRange& x2 = r[2][a2];
        // full tiles: product of the full ranges, row-major ascending
        int nf = 0;
        for (int c0 = x0.full_lo; c0 <= x0.full_hi; ++c0)
          for (int c1 = x1.full_lo; c1 <= x1.full_hi; ++c1)
            for (int c2 = x2.full_lo; c2 <= x2.full_hi; ++c2) {
              m.kv_idx.push_back((c0 * m.nk[1] + c1) * m.nk[2] + c2);
              ++nf;
            }
        // boundary tiles: the rest of the listed product, ascending
        for (int c0 = x0.lo; c0 <= x0.hi; ++c0) {
          const bool f0 = c0 >= x0.full_lo && c0 <= x0.full_hi;
          for (int c1 = x1.lo; c1 <= x1.hi; ++c1) {
            const bool f1 = c1 >= x1.full_lo && c1 <= x1.full_hi;
            for (int c2 = x2.lo; c2 <= x2.hi; ++c2) {
              const bool f2 = c2 >= x2.full_lo && c2 <= x2.full_hi;
              if (f0 && f1 && f2) continue;
              m.kv_idx.push_back((c0 * m.nk[1] + c1) * m.nk[2] + c2);
            }
          }
        }
        m.n_full.push_back(nf);
        m.qptr.push_back((int32_t)m.kv_idx.size());
      }
  return m;
}

TransposedMap transpose_tile_map(const TileMap& m) {
  TransposedMap t;
  const int64_t nK = (int64_t)m.nk[0] * m.nk[1] * m.nk[2];
  const int64_t nQ = (int64_t)m.n_full.size();
  std::vector<int32_t> nf(nK, 0), nb(nK, 0);
  for (int64_t a = 0; a < nQ; ++a)
    for (int32_t e = m.qptr[a]; e < m.qptr[a + 1]; ++e) {
      const bool full = e - m.qptr[a] < m.n_full[a];
      (full ? nf : nb)[m.kv_idx[e]]++;
    }
  t.kptr.assign(nK + 1, 0);
  for (int64_t c = 0; c < nK; ++c) t.kptr[c + 1] = t.kptr[c] + nf[c] + nb[c];
  t.n_full = nf;
  t.q_idx.assign(t.kptr[nK], 0);
  std::vector<int32_t> fpos(nK), bpos(nK);
  for (int64_t c = 0; c < nK; ++c) {
    fpos[c] = t.kptr[c];
    bpos[c] = t.kptr[c] + nf[c];
  }
  // Q tiles visited in ascending order, so each part comes out ascending
  for (int64_t a = 0; a < nQ; ++a)
    for (int32_t e = m.qptr[a]; e < m.qptr[a + 1]; ++e) {
      const int32_t c = m.kv_idx[e];
      const bool full = e - m.qptr[a] < m.n_full[a];
      t.q_idx[full ? fpos[c]++ : bpos[c]++] = (int32_t)a;
    }
  return t;
}

namespace {

int pow2_ceil(int x) { int p = 1; while (p < x) p <<= 1; return p; }

// Power-of-two tile shapes with `tokens` tokens, each extent at most the
// grid extent rounded up to a power of two, and the W extent >= min_w.
void shapes_with_product(const Geometry& g, int tokens, std::vector<std::array<int, 3>>& out, int min_w) {
  const int cap0 = pow2_ceil(g.L[0]), cap1 = pow2_ceil(g.L[1]), cap2 = std::max(pow2_ceil(g.L[2]), min_w);
  for (int a = 1; a <= tokens && a <= cap0; a <<= 1)
    for (int b = 1; a * b <= tokens && b <= cap1; b <<= 1) {
      const int c = tokens / (a * b);
      if (a * b * c != tokens || c > cap2 || c < min_w) continue;
      out.push_back({a, b, c});
    }
  if (out.empty()) {
    // grid smaller than one tile: fill W, then H, then pad along T
    int rem = tokens;
    const int c = std::min(rem, cap2);
    rem /= c;
    const int b = std::min(rem, cap1);
    rem /= b;
    out.push_back({rem, b, c});
  }
}

// Relative cost of a (tile_q, tile_kv) pair: computed slots, with a penalty
// for masked tiles and for the less efficient kernel shapes.
double tile_cost(const TileCounts& c, double q_pen, double kv_pen) {
  const double bfrac = c.nnz ? (double)(c.nnz - c.n_full) / (double)c.nnz : 0.0;
  return (double)c.computed_slots * (1.0 + 0.35 * bfrac) * q_pen * kv_pen;
}

struct Opt { int tok; double pen; };

// Tile token counts a family's kernels take, with their relative per-slot
// cost (measured: the 128-query bf16 kernel is 1.3x slower per slot than the
// 256-query one, 64-key tiles 1.06x slower than 128-key ones).
bool family_options(Family fam, int head_dim, std::vector<Opt>& qopts, std::vector<Opt>& kopts, int& min_kv_w) {
  min_kv_w = 1;
  switch (fam) {
    case Family::F32:
      if (head_dim != 32 && head_dim != 64 && head_dim != 128) return false;
      qopts = {{64, 1.0}};
      kopts = {{64, 1.0}};
      return true;
    case Family::MFMA16:
    case Family::FP8:
      if (head_dim != 64 && head_dim != 128) return false;
      qopts = {{256, 1.0}, {128, 1.3}};
      kopts = {{128, 1.0}, {64, 1.06}};
      min_kv_w = 8;   // the boundary mask works on 8-key groups along W
      return true;
  }
  return false;
}

double shape_penalty(Family fam, int qtok, int ktok) {
  std::vector<Opt> qo, ko;
  int mw;
  if (!family_options(fam, 128, qo, ko, mw)) return 1.0;
  double p = 1.0;
  for (const auto& o : qo) if (o.tok == qtok) p *= o.pen;
  for (const auto& o : ko) if (o.tok == ktok) p *= o.pen;
  return p;
}

}  // namespace

std::vector<Candidate> tile_candidates(const Geometry& g, int head_dim, Family fam, int min_q_w) {
  std::vector<Opt> qopts, kopts;
  int min_kv_w = 1;
  std::vector<Candidate> out;
  if (!family_options(fam, head_dim, qopts, kopts, min_kv_w)) return out;
  for (const auto& qo : qopts) {
    std::vector<std::array<int, 3>> qs;
    shapes_with_product(g, qo.tok, qs, min_q_w);
    for (const auto& ko : kopts) {
      std::vector<std::array<int, 3>> ks;
      shapes_with_product(g, ko.tok, ks, min_kv_w);
      for (const auto& a : qs)
        for (const auto& b : ks) {
          Candidate cd;
          for (int d = 0; d < 3; ++d) { cd.tq[d] = a[d]; cd.tkv[d] = b[d]; }
          cd.c = count_tiles(g, cd.tq, cd.tkv);
          cd.cost = tile_cost(cd.c, qo.pen, ko.pen);
          out.push_back(cd);
        }
    }
  }
  // stable: among equal costs the enumeration order (larger Q tiles, larger
  // KV tiles, T-major shapes first) decides
  std::stable_sort(out.begin(), out.end(), [](const Candidate& x, const Candidate& y) { return x.cost < y.cost; });
  return out;
}

bool choose_tiles(const Geometry& g, int head_dim, Family fam, int tq[3], int tkv[3]) {
  const std::vector<Candidate> cs = tile_candidates(g, head_dim, fam);
  if (cs.empty()) return false;
  for (int d = 0; d < 3; ++d) { tq[d] = cs[0].tq[d]; tkv[d] = cs[0].tkv[d]; }
  return true;
}

// Time model.  The kernel runs one workgroup per (batch, head, Q tile); a CU
// holds up to `slots` of them at once (8-wave workgroups: 1, 4-wave: 2,
// 1-wave fp32: 8) and runs each one's KV-tile visits back to back.  A visit
// costs the tile's computed FLOPs (4 x Q slots x KV slots x D) at the family's
// measured per-CU rate, times the shape penalty, times (1 + kBoundary) when it
// is a boundary tile; `conc` resident workgroups share the CU, and a
// workgroup of w waves gets at most w / 8 of it.  Workgroups are dealt in
// rounds of 256 x slots; the time is rounds x one workgroup's average time,
// plus a launch overhead.  Calibration (one MI355X, kernel ms measured with
// HIP events; boxes differ by a few per cent):
//   bf16 D 128: 1.215e15 FLOP/s of computed work on full tiles (91 %-sparse
//   video, 12.5-13.1 ms); boundary tiles 1.11x (video sliding window, 23.5 %
//   boundary, 69.7-70.6 ms); fp8 D 128: 1.85e15 (4K image, 1.89-1.92 ms);
//   launch 15 us (64x64 image, 35-45 us); fp32: 4.3e13 (16x16 image); bf16
//   D 64: 0.93e15 (the video block problem at head_dim 64, 8.5 ms).
double family_rate(Family fam, int head_dim) {
  switch (fam) {
    case Family::MFMA16: return head_dim == 128 ? 1.215e15 : 0.93e15;
    case Family::FP8: return 1.85e15;
    case Family::F32: return 4.3e13;
  }
  return 1e15;
}

double predict_kernel_ms(const Geometry& g, int batch, int heads, int head_dim, Family fam, const int tq[3],
                         const int tkv[3], const TileCounts& c) {
  constexpr double kLaunchMs = 0.015, kBoundary = 0.11;
  constexpr int kCUs = 256;
  (void)g;
  const int qtok = tq[0] * tq[1] * tq[2], ktok = tkv[0] * tkv[1] * tkv[2];
  const int waves = fam == Family::F32 ? 1 : std::max(1, qtok / 32);
  const int slots = std::max(1, 8 / waves);
  const double n_wg = (double)batch * heads * (double)c.n_q_tiles;
  if (n_wg <= 0 || c.n_q_tiles == 0) return 0.0;
  const double conc = std::min((double)slots, std::ceil(n_wg / kCUs));
  const double per_cu_rate = family_rate(fam, head_dim) / kCUs;
  const double wg_rate = per_cu_rate * std::min(1.0, conc * waves / 8.0) / conc;
  const double tile_flop = 4.0 * qtok * ktok * head_dim * shape_penalty(fam, qtok, ktok);
  const double nb = (double)(c.nnz - c.n_full);
  const double wg_s = ((double)c.n_full + nb * (1.0 + kBoundary)) / (double)c.n_q_tiles * tile_flop / wg_rate;
  const double rounds = std::ceil(n_wg / (kCUs * (double)slots));
  return kLaunchMs + rounds * wg_s * 1e3;
}

}  // namespace na
