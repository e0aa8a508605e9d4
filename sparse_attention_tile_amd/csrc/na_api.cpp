// C ABI of libna.so: argument checks, the plan cache and the launch
// sequence of one GNA forward pass.  Declarations and their contracts are in
// include/na.h.
#include "na.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <tuple>

#include "forward_buffer.hpp"
#include "kernels.hpp"
#include "tilemap.hpp"

namespace {

thread_local std::string g_err;

na_status fail(na_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

na::Geometry make_geom(const int grid[3], const int window[3], const int stride[3]) {
  na::Geometry g;
  for (int d = 0; d < 3; ++d) {
    g.L[d] = grid[d];
    g.w[d] = window[d];
    g.s[d] = stride[d];
  }
  return g;
}

int elem_bytes(na_dtype dt) {
  switch (dt) {
    case NA_F32: return 4;
    case NA_BF16: return 2;
    case NA_FP8_E4M3: return 1;
  }
  return 0;
}

int out_bytes(na_dtype dt) { return dt == NA_F32 ? 4 : 2; }

na::Family family(na_dtype dt) {
  switch (dt) {
    case NA_F32: return na::Family::F32;
    case NA_BF16: return na::Family::MFMA16;
    case NA_FP8_E4M3: return na::Family::FP8;
  }
  return na::Family::F32;
}

bool valid_dtype(int dt) { return dt == NA_F32 || dt == NA_BF16 || dt == NA_FP8_E4M3; }

bool kernel_supported(na_dtype dt, int D, int qtok, int ktok) {
  switch (dt) {
    case NA_F32: return na::attn_f32_supported(D, qtok, ktok);
    case NA_BF16: return na::attn_bf16_supported(D, qtok, ktok);
    case NA_FP8_E4M3: return na::attn_fp8_supported(D, qtok, ktok);
  }
  return false;
}

// ---------------------------------------------------------------------------
// plan cache: host tile map + its device copy, per (device, geometry, tiles)
// ---------------------------------------------------------------------------

struct Plan {
  na::TileMap map;
  int32_t* d_qptr = nullptr;
  int32_t* d_kv = nullptr;
  int32_t* d_nfull = nullptr;
  // transposed map (built the first time the backward needs it)
  bool has_t = false;
  int32_t* d_tptr = nullptr;
  int32_t* d_tidx = nullptr;
  int32_t* d_tnfull = nullptr;
  ~Plan() {
    for (int32_t* q : {d_qptr, d_kv, d_nfull, d_tptr, d_tidx, d_tnfull})
      if (q) (void)hipFree(q);
  }
};

using PlanKey = std::tuple<int, int, int, int, int, int, int, int, int, int, int, int, int, int, int, int,
                           int, int, int>;

std::mutex g_mu;
std::map<PlanKey, std::unique_ptr<Plan>>& plans() {
  static auto* m = new std::map<PlanKey, std::unique_ptr<Plan>>();
  return *m;
}

// Host tile maps of the fixed-buffer forward (na_forward_noalloc), per
// geometry and tile shapes: host memory only, the map is copied into the
// device buffer on each call.
std::map<PlanKey, std::unique_ptr<na::TileMap>>& host_maps() {
  static auto* m = new std::map<PlanKey, std::unique_ptr<na::TileMap>>();
  return *m;
}

na_status get_plan(const na::Geometry& g, const int tq[3], const int tkv[3], Plan** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(NA_ERR_HIP, "hipGetDevice failed");
  // Test hook: NA_FORCE_MASK=1 marks every listed KV tile as a boundary
  // tile, so the kernels mask full tiles too (results must not change).
  const char* fm = std::getenv("NA_FORCE_MASK");
  const int force_mask = (fm && fm[0] == '1') ? 1 : 0;
  PlanKey key{dev,      g.L[0],   g.L[1],   g.L[2],   g.w[0], g.w[1], g.w[2],
              g.s[0],   g.s[1],   g.s[2],   tq[0],  tq[1],  tq[2],
              tkv[0],   tkv[1],   tkv[2],   force_mask, 0,  0};
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = plans().find(key);
  if (it != plans().end()) {
    *out = it->second.get();
    return NA_OK;
  }
  auto p = std::make_unique<Plan>();
  p->map = na::build_tile_map(g, tq, tkv);
  if (force_mask) std::fill(p->map.n_full.begin(), p->map.n_full.end(), 0);
  const size_t nq = p->map.n_full.size();
  const size_t nnz = p->map.kv_idx.size();
  if (hipMalloc(&p->d_qptr, (nq + 1) * sizeof(int32_t)) != hipSuccess ||
      hipMalloc(&p->d_kv, (nnz ? nnz : 1) * sizeof(int32_t)) != hipSuccess ||
      hipMalloc(&p->d_nfull, nq * sizeof(int32_t)) != hipSuccess)
    return fail(NA_ERR_HIP, "hipMalloc of the device tile map failed");
  if (hipMemcpy(p->d_qptr, p->map.qptr.data(), (nq + 1) * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess ||
      (nnz && hipMemcpy(p->d_kv, p->map.kv_idx.data(), nnz * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess) ||
      hipMemcpy(p->d_nfull, p->map.n_full.data(), nq * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess)
    return fail(NA_ERR_HIP, "upload of the device tile map failed");
  *out = p.get();
  plans()[key] = std::move(p);
  return NA_OK;
}

// The plan plus its transposed map on the device.
na_status get_plan_t(const na::Geometry& g, const int tq[3], const int tkv[3], Plan** out) {
  Plan* p = nullptr;
  na_status st = get_plan(g, tq, tkv, &p);
  if (st != NA_OK) return st;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!p->has_t) {
    // a failed attempt leaves no device memory behind (the next call retries)
    auto drop = [&]() {
      for (int32_t** q : {&p->d_tptr, &p->d_tidx, &p->d_tnfull}) {
        if (*q) (void)hipFree(*q);
        *q = nullptr;
      }
    };
    const na::TransposedMap t = na::transpose_tile_map(p->map);
    const size_t nk = t.n_full.size(), nnz = t.q_idx.size();
    if (hipMalloc(&p->d_tptr, (nk + 1) * sizeof(int32_t)) != hipSuccess ||
        hipMalloc(&p->d_tidx, (nnz ? nnz : 1) * sizeof(int32_t)) != hipSuccess ||
        hipMalloc(&p->d_tnfull, (nk ? nk : 1) * sizeof(int32_t)) != hipSuccess) {
      drop();
      return fail(NA_ERR_HIP, "hipMalloc of the transposed tile map failed");
    }
    if (hipMemcpy(p->d_tptr, t.kptr.data(), (nk + 1) * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess ||
        (nnz && hipMemcpy(p->d_tidx, t.q_idx.data(), nnz * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess) ||
        (nk && hipMemcpy(p->d_tnfull, t.n_full.data(), nk * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess)) {
      drop();
      return fail(NA_ERR_HIP, "upload of the transposed tile map failed");
    }
    p->has_t = true;
  }
  *out = p;
  return NA_OK;
}

// Test and tuning hook: NA_TILE_Q / NA_TILE_KV="t,h,w" replace the chosen
// tile shape (the kernel-shape check still applies).  Returns false if the
// variable is set but malformed.
bool tile_override(const char* var, int t[3]) {
  const char* s = std::getenv(var);
  if (!s || !*s) return true;
  int v[3];
  if (std::sscanf(s, "%d,%d,%d", &v[0], &v[1], &v[2]) != 3) return false;
  if (!na::check_tile(v).empty()) return false;
  for (int d = 0; d < 3; ++d) t[d] = v[d];
  return true;
}

// One launch holds fewer than 2^32 work-items (the dispatch packet's grid
// size is 32-bit); the largest kernels here use 512 threads per workgroup.
constexpr int64_t kMaxWorkItems = int64_t(1) << 32;
constexpr int kMaxThreadsPerWg = 512;

// Sizes of the tile-ordered buffers of one problem.
struct Layout {
  int tq[3], tkv[3];
  int nq[3], nk[3];
  size_t q_bytes, kv_bytes, o_bytes, lse_bytes;
  size_t off_q, off_k, off_v, off_o, off_lse, total;
  size_t kv_total;   // k and v copies only (offsets 0 and round256(kv_bytes))
};

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

na_status check_problem(int batch, int heads, int head_dim, const int grid[3], const int window[3],
                        const int stride[3], int dtype, Layout* lay) {
  if (!grid || !window || !stride) return fail(NA_ERR_INVALID_ARG, "grid, window and stride must be non-null");
  if (batch < 0 || heads < 0) return fail(NA_ERR_INVALID_ARG, "batch and heads must be >= 0");
  if (!valid_dtype(dtype)) return fail(NA_ERR_INVALID_ARG, "unknown dtype");
  na::Geometry g = make_geom(grid, window, stride);
  std::string e = na::check_geometry(g);
  if (!e.empty()) return fail(NA_ERR_INVALID_ARG, e);
  const int64_t N = (int64_t)grid[0] * grid[1] * grid[2];
  if (N > (int64_t(1) << 30)) return fail(NA_ERR_UNSUPPORTED, "more than 2^30 tokens");
  na_dtype dt = (na_dtype)dtype;
  if (!na::choose_tiles(g, head_dim, family(dt), lay->tq, lay->tkv))
    return fail(NA_ERR_UNSUPPORTED, "no kernel for head_dim " + std::to_string(head_dim) + " in this dtype");
  if (!tile_override("NA_TILE_Q", lay->tq) || !tile_override("NA_TILE_KV", lay->tkv))
    return fail(NA_ERR_INVALID_ARG, "NA_TILE_Q / NA_TILE_KV must be three powers of two, e.g. 4,8,8");
  const int qtok = lay->tq[0] * lay->tq[1] * lay->tq[2];
  const int ktok = lay->tkv[0] * lay->tkv[1] * lay->tkv[2];
  if (!kernel_supported(dt, head_dim, qtok, ktok) || (dt != NA_F32 && !na::attn_bf16_tile_ok(lay->tkv)))
    return fail(NA_ERR_UNSUPPORTED, "no kernel for this head_dim / tile combination");
  int64_t npq = 1, npk = 1, ntq = 1, ntk = 1;
  for (int d = 0; d < 3; ++d) {
    lay->nq[d] = na::ceil_div(grid[d], lay->tq[d]);
    lay->nk[d] = na::ceil_div(grid[d], lay->tkv[d]);
    npq *= (int64_t)lay->nq[d] * lay->tq[d];
    npk *= (int64_t)lay->nk[d] * lay->tkv[d];
    ntq *= lay->nq[d];
    ntk *= lay->nk[d];
  }
  if ((int64_t)batch * heads * std::max(ntq, ntk) * kMaxThreadsPerWg >= kMaxWorkItems)
    return fail(NA_ERR_UNSUPPORTED, "batch * heads * tiles too large for one launch (fewer than 2^23 workgroups)");
  const size_t bh = (size_t)batch * heads;
  const int eb = elem_bytes(dt);
  lay->q_bytes = bh * npq * head_dim * eb;
  lay->kv_bytes = bh * npk * head_dim * eb;
  lay->o_bytes = bh * npq * head_dim * out_bytes(dt);
  lay->lse_bytes = bh * npq * sizeof(float);
  lay->off_q = 0;
  lay->off_k = lay->off_q + round256(lay->q_bytes);
  lay->off_v = lay->off_k + round256(lay->kv_bytes);
  lay->off_o = lay->off_v + round256(lay->kv_bytes);
  lay->off_lse = lay->off_o + round256(lay->o_bytes);
  lay->total = lay->off_lse + round256(lay->lse_bytes);
  lay->kv_total = 2 * round256(lay->kv_bytes);
  return NA_OK;
}

// Which form na_forward takes (the values of na_forward_mode): 0 permutes q,
// k, v and unpermutes out, lse; 1 permutes k, v only (bf16 and fp8: the
// kernel reads q and writes out / lse in grid order); 2 permutes nothing
// (bf16 without a workspace).  Test hook: NA_NO_FUSED=1 forces form 0.
int forward_mode(na_dtype dt, int head_dim, bool with_workspace) {
  const char* e = std::getenv("NA_NO_FUSED");
  if (e && e[0] == '1') return 0;
  if (dt == NA_FP8_E4M3 && head_dim == 128) return 1;   // no permutation-free fp8 form: needs the workspace
  if (dt != NA_BF16 || !na::attn_bf16_grid_io_supported(head_dim)) return 0;
  return with_workspace ? 1 : 2;
}

na_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return NA_OK;
  return fail(NA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

na_status check_tile_args(int batch, int heads, int head_dim, const int grid[3], const int tile[3], int eb) {
  if (!grid || !tile) return fail(NA_ERR_INVALID_ARG, "grid and tile must be non-null");
  if (batch < 0 || heads < 0 || head_dim < 1) return fail(NA_ERR_INVALID_ARG, "batch, heads >= 0 and head_dim >= 1 needed");
  for (int d = 0; d < 3; ++d)
    if (grid[d] < 1) return fail(NA_ERR_INVALID_ARG, "grid extents must be >= 1");
  std::string e = na::check_tile(tile);
  if (!e.empty()) return fail(NA_ERR_INVALID_ARG, e);
  if (eb != 1 && eb != 2 && eb != 4) return fail(NA_ERR_INVALID_ARG, "elem_bytes must be 1, 2 or 4");
  const int row = head_dim * eb;
  if (row % 16 != 0 || ((row / 16) & (row / 16 - 1)) != 0)
    return fail(NA_ERR_UNSUPPORTED, "head_dim * elem_bytes must be 16 times a power of two");
  const int64_t tt = (int64_t)tile[0] * tile[1] * tile[2];
  if (tt > 1024) return fail(NA_ERR_UNSUPPORTED, "more than 1024 tokens per tile");
  if ((int64_t)grid[0] * grid[1] * grid[2] > (int64_t(1) << 30)) return fail(NA_ERR_UNSUPPORTED, "more than 2^30 tokens");
  int64_t ntiles = 1;
  for (int d = 0; d < 3; ++d) ntiles *= na::ceil_div(grid[d], tile[d]);
  if ((int64_t)batch * heads * ntiles * 256 >= kMaxWorkItems)   // one 256-thread workgroup per tile
    return fail(NA_ERR_UNSUPPORTED, "batch * heads * tiles too large for one launch");
  return NA_OK;
}

}  // namespace

extern "C" {

const char* na_last_error(void) { return g_err.c_str(); }

void na_release_cache(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  plans().clear();
  host_maps().clear();
}

na_status na_choose_tiles(const int grid[3], const int window[3], const int stride[3], int head_dim,
                          na_dtype dtype, int tile_q[3], int tile_kv[3]) {
  g_err.clear();
  if (!tile_q || !tile_kv) return fail(NA_ERR_INVALID_ARG, "tile_q and tile_kv must be non-null");
  Layout lay;
  na_status st = check_problem(1, 1, head_dim, grid, window, stride, (int)dtype, &lay);
  if (st != NA_OK) return st;
  for (int d = 0; d < 3; ++d) {
    tile_q[d] = lay.tq[d];
    tile_kv[d] = lay.tkv[d];
  }
  return NA_OK;
}

static void fill_sim(int batch, int heads, int head_dim, const na::Geometry& g, na_dtype dtype, const int tq[3],
                     const int tkv[3], const na::TileCounts& c, double cost, na_sim_result* r) {
  for (int d = 0; d < 3; ++d) {
    r->tile_q[d] = tq[d];
    r->tile_kv[d] = tkv[d];
  }
  r->stats.n_q_tiles = c.n_q_tiles;
  r->stats.n_kv_tiles = c.n_kv_tiles;
  r->stats.nnz = c.nnz;
  r->stats.n_full = c.n_full;
  r->stats.n_boundary = c.nnz - c.n_full;
  r->stats.computed_slots = c.computed_slots;
  r->stats.effective_slots = c.effective_slots;
  r->tile_efficiency = c.computed_slots ? (double)c.effective_slots / (double)c.computed_slots : 1.0;
  const double N = (double)g.L[0] * g.L[1] * g.L[2];
  const double W = (double)g.w[0] * g.w[1] * g.w[2];
  r->flop_ratio_vs_dense = N / W;
  // the dense call: window = grid, stride 1, with the tiles it would choose
  na::Geometry dg = g;
  for (int d = 0; d < 3; ++d) {
    dg.w[d] = g.L[d];
    dg.s[d] = 1;
  }
  int dq[3], dk[3];
  double dense_computed = N * N;
  if (na::choose_tiles(dg, head_dim, family(dtype), dq, dk))
    dense_computed = (double)na::count_tiles(dg, dq, dk).computed_slots;
  r->speedup_bound = c.computed_slots ? dense_computed / (double)c.computed_slots : 0.0;
  r->perfectly_block_sparse = c.nnz == c.n_full ? 1 : 0;
  r->form = forward_mode(dtype, head_dim, true);
  r->cost = cost;
  r->predicted_kernel_ms = na::predict_kernel_ms(g, batch, heads, head_dim, family(dtype), tq, tkv, c);
  // permutation passes at the measured ~5 TB/s (bytes read + written) plus
  // ~8 us per launch
  int64_t npq = 1, npk = 1;
  for (int d = 0; d < 3; ++d) {
    npq *= (int64_t)na::ceil_div(g.L[d], tq[d]) * tq[d];
    npk *= (int64_t)na::ceil_div(g.L[d], tkv[d]) * tkv[d];
  }
  const double bh = (double)batch * heads, eb = elem_bytes(dtype), ob = out_bytes(dtype);
  double bytes = 2.0 * bh * (N + (double)npk) * head_dim * eb;   // k and v
  if (r->form == 0)
    bytes += bh * (N + (double)npq) * head_dim * eb + bh * (N + (double)npq) * (head_dim * ob + 4.0);
  const int launches = r->form == 0 ? 5 : 2;
  r->predicted_forward_ms = r->predicted_kernel_ms + bytes / 5.0e12 * 1e3 + launches * 0.008;
}

na_status na_simulate(int batch, int heads, int head_dim, const int grid[3], const int window[3], const int stride[3],
                      na_dtype dtype, const int tile_q[3], const int tile_kv[3], na_sim_result* out) {
  g_err.clear();
  if (!out) return fail(NA_ERR_INVALID_ARG, "out must be non-null");
  if ((tile_q == nullptr) != (tile_kv == nullptr)) return fail(NA_ERR_INVALID_ARG, "pass both tile shapes or neither");
  Layout lay;
  na_status st = check_problem(batch, heads, head_dim, grid, window, stride, (int)dtype, &lay);
  if (st != NA_OK) return st;
  na::Geometry g = make_geom(grid, window, stride);
  int tq[3], tk[3];
  for (int d = 0; d < 3; ++d) {
    tq[d] = tile_q ? tile_q[d] : lay.tq[d];
    tk[d] = tile_kv ? tile_kv[d] : lay.tkv[d];
  }
  if (!na::check_tile(tq).empty() || !na::check_tile(tk).empty())
    return fail(NA_ERR_INVALID_ARG, "tile extents must be powers of two");
  const na::TileCounts c = na::count_tiles(g, tq, tk);
  double cost = -1.0;
  for (const auto& cd : na::tile_candidates(g, head_dim, family(dtype)))
    if (std::equal(cd.tq, cd.tq + 3, tq) && std::equal(cd.tkv, cd.tkv + 3, tk)) cost = cd.cost;
  fill_sim(batch, heads, head_dim, g, dtype, tq, tk, c, cost, out);
  return NA_OK;
}

int na_tile_candidates(int batch, int heads, int head_dim, const int grid[3], const int window[3],
                       const int stride[3], na_dtype dtype, na_sim_result* out, int capacity) {
  g_err.clear();
  if (capacity < 0 || (capacity > 0 && !out)) return fail(NA_ERR_INVALID_ARG, "out must hold capacity entries");
  Layout lay;
  na_status st = check_problem(batch, heads, head_dim, grid, window, stride, (int)dtype, &lay);
  if (st != NA_OK) return st;
  na::Geometry g = make_geom(grid, window, stride);
  const auto cs = na::tile_candidates(g, head_dim, family(dtype));
  for (int i = 0; i < (int)cs.size() && i < capacity; ++i)
    fill_sim(batch, heads, head_dim, g, dtype, cs[i].tq, cs[i].tkv, cs[i].c, cs[i].cost, &out[i]);
  return (int)cs.size();
}

na_status na_build_tile_map(const int grid[3], const int window[3], const int stride[3], const int tile_q[3],
                            const int tile_kv[3], int32_t* qptr, int32_t* kv_idx, int32_t* n_full,
                            int64_t kv_capacity, int64_t* nnz_out, na_tilemap_stats* stats) {
  g_err.clear();
  if (!grid || !window || !stride || !tile_q || !tile_kv)
    return fail(NA_ERR_INVALID_ARG, "geometry and tile arrays must be non-null");
  na::Geometry g = make_geom(grid, window, stride);
  std::string e = na::check_geometry(g);
  if (e.empty()) e = na::check_tile(tile_q);
  if (e.empty()) e = na::check_tile(tile_kv);
  if (!e.empty()) return fail(NA_ERR_INVALID_ARG, e);
  na::TileCounts c = na::count_tiles(g, tile_q, tile_kv);
  if (c.nnz > INT32_MAX || c.n_q_tiles > INT32_MAX)
    return fail(NA_ERR_UNSUPPORTED, "tile map larger than 2^31 entries");
  if (nnz_out) *nnz_out = c.nnz;
  if (stats) {
    stats->n_q_tiles = c.n_q_tiles;
    stats->n_kv_tiles = c.n_kv_tiles;
    stats->nnz = c.nnz;
    stats->n_full = c.n_full;
    stats->n_boundary = c.nnz - c.n_full;
    stats->computed_slots = c.computed_slots;
    stats->effective_slots = c.effective_slots;
  }
  if (!qptr && !kv_idx && !n_full) return NA_OK;
  if (kv_idx && kv_capacity < c.nnz) return fail(NA_ERR_INVALID_ARG, "kv_capacity smaller than nnz");
  na::TileMap m = na::build_tile_map(g, tile_q, tile_kv);
  if (qptr) std::memcpy(qptr, m.qptr.data(), m.qptr.size() * sizeof(int32_t));
  if (kv_idx && !m.kv_idx.empty()) std::memcpy(kv_idx, m.kv_idx.data(), m.kv_idx.size() * sizeof(int32_t));
  if (n_full) std::memcpy(n_full, m.n_full.data(), m.n_full.size() * sizeof(int32_t));
  return NA_OK;
}

size_t na_workspace_bytes(int batch, int heads, int head_dim, const int grid[3], const int window[3],
                          const int stride[3], na_dtype dtype) {
  g_err.clear();
  Layout lay;
  if (check_problem(batch, heads, head_dim, grid, window, stride, (int)dtype, &lay) != NA_OK) return 0;
  if (lay.total && forward_mode(dtype, head_dim, true) == 1) return lay.kv_total;
  return lay.total;
}

int na_forward_mode(na_dtype dtype, int head_dim, int with_workspace) {
  return forward_mode(dtype, head_dim, with_workspace != 0);
}

na_status na_permute(const void* x, void* xt, int batch, int heads, int head_dim, const int grid[3],
                     const int tile[3], int elem_bytes, int transpose, void* stream) {
  g_err.clear();
  na_status st = check_tile_args(batch, heads, head_dim, grid, tile, elem_bytes);
  if (st != NA_OK) return st;
  if (!x || !xt) return fail(NA_ERR_INVALID_ARG, "x and xt must be non-null");
  if (!aligned16(x) || !aligned16(xt)) return fail(NA_ERR_INVALID_ARG, "x and xt must be 16-byte aligned");
  if (transpose != 0 && transpose != 1) return fail(NA_ERR_INVALID_ARG, "transpose must be 0 or 1");
  if (transpose) {
    const int tt = tile[0] * tile[1] * tile[2];
    if (tt * elem_bytes % 16 != 0)
      return fail(NA_ERR_UNSUPPORTED, "transposed tiles need tile_tokens * elem_bytes to be a multiple of 16");
    if (na::permute_transpose_lds_bytes(head_dim, tt, elem_bytes) > 65536)
      return fail(NA_ERR_UNSUPPORTED, "transposed tile does not fit in 64 KiB of LDS");
  }
  if (batch == 0 || heads == 0) return NA_OK;
  return hip_status(na::launch_permute(x, xt, batch, heads, head_dim, grid, tile, elem_bytes, transpose,
                                       (hipStream_t)stream),
                    "permute launch");
}

na_status na_unpermute(const void* xt, void* x, int batch, int heads, int head_dim, const int grid[3],
                       const int tile[3], int elem_bytes, void* stream) {
  g_err.clear();
  na_status st = check_tile_args(batch, heads, head_dim, grid, tile, elem_bytes);
  if (st != NA_OK) return st;
  if (!x || !xt) return fail(NA_ERR_INVALID_ARG, "x and xt must be non-null");
  if (!aligned16(x) || !aligned16(xt)) return fail(NA_ERR_INVALID_ARG, "x and xt must be 16-byte aligned");
  if (batch == 0 || heads == 0) return NA_OK;
  return hip_status(na::launch_unpermute(xt, x, batch, heads, head_dim, grid, tile, elem_bytes,
                                         (hipStream_t)stream),
                    "unpermute launch");
}

na_status na_unpermute_lse(const float* lse_t, float* lse, int batch, int heads, const int grid[3],
                           const int tile[3], void* stream) {
  g_err.clear();
  na_status st = check_tile_args(batch, heads, 4, grid, tile, 4);
  if (st != NA_OK) return st;
  if (!lse_t || !lse) return fail(NA_ERR_INVALID_ARG, "lse_t and lse must be non-null");
  if ((reinterpret_cast<uintptr_t>(lse_t) & 3u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(NA_ERR_INVALID_ARG, "lse_t and lse must be 4-byte aligned");
  if (batch == 0 || heads == 0) return NA_OK;
  return hip_status(na::launch_unpermute_lse(lse_t, lse, batch, heads, grid, tile, (hipStream_t)stream),
                    "lse unpermute launch");
}

// Kernel arguments of one problem: geometry, tiles and a device tile map.
static na::AttnArgs attn_args(const na::Geometry& g, const int32_t* qptr, const int32_t* kv_idx,
                              const int32_t* n_full, const int tq[3], const int tkv[3], int batch, int heads,
                              int head_dim, float scale) {
  na::AttnArgs a{};
  a.qptr = qptr;
  a.kv_idx = kv_idx;
  a.n_full = n_full;
  a.batch = batch;
  a.heads = heads;
  a.head_dim = head_dim;
  for (int d = 0; d < 3; ++d) {
    a.L[d] = g.L[d];
    a.w[d] = g.w[d];
    a.s[d] = g.s[d];
    a.tq[d] = tq[d];
    a.tkv[d] = tkv[d];
    a.nq[d] = na::ceil_div(g.L[d], tq[d]);
    a.nk[d] = na::ceil_div(g.L[d], tkv[d]);
  }
  a.scale = scale;
  a.v_scale = 1.0f;
  return a;
}

// ... with the map of a cached plan.
static na::AttnArgs attn_args(const na::Geometry& g, const Plan* plan, const int tq[3], const int tkv[3],
                              int batch, int heads, int head_dim, float scale) {
  return attn_args(g, plan->d_qptr, plan->d_kv, plan->d_nfull, tq, tkv, batch, heads, head_dim, scale);
}

static na_status attend_impl(const void* qt, const void* kt, const void* vt, void* ot, float* lse_t, int batch,
                             int heads, int head_dim, const int grid[3], const int window[3], const int stride[3],
                             const Layout& lay, float scale, na_dtype dtype, const float* qkv_scale,
                             int io_mode, hipStream_t stream) {
  na::Geometry g = make_geom(grid, window, stride);
  Plan* plan = nullptr;
  na_status st = get_plan(g, lay.tq, lay.tkv, &plan);
  if (st != NA_OK) return st;
  na::AttnArgs a = attn_args(g, plan, lay.tq, lay.tkv, batch, heads, head_dim, scale);
  a.qt = qt;
  a.kt = kt;
  a.vt = vt;
  a.ot = ot;
  a.lse_t = lse_t;
  a.io_mode = io_mode;
  if (dtype == NA_FP8_E4M3 && qkv_scale) {
    a.scale = scale * qkv_scale[0] * qkv_scale[1];
    a.v_scale = qkv_scale[2];
  }
  hipError_t e = hipSuccess;
  switch (dtype) {
    case NA_F32: e = na::launch_attn_f32(a, stream); break;
    case NA_BF16: e = na::launch_attn_bf16(a, stream); break;
    case NA_FP8_E4M3: e = na::launch_attn_fp8(a, stream); break;
  }
  return hip_status(e, "attention launch");
}

static na_status check_scales(float scale, na_dtype dtype, const float* qkv_scale) {
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(NA_ERR_INVALID_ARG, "scale must be finite and >= 0 (fold a sign into q)");
  if (dtype == NA_FP8_E4M3 && qkv_scale) {
    for (int i = 0; i < 3; ++i)
      if (!std::isfinite(qkv_scale[i]) || qkv_scale[i] <= 0.f)
        return fail(NA_ERR_INVALID_ARG, "qkv_scale entries must be finite and > 0");
  }
  return NA_OK;
}

na_status na_attend_tiled(const void* qt, const void* kt, const void* vt, void* ot, float* lse_t, int batch,
                          int heads, int head_dim, const int grid[3], const int window[3], const int stride[3],
                          const int tile_q[3], const int tile_kv[3], float scale, na_dtype dtype,
                          const float* qkv_scale, void* stream) {
  g_err.clear();
  Layout lay;
  na_status st = check_problem(batch, heads, head_dim, grid, window, stride, (int)dtype, &lay);
  if (st != NA_OK) return st;
  if (!tile_q || !tile_kv) return fail(NA_ERR_INVALID_ARG, "tile_q and tile_kv must be non-null");
  for (int d = 0; d < 3; ++d)
    if (tile_q[d] != lay.tq[d] || tile_kv[d] != lay.tkv[d])
      return fail(NA_ERR_INVALID_ARG, "tile shapes differ from na_choose_tiles()");
  if (batch == 0 || heads == 0) return NA_OK;
  if (!qt || !kt || !vt || !ot) return fail(NA_ERR_INVALID_ARG, "qt, kt, vt and ot must be non-null");
  if (!aligned16(qt) || !aligned16(kt) || !aligned16(vt) || !aligned16(ot) || (lse_t && !aligned16(lse_t)))
    return fail(NA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  st = check_scales(scale, dtype, qkv_scale);
  if (st != NA_OK) return st;
  return attend_impl(qt, kt, vt, ot, lse_t, batch, heads, head_dim, grid, window, stride, lay, scale, dtype,
                     qkv_scale, na::IO_TILE, (hipStream_t)stream);
}

na_status na_attend_kv_tiled(const void* q, const void* kt, const void* vt, void* out, float* lse, int batch,
                             int heads, int head_dim, const int grid[3], const int window[3], const int stride[3],
                             const int tile_kv[3], float scale, na_dtype dtype, const float* qkv_scale,
                             void* stream) {
  g_err.clear();
  Layout lay;
  na_status st = check_problem(batch, heads, head_dim, grid, window, stride, (int)dtype, &lay);
  if (st != NA_OK) return st;
  if (!tile_kv) return fail(NA_ERR_INVALID_ARG, "tile_kv must be non-null");
  for (int d = 0; d < 3; ++d)
    if (tile_kv[d] != lay.tkv[d]) return fail(NA_ERR_INVALID_ARG, "tile_kv differs from na_choose_tiles()");
  if (!((dtype == NA_BF16 && na::attn_bf16_grid_io_supported(head_dim)) || (dtype == NA_FP8_E4M3 && head_dim == 128)))
    return fail(NA_ERR_UNSUPPORTED, "grid-order q / out need bf16 with head_dim 64 / 128 or fp8 with 128");
  if (batch == 0 || heads == 0) return NA_OK;
  if (!q || !kt || !vt || !out) return fail(NA_ERR_INVALID_ARG, "q, kt, vt and out must be non-null");
  if (!aligned16(q) || !aligned16(kt) || !aligned16(vt) || !aligned16(out))
    return fail(NA_ERR_INVALID_ARG, "q, kt, vt and out must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(NA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  st = check_scales(scale, dtype, qkv_scale);
  if (st != NA_OK) return st;
  return attend_impl(q, kt, vt, out, lse, batch, heads, head_dim, grid, window, stride, lay, scale, dtype, qkv_scale,
                     na::IO_QO, (hipStream_t)stream);
}

na_status na_forward(const void* q, const void* k, const void* v, void* out, float* lse, int batch, int heads,
                     int head_dim, const int grid[3], const int window[3], const int stride[3], float scale,
                     na_dtype dtype, const float* qkv_scale, void* workspace, size_t workspace_bytes,
                     void* stream) {
  g_err.clear();
  Layout lay;
  na_status st = check_problem(batch, heads, head_dim, grid, window, stride, (int)dtype, &lay);
  if (st != NA_OK) return st;
  if (batch == 0 || heads == 0) return NA_OK;  // empty problem: nothing to do
  if (!q || !k || !v || !out) return fail(NA_ERR_INVALID_ARG, "q, k, v and out must be non-null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(NA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(NA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  st = check_scales(scale, dtype, qkv_scale);
  if (st != NA_OK) return st;
  const int mode = forward_mode(dtype, head_dim, workspace != nullptr);
  if (mode == 2) {
    // no workspace: the kernel gathers K / V tiles from grid order and reads
    // and writes q, out, lse in place (no permutation pass)
    return attend_impl(q, k, v, out, lse, batch, heads, head_dim, grid, window, stride, lay, scale, dtype,
                       qkv_scale, na::IO_GRID, (hipStream_t)stream);
  }
  if (!workspace) return fail(NA_ERR_INVALID_ARG, "workspace must be non-null for this dtype / head_dim");
  if (!aligned16(workspace)) return fail(NA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const size_t need = mode == 1 ? lay.kv_total : lay.total;
  if (workspace_bytes < need)
    return fail(NA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  if ((head_dim * elem_bytes(dtype)) % 16 != 0 || (head_dim * out_bytes(dtype)) % 16 != 0)
    return fail(NA_ERR_UNSUPPORTED, "head_dim too small for 16-byte rows");
  // Make sure the plan exists before anything is enqueued, so a failing
  // upload leaves the stream untouched.
  Plan* plan = nullptr;
  st = get_plan(make_geom(grid, window, stride), lay.tq, lay.tkv, &plan);
  if (st != NA_OK) return st;

  char* ws = static_cast<char*>(workspace);
  const int eb = elem_bytes(dtype);
  const int vtrans = dtype == NA_F32 ? 0 : 1;
  hipStream_t s = (hipStream_t)stream;
  if (mode == 1) {
    void* kt = ws;
    void* vt = ws + round256(lay.kv_bytes);
    if ((st = hip_status(na::launch_permute(k, kt, batch, heads, head_dim, grid, lay.tkv, eb, 0, s), "permute k")))
      return st;
    if ((st = hip_status(na::launch_permute(v, vt, batch, heads, head_dim, grid, lay.tkv, eb, vtrans, s),
                         "permute v")))
      return st;
    return attend_impl(q, kt, vt, out, lse, batch, heads, head_dim, grid, window, stride, lay, scale, dtype,
                       qkv_scale, na::IO_QO, s);
  }
  void* qt = ws + lay.off_q;
  void* kt = ws + lay.off_k;
  void* vt = ws + lay.off_v;
  void* ot = ws + lay.off_o;
  float* lt = reinterpret_cast<float*>(ws + lay.off_lse);
  if ((st = hip_status(na::launch_permute(q, qt, batch, heads, head_dim, grid, lay.tq, eb, 0, s), "permute q")))
    return st;
  if ((st = hip_status(na::launch_permute(k, kt, batch, heads, head_dim, grid, lay.tkv, eb, 0, s), "permute k")))
    return st;
  if ((st = hip_status(na::launch_permute(v, vt, batch, heads, head_dim, grid, lay.tkv, eb, vtrans, s),
                       "permute v")))
    return st;
  st = attend_impl(qt, kt, vt, ot, lse ? lt : nullptr, batch, heads, head_dim, grid, window, stride, lay, scale,
                   dtype, qkv_scale, na::IO_TILE, s);
  if (st != NA_OK) return st;
  if ((st = hip_status(na::launch_unpermute(ot, out, batch, heads, head_dim, grid, lay.tq, out_bytes(dtype), s),
                       "unpermute out")))
    return st;
  if (lse) {
    if ((st = hip_status(na::launch_unpermute_lse(lt, lse, batch, heads, grid, lay.tq, s), "unpermute lse")))
      return st;
  }
  return NA_OK;
}

// ---------------------------------------------------------------------------
// the forward with its tile map in a fixed device buffer (na_forward_noalloc)

}  // extern "C"

namespace na {

// na_forward's form 2 (the kernel reads q, k, v and writes out, lse in grid
// order) with the tile map copied on `stream` into the device memory
// get_buffer() returns (buffer_bytes long) instead of a cached allocation.
// The size check comes before get_buffer is called.
na_status forward_in_buffer(const void* q, const void* k, const void* v, void* out, float* lse, int batch,
                            int heads, int head_dim, const int grid[3], const int window[3], const int stride[3],
                            float scale, na_dtype dtype, void* stream, size_t buffer_bytes,
                            hipError_t (*get_buffer)(void** ptr)) {
  g_err.clear();
  Layout lay;
  na_status st = check_problem(batch, heads, head_dim, grid, window, stride, (int)dtype, &lay);
  if (st != NA_OK) return st;
  if (dtype != NA_BF16 || !na::attn_bf16_grid_io_supported(head_dim))
    return fail(NA_ERR_UNSUPPORTED, "na_forward_noalloc runs bf16 with head_dim 64 or 128");
  if (batch == 0 || heads == 0) return NA_OK;
  if (!q || !k || !v || !out) return fail(NA_ERR_INVALID_ARG, "q, k, v and out must be non-null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(NA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(NA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  st = check_scales(scale, dtype, nullptr);
  if (st != NA_OK) return st;
  const na::Geometry g = make_geom(grid, window, stride);
  const na::TileCounts c = na::count_tiles(g, lay.tq, lay.tkv);
  const size_t off_kv = round256((size_t)(c.n_q_tiles + 1) * sizeof(int32_t));
  const size_t off_nf = off_kv + round256((size_t)std::max<int64_t>(c.nnz, 1) * sizeof(int32_t));
  const size_t need = off_nf + round256((size_t)c.n_q_tiles * sizeof(int32_t));
  if (need > buffer_bytes)
    return fail(NA_ERR_UNSUPPORTED, "the tile map of this problem needs " + std::to_string(need) +
                                        " bytes, more than the fixed " + std::to_string(buffer_bytes) +
                                        "-byte device buffer of na_forward_noalloc");
  const na::TileMap* map = nullptr;
  {
    const char* fm = std::getenv("NA_FORCE_MASK");
    const int force_mask = (fm && fm[0] == '1') ? 1 : 0;
    PlanKey key{-1,        g.L[0],    g.L[1],    g.L[2],    g.w[0], g.w[1], g.w[2],
                g.s[0],    g.s[1],    g.s[2],    lay.tq[0], lay.tq[1], lay.tq[2],
                lay.tkv[0], lay.tkv[1], lay.tkv[2], force_mask, 0,        0};
    std::lock_guard<std::mutex> lk(g_mu);
    auto& hm = host_maps();
    auto it = hm.find(key);
    if (it == hm.end()) {
      auto m = std::make_unique<na::TileMap>(na::build_tile_map(g, lay.tq, lay.tkv));
      if (force_mask) std::fill(m->n_full.begin(), m->n_full.end(), 0);
      it = hm.emplace(key, std::move(m)).first;
    }
    map = it->second.get();
  }
  void* base = nullptr;
  if ((st = hip_status(get_buffer(&base), "device address of the fixed buffer"))) return st;
  char* b = static_cast<char*>(base);
  hipStream_t s = (hipStream_t)stream;
  const size_t nq = map->n_full.size(), nnz = map->kv_idx.size();
  if ((st = hip_status(hipMemcpyAsync(b, map->qptr.data(), (nq + 1) * sizeof(int32_t), hipMemcpyHostToDevice, s),
                       "tile map copy")) ||
      (nnz && (st = hip_status(hipMemcpyAsync(b + off_kv, map->kv_idx.data(), nnz * sizeof(int32_t),
                                               hipMemcpyHostToDevice, s),
                               "tile map copy"))) ||
      (st = hip_status(hipMemcpyAsync(b + off_nf, map->n_full.data(), nq * sizeof(int32_t), hipMemcpyHostToDevice, s),
                       "tile map copy")))
    return st;
  na::AttnArgs a = attn_args(g, reinterpret_cast<const int32_t*>(b), reinterpret_cast<const int32_t*>(b + off_kv),
                             reinterpret_cast<const int32_t*>(b + off_nf), lay.tq, lay.tkv, batch, heads, head_dim,
                             scale);
  a.qt = q;
  a.kt = k;
  a.vt = v;
  a.ot = out;
  a.lse_t = lse;
  a.io_mode = na::IO_GRID;
  return hip_status(na::launch_attn_bf16(a, s), "attention launch");
}

}  // namespace na

extern "C" {

// ---------------------------------------------------------------------------
// backward

namespace {

// Tile shapes and tile-order buffers of one backward problem.
struct BwdLayout {
  int tq[3], tkv[3];
  int dq_tq[3];   // Q tiles of the dq kernel (256 tokens when a pair with these KV tiles exists, else tq)
  size_t q_bytes, kv_bytes, stat_bytes;
  size_t off_q, off_k, off_v, off_do, off_l, off_d, total;
};

na_status check_bwd(int batch, int heads, int head_dim, const int grid[3], const int window[3], const int stride[3],
                    na_dtype dtype, BwdLayout* b) {
  Layout lay;
  na_status st = check_problem(batch, heads, head_dim, grid, window, stride, (int)dtype, &lay);
  if (st != NA_OK) return st;
  if (dtype != NA_BF16 || (head_dim != 64 && head_dim != 128))
    return fail(NA_ERR_UNSUPPORTED, "the backward is built for bf16 with head_dim 64 or 128");
  // 128-query and 128-key tiles, both at least 8 wide along W: the cheapest
  // such pair of the forward's candidates (with Q tiles padded to 8 along W
  // when the grid is narrower)
  const na::Geometry g = make_geom(grid, window, stride);
  bool found = false;
  for (const auto& c : na::tile_candidates(g, head_dim, na::Family::MFMA16, 8)) {
    if (c.tq[0] * c.tq[1] * c.tq[2] != 128 || c.tkv[0] * c.tkv[1] * c.tkv[2] != 128 || c.tq[2] < 8 ||
        c.tkv[2] < 8)
      continue;
    for (int d = 0; d < 3; ++d) {
      b->tq[d] = c.tq[d];
      b->tkv[d] = c.tkv[d];
    }
    found = true;
    break;
  }
  if (!found) return fail(NA_ERR_UNSUPPORTED, "no 128 x 128 tile pair at least 8 wide along W fits this grid");
  // the dq kernel: the cheapest 256-query tile paired with the same KV tiles
  // (8 waves, two per SIMD), else the 128-query tile
  for (int d = 0; d < 3; ++d) b->dq_tq[d] = b->tq[d];
  for (const auto& c : na::tile_candidates(g, head_dim, na::Family::MFMA16)) {
    if (c.tq[0] * c.tq[1] * c.tq[2] != 256 || !std::equal(c.tkv, c.tkv + 3, b->tkv)) continue;
    for (int d = 0; d < 3; ++d) b->dq_tq[d] = c.tq[d];
    break;
  }
  int64_t npq = 1, npk = 1;
  for (int d = 0; d < 3; ++d) {
    npq *= (int64_t)na::ceil_div(grid[d], b->tq[d]) * b->tq[d];
    npk *= (int64_t)na::ceil_div(grid[d], b->tkv[d]) * b->tkv[d];
  }
  const size_t bh = (size_t)batch * heads;
  b->q_bytes = bh * npq * head_dim * 2;
  b->kv_bytes = bh * npk * head_dim * 2;
  b->stat_bytes = bh * npq * sizeof(float);
  b->off_q = 0;
  b->off_k = b->off_q + round256(b->q_bytes);
  b->off_v = b->off_k + round256(b->kv_bytes);
  b->off_do = b->off_v + round256(b->kv_bytes);
  b->off_l = b->off_do + round256(b->q_bytes);
  b->off_d = b->off_l + round256(b->stat_bytes);
  b->total = b->off_d + round256(b->stat_bytes);
  return NA_OK;
}

}  // namespace

size_t na_backward_workspace_bytes(int batch, int heads, int head_dim, const int grid[3], const int window[3],
                                   const int stride[3], na_dtype dtype) {
  g_err.clear();
  BwdLayout b;
  if (check_bwd(batch, heads, head_dim, grid, window, stride, dtype, &b) != NA_OK) return 0;
  return b.total;
}

na_status na_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int batch, int heads, int head_dim,
                      const int grid[3], const int window[3], const int stride[3], float scale, na_dtype dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  BwdLayout b;
  na_status st = check_bwd(batch, heads, head_dim, grid, window, stride, dtype, &b);
  if (st != NA_OK) return st;
  if (batch == 0 || heads == 0) return NA_OK;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
    return fail(NA_ERR_INVALID_ARG, "q, k, v, out, dout, lse, dq, dk and dv must be non-null");
  for (const void* x : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(x)) return fail(NA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(NA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  st = check_scales(scale, dtype, nullptr);
  if (st != NA_OK) return st;
  if (!workspace) return fail(NA_ERR_INVALID_ARG, "workspace must be non-null");
  if (!aligned16(workspace)) return fail(NA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (workspace_bytes < b.total)
    return fail(NA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(b.total) + " bytes");
  const na::Geometry g = make_geom(grid, window, stride);
  Plan* plan = nullptr;
  st = get_plan_t(g, b.tq, b.tkv, &plan);
  if (st != NA_OK) return st;
  Plan* plan_dq = nullptr;
  st = get_plan(g, b.dq_tq, b.tkv, &plan_dq);
  if (st != NA_OK) return st;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = (hipStream_t)stream;
  void* qt = ws + b.off_q;
  void* kt = ws + b.off_k;
  void* vt = ws + b.off_v;
  void* dot = ws + b.off_do;
  if ((st = hip_status(na::launch_permute(q, qt, batch, heads, head_dim, grid, b.tq, 2, 0, s), "permute q")) ||
      (st = hip_status(na::launch_permute(k, kt, batch, heads, head_dim, grid, b.tkv, 2, 0, s), "permute k")) ||
      (st = hip_status(na::launch_permute(v, vt, batch, heads, head_dim, grid, b.tkv, 2, 0, s), "permute v")) ||
      (st = hip_status(na::launch_permute(dout, dot, batch, heads, head_dim, grid, b.tq, 2, 0, s), "permute dout")))
    return st;
  na::BwdArgs a{};
  a.attn = attn_args(g, plan, b.tq, b.tkv, batch, heads, head_dim, scale);
  a.attn.qt = qt;
  a.attn.kt = kt;
  a.attn.vt = vt;
  a.dq_attn = attn_args(g, plan_dq, b.dq_tq, b.tkv, batch, heads, head_dim, scale);
  a.dq_attn.qt = qt;
  a.dq_attn.kt = kt;
  a.dq_attn.vt = vt;
  a.q = q;
  a.dot = dot;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.lse2_t = reinterpret_cast<float*>(ws + b.off_l);
  a.d_t = reinterpret_cast<float*>(ws + b.off_d);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.tqptr = plan->d_tptr;
  a.tq_idx = plan->d_tidx;
  a.tn_full = plan->d_tnfull;
  return hip_status(na::launch_bwd(a, s), "backward launch");
}

// ---------------------------------------------------------------------------
// content-selected block sparsity (top-k KV tiles per Q tile)

namespace {

struct TopkLayout {
  int tq[3], tkv[3];
  int nq, nk;
  size_t off_qm, off_km, off_idx, off_nf, off_qptr, off_kt, off_vt, total;
};

na_status check_topk(int batch, int heads, int head_dim, const int grid[3], int keep, na_dtype dtype,
                     TopkLayout* t) {
  if (!grid) return fail(NA_ERR_INVALID_ARG, "grid must be non-null");
  const int ones[3] = {1, 1, 1};
  Layout lay;   // the blocks are the tiles of the dense geometry (window = grid)
  na_status st = check_problem(batch, heads, head_dim, grid, grid, ones, (int)dtype, &lay);
  if (st != NA_OK) return st;
  if (dtype != NA_BF16 || !na::attn_bf16_grid_io_supported(head_dim))
    return fail(NA_ERR_UNSUPPORTED, "top-k selection is built for bf16 with head_dim 64 or 128");
  t->nq = lay.nq[0] * lay.nq[1] * lay.nq[2];
  t->nk = lay.nk[0] * lay.nk[1] * lay.nk[2];
  for (int d = 0; d < 3; ++d) {
    t->tq[d] = lay.tq[d];
    t->tkv[d] = lay.tkv[d];
  }
  if (keep < 1 || keep > t->nk) return fail(NA_ERR_INVALID_ARG, "keep must be in [1, number of KV tiles]");
  if (!na::topk_select_supported(t->nk, head_dim))
    return fail(NA_ERR_UNSUPPORTED, "more than 4096 KV tiles for the selection kernel");
  const size_t bh = (size_t)batch * heads;
  if (bh * (size_t)t->nq * (size_t)keep >= (size_t(1) << 31))
    return fail(NA_ERR_UNSUPPORTED, "tile map larger than 2^31 entries");
  t->off_qm = 0;
  t->off_km = t->off_qm + round256(bh * t->nq * head_dim * 4);
  t->off_idx = t->off_km + round256(bh * t->nk * head_dim * 4);
  t->off_nf = t->off_idx + round256(bh * t->nq * (size_t)keep * 4);
  t->off_qptr = t->off_nf + round256(bh * t->nq * 4);
  t->off_kt = t->off_qptr + round256(((size_t)t->nq + 1) * 4);
  t->off_vt = t->off_kt + round256(lay.kv_bytes);
  t->total = t->off_vt + round256(lay.kv_bytes);
  return NA_OK;
}

na_status topk_select_impl(const void* q, const void* k, int batch, int heads, int head_dim, const int grid[3],
                           int keep, const TopkLayout& t, char* ws, int32_t* kv_idx, int32_t* n_full,
                           hipStream_t s) {
  na::TopkArgs a{};
  a.geom.batch = batch;
  a.geom.heads = heads;
  a.geom.head_dim = head_dim;
  for (int d = 0; d < 3; ++d) {
    a.geom.L[d] = grid[d];
    a.geom.tq[d] = t.tq[d];
    a.geom.tkv[d] = t.tkv[d];
  }
  a.nq = t.nq;
  a.nk = t.nk;
  a.keep = keep;
  a.q = q;
  a.k = k;
  a.qm = reinterpret_cast<float*>(ws + t.off_qm);
  a.km = reinterpret_cast<float*>(ws + t.off_km);
  a.kv_idx = kv_idx;
  a.n_full = n_full;
  a.qptr = reinterpret_cast<int32_t*>(ws + t.off_qptr);
  return hip_status(na::launch_topk_select(a, s), "top-k selection launch");
}

}  // namespace

na_status na_topk_tiles(const int grid[3], int head_dim, na_dtype dtype, int tile_q[3], int tile_kv[3]) {
  g_err.clear();
  if (!tile_q || !tile_kv) return fail(NA_ERR_INVALID_ARG, "tile_q and tile_kv must be non-null");
  TopkLayout t;
  na_status st = check_topk(1, 1, head_dim, grid, 1, dtype, &t);
  if (st != NA_OK) return st;
  for (int d = 0; d < 3; ++d) {
    tile_q[d] = t.tq[d];
    tile_kv[d] = t.tkv[d];
  }
  return NA_OK;
}

size_t na_topk_workspace_bytes(int batch, int heads, int head_dim, const int grid[3], int keep, na_dtype dtype) {
  g_err.clear();
  TopkLayout t;
  if (check_topk(batch, heads, head_dim, grid, keep, dtype, &t) != NA_OK) return 0;
  return (batch == 0 || heads == 0) ? 0 : t.total;
}

na_status na_topk_select(const void* q, const void* k, int batch, int heads, int head_dim, const int grid[3],
                         int keep, na_dtype dtype, int32_t* kv_idx, int32_t* n_full, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_err.clear();
  TopkLayout t;
  na_status st = check_topk(batch, heads, head_dim, grid, keep, dtype, &t);
  if (st != NA_OK) return st;
  if (batch == 0 || heads == 0) return NA_OK;
  if (!q || !k || !kv_idx || !n_full) return fail(NA_ERR_INVALID_ARG, "q, k, kv_idx and n_full must be non-null");
  if (!aligned16(q) || !aligned16(k)) return fail(NA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(kv_idx) | reinterpret_cast<uintptr_t>(n_full)) & 3u)
    return fail(NA_ERR_INVALID_ARG, "kv_idx and n_full must be 4-byte aligned");
  if (!workspace || !aligned16(workspace)) return fail(NA_ERR_INVALID_ARG, "workspace must be non-null and aligned");
  if (workspace_bytes < t.total)
    return fail(NA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(t.total) + " bytes");
  return topk_select_impl(q, k, batch, heads, head_dim, grid, keep, t, static_cast<char*>(workspace), kv_idx, n_full,
                          (hipStream_t)stream);
}

na_status na_topk_forward(const void* q, const void* k, const void* v, void* out, float* lse, int batch, int heads,
                          int head_dim, const int grid[3], int keep, float scale, na_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_err.clear();
  TopkLayout t;
  na_status st = check_topk(batch, heads, head_dim, grid, keep, dtype, &t);
  if (st != NA_OK) return st;
  if (batch == 0 || heads == 0) return NA_OK;
  if (!q || !k || !v || !out) return fail(NA_ERR_INVALID_ARG, "q, k, v and out must be non-null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(NA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(NA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  st = check_scales(scale, dtype, nullptr);
  if (st != NA_OK) return st;
  if (!workspace || !aligned16(workspace)) return fail(NA_ERR_INVALID_ARG, "workspace must be non-null and aligned");
  if (workspace_bytes < t.total)
    return fail(NA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(t.total) + " bytes");
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = (hipStream_t)stream;
  int32_t* kv_idx = reinterpret_cast<int32_t*>(ws + t.off_idx);
  int32_t* n_full = reinterpret_cast<int32_t*>(ws + t.off_nf);
  st = topk_select_impl(q, k, batch, heads, head_dim, grid, keep, t, ws, kv_idx, n_full, s);
  if (st != NA_OK) return st;
  void* kt = ws + t.off_kt;
  void* vt = ws + t.off_vt;
  if ((st = hip_status(na::launch_permute(k, kt, batch, heads, head_dim, grid, t.tkv, 2, 0, s), "permute k")) ||
      (st = hip_status(na::launch_permute(v, vt, batch, heads, head_dim, grid, t.tkv, 2, 1, s), "permute v")))
    return st;
  na::AttnArgs a{};
  a.qt = q;
  a.kt = kt;
  a.vt = vt;
  a.ot = out;
  a.lse_t = lse;
  a.qptr = reinterpret_cast<int32_t*>(ws + t.off_qptr);
  a.kv_idx = kv_idx;
  a.n_full = n_full;
  a.batch = batch;
  a.heads = heads;
  a.head_dim = head_dim;
  for (int d = 0; d < 3; ++d) {
    a.L[d] = grid[d];
    a.w[d] = grid[d];   // window = grid: the mask keeps every real key of a listed tile
    a.s[d] = 1;
    a.tq[d] = t.tq[d];
    a.tkv[d] = t.tkv[d];
    a.nq[d] = na::ceil_div(grid[d], t.tq[d]);
    a.nk[d] = na::ceil_div(grid[d], t.tkv[d]);
  }
  a.scale = scale;
  a.v_scale = 1.0f;
  a.io_mode = na::IO_QO;
  a.map_bh_kv = (int64_t)t.nq * keep;
  a.map_bh_nf = t.nq;
  return hip_status(na::launch_attn_bf16(a, s), "top-k attention launch");
}

}  // extern "C"
