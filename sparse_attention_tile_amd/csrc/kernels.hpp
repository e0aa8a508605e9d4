// Launchers of the HIP kernels (defined in the .hip files) and the argument
// block they share.  Host code validates everything before calling these.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace na {

// Layouts of the attention kernel's tensors: all in tile order; q / out / lse
// in grid order with k / v in tile order; all in grid order.
enum IoMode { IO_TILE = 0, IO_QO = 1, IO_GRID = 2 };

struct AttnArgs {
  const void* qt;          // q, tile order (tile_q tiles)
  const void* kt;          // k, tile order (tile_kv tiles)
  const void* vt;          // v, transposed tile order (tile_kv tiles)
  void* ot;                // out, tile order (tile_q tiles)
  float* lse_t;            // lse, tile order, may be null
  const int32_t* qptr;     // device tile map
  const int32_t* kv_idx;
  const int32_t* n_full;
  int batch, heads, head_dim;
  int L[3], w[3], s[3];    // grid, window, stride (T, H, W)
  int tq[3], tkv[3];       // tile extents (powers of two)
  int nq[3], nk[3];        // tiles per axis
  float scale;             // multiplies q.k (fp8: includes the q and k scales)
  float v_scale;           // fp8: multiplies the output; else 1
  int io_mode;             // IO_TILE, IO_QO or IO_GRID (tensor layouts, see attn_bf16.hip)
  // per-(batch, head) tile maps (bf16 kernel only): row a of (batch, head)
  // bh lists kv_idx[qptr[a] + bh * map_bh_kv ..] and has n_full[a + bh *
  // map_bh_nf] full tiles; both 0 for a map shared by every (batch, head)
  int64_t map_bh_kv;
  int map_bh_nf;
};

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st);
hipError_t launch_attn_fp8(const AttnArgs& a, hipStream_t st);

// Kernel shapes the attention launchers accept (host-side check).
bool attn_bf16_supported(int head_dim, int q_tokens, int kv_tokens);
bool attn_fp8_supported(int head_dim, int q_tokens, int kv_tokens);
bool attn_f32_supported(int head_dim, int q_tokens, int kv_tokens);
// The bf16/fp8 kernels need KV tiles at least 8 tokens wide along W.
bool attn_bf16_tile_ok(const int tile_kv[3]);
// Whether the bf16 kernel can read and write grid order directly.
bool attn_bf16_grid_io_supported(int head_dim);

// Backward pass (bf16): the forward's problem description plus the extra
// tensors.  attn.qt/kt/vt hold q, k, v in tile order (plain rows); dot holds
// dO in tile order; out, dout, lse are the caller's grid-order tensors;
// lse2_t and d_t are tile-order fp32 scratch the prep kernel fills; dq, dk,
// dv are written in grid order; tqptr/tq_idx/tn_full are the transposed tile
// map (per KV tile, its Q tiles, full ones first).
struct BwdArgs {
  AttnArgs attn;
  // the dq kernel's problem: its own tile map; KV tiles as attn's, Q tiles of
  // 256 tokens (then q, dout, out, lse are read in grid order) or attn's
  AttnArgs dq_attn;
  const void* q;
  const void* dot;
  const void* out;
  const void* dout;
  const float* lse;
  float* lse2_t;
  float* d_t;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* tqptr;
  const int32_t* tq_idx;
  const int32_t* tn_full;
};
hipError_t launch_bwd(const BwdArgs& a, hipStream_t st);
bool attn_bwd_supported(int head_dim, int q_tokens, int kv_tokens);

// Content-selected block sparsity: geometry of the pooling / selection
// kernels and their buffers.  q and k are the caller's grid-order bf16
// tensors; qm [B*heads, nq, D] and km [B*heads, D, nk] fp32 scratch for the
// block means; kv_idx [B*heads, nq, keep], n_full [B*heads, nq] and
// qptr [nq + 1] (the row starts a * keep) are the per-(batch, head) tile map.
struct TopkGeom {
  int batch, heads, head_dim;
  int L[3];
  int tq[3], tkv[3];
};
struct TopkArgs {
  TopkGeom geom;
  int nq, nk, keep;
  const void* q;
  const void* k;
  float* qm;
  float* km;
  int32_t* kv_idx;
  int32_t* n_full;
  int32_t* qptr;
};
hipError_t launch_topk_select(const TopkArgs& a, hipStream_t st);
// Whether the selection kernel handles nk KV tiles at head_dim (its sort
// keys live in LDS: up to 4096 tiles).
bool topk_select_supported(int nk, int head_dim);

// LDS bytes the transposed permutation needs for one tile (must be <= 64 KiB).
size_t permute_transpose_lds_bytes(int head_dim, int tile_tokens, int elem_bytes);

hipError_t launch_permute(const void* x, void* xt, int batch, int heads, int head_dim,
                          const int grid[3], const int tile[3], int elem_bytes, int transpose,
                          hipStream_t st);
hipError_t launch_unpermute(const void* xt, void* x, int batch, int heads, int head_dim,
                            const int grid[3], const int tile[3], int elem_bytes, hipStream_t st);
hipError_t launch_unpermute_lse(const float* lse_t, float* lse, int batch, int heads,
                                const int grid[3], const int tile[3], hipStream_t st);

}  // namespace na
