/*
 * na.h -- C ABI of the MI355X (gfx950) Generalized Neighborhood Attention
 * forward library (libna.so).
 *
 * Page citations name the pages by title:
 *   GNA page  = "GNA Sparse Attention Mechanism: Vision-Transformer Compute
 *               Optimisation in Practice"
 *   tutorial  = "Video-generation inference speed-up: sparse attention
 *               configuration tutorial"
 *   SLA page  = "Sparse attention in video and image generation:
 *               optimisation practice"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Geometry.  A token grid always has three extents, in (T, H, W) order:
 *   grid[3], window[3], stride[3].  A 2-D image passes T = 1 (window 1,
 *   stride 1); a 1-D sequence passes T = H = 1.  Every axis must satisfy
 *   1 <= stride <= window <= grid, else NA_ERR_INVALID_ARG.
 *
 * Which keys a query sees (GNA page, section 1.1).  On each axis the
 * queries form stride groups g = floor(i / s); the group's leader is its
 * centre min(g*s + floor(s/2), L-1); the window of every query in the group
 * starts at clamp(leader - floor(w/2), 0, L - w) and holds w keys.  The
 * key set of a query is the product of its per-axis windows, so every query
 * attends exactly prod(window) keys.  s = 1 is sliding-window neighborhood
 * attention; s > 1 is the block pattern.  No dilation, no causal mask.
 *
 * Token layout ("grid order").  q, k, v and out are contiguous
 *   [batch, T, H, W, heads, head_dim]; lse is [batch, T, H, W, heads].
 *
 * Tile layout ("tile order", private to this library, produced by
 * na_permute).  The grid is cut into boxes of tile[3] tokens (each extent a
 * power of two); each axis is padded with zeros to a whole number of tiles.
 * A tile-ordered tensor is [batch, heads, n_tiles, tile_tokens, head_dim]
 * with tiles and the tokens inside a tile both row-major over (T, H, W).
 * The "transposed" variant stores every tile as [head_dim, tile_tokens].
 *
 * Pointers.  "device" pointers are HIP device memory owned by the caller;
 * they must be 16-byte aligned.  "host" pointers are ordinary host memory.
 * The library never frees caller memory.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Device entry points only enqueue work: they return before it
 * runs and do not synchronise.  The first na_forward / na_backward call
 * for a geometry builds its plan (host tile map, allocated and uploaded
 * synchronously); after that these calls only launch kernels, so they can
 * be captured in a HIP graph (tested: every replay equals the eager call).
 *
 * Empty problems.  batch == 0 or heads == 0 is valid: device entry points
 * then launch nothing and return NA_OK (pointers are not checked).
 *
 * Errors.  Every entry point validates its arguments before launching
 * anything; on failure it returns a negative na_status, launches nothing and
 * leaves a message for na_last_error().  No entry point throws, prints or
 * aborts.  Problems whose launch would exceed 2^32 work-items (batch * heads
 * * tiles * 512 threads), or grids of more than 2^30 tokens, are refused
 * with NA_ERR_UNSUPPORTED.
 *
 * Test and tuning hooks (environment variables, read at each call; unset in
 * normal use, and no hook changes a result beyond floating-point rounding):
 *   NA_NO_FUSED=1       na_forward takes form 0 (see na_forward_mode);
 *   NA_TILE_Q, NA_TILE_KV="t,h,w"  replace the chosen tile shapes (the kernel
 *                       shape rules still apply; malformed -> INVALID_ARG);
 *   NA_FORCE_MASK=1     every listed KV tile is treated as a boundary tile
 *                       (results are bit-identical);
 *   NA_DKDV_SPLIT=0     na_backward's dk/dv kernel runs one wave per 32 keys
 *                       for both gradients instead of one wave per gradient
 *                       (results are bit-identical).
 */
#ifndef NA_H_
#define NA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum na_status {
  NA_OK = 0,
  NA_ERR_INVALID_ARG = -1,  /* geometry, null/misaligned pointer, sizes      */
  NA_ERR_UNSUPPORTED = -2,  /* valid but not built: head_dim, dtype, tiles   */
  NA_ERR_WORKSPACE = -3,    /* workspace smaller than na_workspace_bytes()   */
  NA_ERR_HIP = -4           /* the HIP runtime reported an error             */
} na_status;

typedef enum na_dtype {
  NA_F32 = 0,       /* fp32 in, fp32 out, fp32 arithmetic throughout       */
  NA_BF16 = 1,      /* bf16 in/out; fp32 softmax and accumulation          */
  NA_FP8_E4M3 = 2   /* OCP e4m3fn in with per-tensor scales, bf16 out      */
} na_dtype;

/* Counts of one tile map, per (batch, head).  "slots" are query-key pairs:
 * computed_slots = nnz * tile_q_tokens * tile_kv_tokens (what the kernel
 * multiplies), effective_slots = N * prod(window) (what the method needs). */
typedef struct na_tilemap_stats {
  int64_t n_q_tiles;
  int64_t n_kv_tiles;
  int64_t nnz;
  int64_t n_full;
  int64_t n_boundary;
  int64_t computed_slots;
  int64_t effective_slots;
} na_tilemap_stats;

/* One tile-shape configuration as the analytic model sees it. */
typedef struct na_sim_result {
  int32_t tile_q[3];
  int32_t tile_kv[3];
  na_tilemap_stats stats;        /* per (batch, head)                       */
  double tile_efficiency;        /* effective / computed slots              */
  double flop_ratio_vs_dense;    /* N / prod(window): FLOPs of the dense call
                                    over FLOPs of this one                  */
  double speedup_bound;          /* computed slots of the dense call (window
                                    = grid, its own tiles) over computed slots
                                    of this one: the speedup over dense that
                                    the tile-level work allows at equal
                                    per-slot speed                          */
  int32_t perfectly_block_sparse;/* 1 iff every listed KV tile is full: KV
                                    tile edges align with every window, no
                                    key slot is masked (padded query rows,
                                    counted in tile_efficiency, aside)      */
  int32_t form;                  /* na_forward_mode with a workspace        */
  double cost;                   /* the tile chooser's relative cost        */
  double predicted_kernel_ms;    /* attention kernel on one MI355X          */
  double predicted_forward_ms;   /* plus the permutations of `form`         */
} na_sim_result;

/* ---------------------------------------------------------------------- */
/* Host-only entry points (no HIP call; usable without a GPU).            */
/* ---------------------------------------------------------------------- */

/* Tile shapes the library uses for a problem (GNA page, section 1.2:
 * decoupled query and key/value tile sizes T_Q and T_KV).  Writes
 * tile_q[3] and tile_kv[3] (host).  Returns NA_ERR_UNSUPPORTED when no
 * kernel is built for (head_dim, dtype). */
na_status na_choose_tiles(const int grid[3], const int window[3],
                          const int stride[3], int head_dim, na_dtype dtype,
                          int tile_q[3], int tile_kv[3]);

/* Host tile-map builder (GNA page, section 1.1: the stride decides the
 * range of KV tiles each Q tile visits; section 2.1: only KV tiles not
 * fully inside the window need the fine-grained mask).
 *
 * Output is CSR over query tiles in row-major tile order:
 *   qptr[n_q_tiles + 1], kv_idx[nnz] (row-major linear KV-tile index),
 *   n_full[n_q_tiles].
 * Inside row a the first n_full[a] entries are *full* tiles (every real
 * query of the Q tile attends every slot of the KV tile, so the tile has no
 * padding) and the rest are *boundary* tiles; each part is ascending.
 * A KV tile is listed iff at least one of its (query, key) pairs is
 * attended.
 *
 * Any of qptr, kv_idx, n_full may be NULL (then only the counts are
 * produced).  kv_capacity is the length of kv_idx; if it is smaller than
 * nnz the call returns NA_ERR_INVALID_ARG and writes nothing but *nnz_out
 * and *stats.  tile extents must be powers of two.  nnz_out and stats may
 * be NULL. */
na_status na_build_tile_map(const int grid[3], const int window[3],
                            const int stride[3], const int tile_q[3],
                            const int tile_kv[3], int32_t* qptr,
                            int32_t* kv_idx, int32_t* n_full,
                            int64_t kv_capacity, int64_t* nnz_out,
                            na_tilemap_stats* stats);

/* Analytic model of one problem (GNA page, sections 4.2 and 5: check the
 * theoretical speedup bound of a configuration with a simulator before
 * running it, and pick the tiling per hardware).  From the tile map alone it
 * reports computed vs effective work, whether the configuration is perfectly
 * block-sparse, the speedup bound over the dense call, and a predicted
 * MI355X time from a per-CU serial model calibrated on the measured kernels.
 * tile_q / tile_kv: the shapes to evaluate (powers of two), or both NULL for
 * the shapes na_choose_tiles picks.  Writes *out (host).  Errors as
 * na_choose_tiles. */
na_status na_simulate(int batch, int heads, int head_dim, const int grid[3],
                      const int window[3], const int stride[3],
                      na_dtype dtype, const int tile_q[3],
                      const int tile_kv[3], na_sim_result* out);

/* Every tile-shape pair na_choose_tiles considers for the problem, sorted by
 * its cost (out[0] is the chosen pair), each evaluated as by na_simulate.
 * Writes min(count, capacity) entries to out (host; may be NULL when
 * capacity is 0) and returns the total count, or a negative na_status. */
int na_tile_candidates(int batch, int heads, int head_dim, const int grid[3],
                       const int window[3], const int stride[3],
                       na_dtype dtype, na_sim_result* out, int capacity);

/* Bytes of device workspace na_forward needs for this problem: the
 * tile-ordered copies it makes (form 1 of na_forward_mode: k and v; form 0:
 * q, k, v, out and lse).  It grows linearly with the token count: no N x N
 * buffer exists (tutorial, section 3.3).  Returns 0 if
 * the arguments are invalid or unsupported (na_last_error() says why) and
 * for an empty problem (then na_last_error() is ""). */
size_t na_workspace_bytes(int batch, int heads, int head_dim,
                          const int grid[3], const int window[3],
                          const int stride[3], na_dtype dtype);

/* The form na_forward takes for this dtype and head_dim:
 *   0  permute q, k, v to tile order, tiled kernel, unpermute out and lse;
 *   1  permute k, v only; the kernel reads q and writes out and lse in grid
 *      order (bf16 with head_dim 64 / 128 and a workspace; fp8 with 128);
 *   2  no permutation and no workspace: the kernel also gathers the k / v
 *      tiles from grid order (bf16, head_dim 64 / 128, workspace NULL).
 * with_workspace says whether the call would pass a workspace.  The
 * environment variable NA_NO_FUSED=1, read at each call, forces form 0 (a
 * test hook).  Never fails. */
int na_forward_mode(na_dtype dtype, int head_dim, int with_workspace);

/* Message of the last failing call on this thread ("" if none).  Valid
 * until the next call on the same thread. */
const char* na_last_error(void);

/* Frees every cached plan (host and device tile maps).  Must not be called
 * while work that uses a plan may still run on a stream. */
void na_release_cache(void);

/* ---------------------------------------------------------------------- */
/* Device entry points (enqueue on `stream`).                             */
/* ---------------------------------------------------------------------- */

/* One GNA forward pass (GNA page, sections 1.1 and 2.1-2.2).
 *   bf16 (head_dim 64/128) with a workspace: permute k and v to tile order;
 *   one kernel reads the q rows and writes out and lse in grid order.
 *   bf16 (head_dim 64/128) with workspace == NULL: no permutation at all --
 *   the kernel also gathers the k / v tiles from grid order (the permutation
 *   the page plans to fuse away, section 2.2, does not exist).  Slower than
 *   the form above on the video workload (the token-by-token gather), but
 *   needs no memory beyond the outputs.
 *   fp8 (head_dim 128): as bf16 with a workspace -- permute k and v, the
 *   kernel reads q and writes out and lse in grid order (a workspace is
 *   required).
 *   fp32: permute q, k, v to tile order (zero padding), run the tiled
 *   attention kernel, permute out and lse back to grid order.
 * na_forward_mode() tells which form a call takes.  When q is read in grid
 * order, the padding slots of ragged Q tiles read real tokens of the grid
 * (results discarded); when k / v are gathered, padding slots of ragged KV
 * tiles read real tokens (masked, multiplied by zero).  So q, k, v must hold
 * finite values everywhere, not only inside the windows.
 *
 * q, k, v  device, [batch, T, H, W, heads, head_dim], dtype `dtype`.
 * out      device, same shape; fp32 for NA_F32, bf16 for NA_BF16 and
 *          NA_FP8_E4M3.
 * lse      device, [batch, T, H, W, heads] fp32, natural-log logsumexp of
 *          the scaled scores of each query; may be NULL.
 * scale    multiplies q.k before the softmax (usually 1/sqrt(head_dim));
 *          finite and >= 0 (a negative factor belongs in q).
 * qkv_scale host, 3 floats: dequantisation multipliers of q, k, v for
 *          NA_FP8_E4M3 (NULL means 1, 1, 1); ignored for other dtypes.
 * workspace device, caller-owned, >= na_workspace_bytes(...) bytes; may be
 *          NULL for bf16 with head_dim 64 / 128 (workspace_bytes ignored).
 * head_dim must be 32 (NA_F32), 64 or 128 (NA_BF16, NA_FP8_E4M3).
 *
 * Softmax statistics and accumulation are fp32 in every mode (SLA page,
 * section 3.1).  The first call for a geometry builds and uploads the tile
 * map (cached); later calls allocate nothing. */
na_status na_forward(const void* q, const void* k, const void* v, void* out,
                     float* lse, int batch, int heads, int head_dim,
                     const int grid[3], const int window[3],
                     const int stride[3], float scale, na_dtype dtype,
                     const float* qkv_scale, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Token permutation, grid order -> tile order, with zero padding (GNA page,
 * section 2.2: the permutation before the kernel, fused with padding).
 *
 * x   device, [batch, T, H, W, heads, head_dim], elements of elem_bytes
 *     (1, 2 or 4) bytes.
 * xt  device, [batch, heads, n_tiles, tile_tokens, head_dim] (transpose=0)
 *     or [batch, heads, n_tiles, head_dim, tile_tokens] (transpose=1).
 *     Every element is written, padding slots with zero.
 * head_dim * elem_bytes must be a multiple of 16. */
na_status na_permute(const void* x, void* xt, int batch, int heads,
                     int head_dim, const int grid[3], const int tile[3],
                     int elem_bytes, int transpose, void* stream);

/* Inverse token permutation, tile order -> grid order, padding dropped
 * (GNA page, section 2.2: the reverse permutation after the kernel).
 * xt is [batch, heads, n_tiles, tile_tokens, head_dim]; x is
 * [batch, T, H, W, heads, head_dim]. */
na_status na_unpermute(const void* xt, void* x, int batch, int heads,
                       int head_dim, const int grid[3], const int tile[3],
                       int elem_bytes, void* stream);

/* Inverse permutation of the logsumexp: lse_t [batch, heads, n_tiles,
 * tile_tokens] fp32 -> lse [batch, T, H, W, heads] fp32. */
na_status na_unpermute_lse(const float* lse_t, float* lse, int batch,
                           int heads, const int grid[3], const int tile[3],
                           void* stream);

/* The fused attention kernel alone, on tile-ordered tensors (GNA page,
 * sections 1.1 and 2.1; tutorial, section 3.3: block-wise online softmax).
 *
 * qt      device, q in tile order with tile_q tiles.
 * kt      device, k in tile order with tile_kv tiles.
 * vt      device, v in *transposed* tile order with tile_kv tiles (fp32 mode:
 *         plain tile order).
 * ot      device, [batch, heads, n_q_tiles, tile_q_tokens, head_dim], fp32
 *         for NA_F32 else bf16; rows of padding queries hold finite values
 *         that carry no meaning.
 * lse_t   device, [batch, heads, n_q_tiles, tile_q_tokens] fp32, or NULL.
 * tile_q/tile_kv must be what na_choose_tiles returns for the problem.
 * Other arguments as for na_forward. */
na_status na_attend_tiled(const void* qt, const void* kt, const void* vt,
                          void* ot, float* lse_t, int batch, int heads,
                          int head_dim, const int grid[3], const int window[3],
                          const int stride[3], const int tile_q[3],
                          const int tile_kv[3], float scale, na_dtype dtype,
                          const float* qkv_scale, void* stream);

/* The attention kernel of na_forward's form 1 alone (GNA page, sections 1.1
 * and 2.1-2.2): q, out and lse in grid order, k and v already in tile order
 * (as na_permute writes them: kt plain, vt transposed, both with tile_kv
 * tiles).  bf16 with head_dim 64 or 128, or fp8 e4m3 with head_dim 128
 * (else NA_ERR_UNSUPPORTED).
 *
 * q       device, [batch, T, H, W, heads, head_dim] in `dtype`.
 * out     device, same shape, bf16.
 * lse     device, [batch, T, H, W, heads] fp32, or NULL.
 * tile_kv must be what na_choose_tiles returns for the problem.
 * Other arguments (qkv_scale: fp8 dequantisation, NULL means 1, 1, 1) as
 * for na_forward. */
na_status na_attend_kv_tiled(const void* q, const void* kt, const void* vt,
                             void* out, float* lse, int batch, int heads,
                             int head_dim, const int grid[3],
                             const int window[3], const int stride[3],
                             const int tile_kv[3], float scale, na_dtype dtype,
                             const float* qkv_scale, void* stream);

/* ---------------------------------------------------------------------- */
/* Content-selected block sparsity (bf16).                                 */
/* ---------------------------------------------------------------------- */
/* The tutorial (section 6) scores blocks by importance, keeps the best ones
 * and skips the rest whole; the overview page (section 2.2) names top-k
 * selection.  Here: blocks are the library's tiles of the dense geometry
 * (na_topk_tiles), score(a, c) = <mean q over the real tokens of Q tile a,
 * mean k over the real tokens of KV tile c>, and each Q tile keeps its
 * `keep` best KV tiles (equal scores: lower index first); every query of a
 * Q tile attends to every real key of its kept tiles.  Scores are evaluated
 * in float32 in a fixed order (token-by-token sums in in-tile row-major
 * order, IEEE division by the count, product-by-product sums over the head
 * dimension, no fused multiply-add), so the selection is reproducible bit
 * for bit.  bf16, head_dim 64 or 128; 1 <= keep <= number of KV tiles;
 * at most 4096 KV tiles (else NA_ERR_UNSUPPORTED). */

/* Tile (block) shapes top-k selection uses for this grid (host). */
na_status na_topk_tiles(const int grid[3], int head_dim, na_dtype dtype,
                        int tile_q[3], int tile_kv[3]);

/* Device workspace bytes of na_topk_select / na_topk_forward (linear in N
 * plus the B*heads*nQ*keep tile map). 0 if invalid (na_last_error()). */
size_t na_topk_workspace_bytes(int batch, int heads, int head_dim,
                               const int grid[3], int keep, na_dtype dtype);

/* The selection alone.  kv_idx: device int32 [batch*heads, nQ, keep], each
 * row full tiles (no padding slot) first, then the others, each ascending;
 * n_full: device int32 [batch*heads, nQ].  q, k as for na_forward. */
na_status na_topk_select(const void* q, const void* k, int batch, int heads,
                         int head_dim, const int grid[3], int keep,
                         na_dtype dtype, int32_t* kv_idx, int32_t* n_full,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* Selection, then attention over the kept tiles (k and v permuted to tile
 * order; the bf16 attention kernel reads q and writes out and lse in grid
 * order, one tile map per (batch, head)).  Tensors and errors as for
 * na_forward (lse may be NULL). */
na_status na_topk_forward(const void* q, const void* k, const void* v,
                          void* out, float* lse, int batch, int heads,
                          int head_dim, const int grid[3], int keep,
                          float scale, na_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* Backward pass (bf16).                                                   */
/* ---------------------------------------------------------------------- */

/* Bytes of device workspace na_backward needs: tile-ordered copies of q, k,
 * v and dout plus two fp32 rows per query (linear in N).  0 if the problem
 * is invalid or unsupported (na_last_error() says why) or empty. */
size_t na_backward_workspace_bytes(int batch, int heads, int head_dim,
                                   const int grid[3], const int window[3],
                                   const int stride[3], na_dtype dtype);

/* Gradients of na_forward (GNA page, section 5: training with the sparse
 * pattern is the pages' next step; softmax statistics in fp32, SLA page,
 * section 3.1) for the loss sum <dout, out>, with no gradient through lse:
 *   p_ij = exp(scale q_i.k_j - lse_i),  D_i = <dout_i, out_i>,
 *   dS_ij = p_ij (dout_i.v_j - D_i),
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 *   dv_j = sum_i p_ij dout_i
 * over exactly the forward's (query, key) pairs.  bf16 with head_dim 64 or
 * 128 only (else NA_ERR_UNSUPPORTED).  It runs on 128-token Q and KV tiles
 * at least 8 wide along W (padded to 8 when the grid is narrower).
 *
 * q, k, v  device, the forward's inputs, [batch, T, H, W, heads, head_dim].
 * out, lse device, the forward's outputs for these inputs (out bf16 as
 *          na_forward wrote it; lse fp32 [batch, T, H, W, heads]).
 * dout     device, gradient of the loss with respect to out, same layout.
 * dq, dk, dv device, bf16, same layout as q; every element is written.
 * workspace device, caller-owned, >= na_backward_workspace_bytes(...).
 * Accumulation is fp32; P and dS enter the matrix products as bf16.  No
 * atomics: each output row is computed by one workgroup, so results are
 * deterministic.  Other arguments and errors as for na_forward. */
na_status na_backward(const void* q, const void* k, const void* v,
                      const void* out, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, int batch, int heads,
                      int head_dim, const int grid[3], const int window[3],
                      const int stride[3], float scale, na_dtype dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the fixed device buffer na_forward_noalloc keeps its tile map in
 * (one per GPU, held until the process ends). */
#define NA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* na_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * calls no hipMalloc / hipFree and allocates no device memory: the tile map
 * the kernel walks goes into a fixed device buffer of
 * NA_NOALLOC_SCRATCH_BYTES per GPU, copied there (hipMemcpyAsync on
 * `stream`, from a host-side map the library builds and caches on the first
 * call for a geometry) before the kernel on every call.
 * It computes what na_forward's form 2 computes (bf16, head_dim 64 or 128,
 * no workspace: the kernel reads q, k, v and writes out, lse in grid order),
 * bit for bit.  Other dtypes or head dims: NA_ERR_UNSUPPORTED.  A problem
 * whose tile map (4 bytes per Q tile twice, plus 4 per listed KV tile, each
 * part rounded up to 256 bytes) exceeds NA_NOALLOC_SCRATCH_BYTES is refused
 * with NA_ERR_UNSUPPORTED before anything is enqueued.
 * Every call on one GPU shares that GPU's buffer, which keeps the last
 * call's contents: calls that overlap on one GPU (different streams, no
 * ordering between them) race and may produce wrong results.
 * After a first call for a geometry on a device (which builds the host map
 * and looks up the buffer's address), a call may be captured into a HIP
 * graph: the capture holds the map copy and the kernel, so each replay
 * rewrites the buffer before using it.
 * Arguments, layouts and other errors as for na_forward. */
na_status na_forward_noalloc(const void* q, const void* k, const void* v,
                             void* out, float* lse, int batch, int heads,
                             int head_dim, const int grid[3],
                             const int window[3], const int stride[3],
                             float scale, na_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NA_H_ */
