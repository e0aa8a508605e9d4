/* Plain C99 client of the library's host entry points (no GPU needed):
 * proves include/na.h is a C header and that libna.so links and runs from
 * C.  Prints one line per check as "name value ..." for the test to compare
 * with the oracle. */
#include <stdio.h>
#include <stdlib.h>

#include "na.h"

int main(void) {
  const int grid[3] = {30, 48, 80}, window[3] = {18, 24, 24}, stride[3] = {16, 8, 8};
  int tq[3], tk[3];
  if (na_choose_tiles(grid, window, stride, 128, NA_BF16, tq, tk) != NA_OK) {
    printf("error %s\n", na_last_error());
    return 1;
  }
  printf("tiles %d %d %d %d %d %d\n", tq[0], tq[1], tq[2], tk[0], tk[1], tk[2]);

  int nq = 1;
  for (int d = 0; d < 3; ++d) nq *= (grid[d] + tq[d] - 1) / tq[d];
  int32_t* qptr = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nq + 1));
  int32_t* nfull = (int32_t*)malloc(sizeof(int32_t) * (size_t)nq);
  int64_t nnz = 0;
  na_tilemap_stats st;
  /* size query first (no kv_idx), then the real call */
  na_status s = na_build_tile_map(grid, window, stride, tq, tk, qptr, NULL, nfull, 0, &nnz, &st);
  if (s != NA_OK && s != NA_ERR_WORKSPACE && s != NA_ERR_INVALID_ARG) {
    printf("error %s\n", na_last_error());
    return 1;
  }
  int32_t* kv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
  s = na_build_tile_map(grid, window, stride, tq, tk, qptr, kv, nfull, nnz, &nnz, &st);
  if (s != NA_OK) {
    printf("error %s\n", na_last_error());
    return 1;
  }
  long long ksum = 0;
  for (int64_t i = 0; i < nnz; ++i) ksum += kv[i];
  printf("map %lld %lld %lld %lld %lld %lld\n", (long long)st.n_q_tiles, (long long)st.nnz, (long long)st.n_full,
         (long long)st.n_boundary, (long long)st.computed_slots, (long long)st.effective_slots);
  printf("kvsum %lld qptr_last %d\n", ksum, qptr[nq]);

  na_sim_result r;
  if (na_simulate(1, 24, 128, grid, window, stride, NA_BF16, NULL, NULL, &r) != NA_OK) {
    printf("error %s\n", na_last_error());
    return 1;
  }
  printf("sim %d %.6f\n", r.perfectly_block_sparse, r.tile_efficiency);
  printf("workspace %zu\n", na_workspace_bytes(1, 24, 128, grid, window, stride, NA_BF16));
  /* an argument error is reported, not thrown */
  const int bad[3] = {1, 17, 5};
  printf("bad %d\n", (int)na_choose_tiles(grid, bad, stride, 128, NA_BF16, tq, tk));
  free(qptr);
  free(nfull);
  free(kv);
  return 0;
}
