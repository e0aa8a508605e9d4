"""CPU oracle for the GNA sparse-attention forward and backward passes.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the test-suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code, header, table or helper with the HIP library.

Everything here is plain NumPy in float64 and follows the pages'
definitions directly (no blocking, fusion or reordering beyond what the
definition states):

* ``window_start`` / ``key_set`` -- which keys a query sees
  ("GNA Sparse Attention Mechanism: Vision-Transformer Compute Optimisation
  in Practice", section 1.1: a fixed window around each query, with a stride
  that makes the window move in jumps between stride groups).
* ``attend`` -- exact masked softmax attention over that key set, with the
  natural-log logsumexp ("Video-generation inference speed-up: sparse
  attention configuration tutorial", section 3.3, attention over the kept
  connections without an L x L matrix; softmax kept in FP32 or wider,
  "Sparse attention in video and image generation: optimisation practice",
  section 3.1).
* ``attend_backward`` -- the gradients of ``attend`` for the loss
  sum <dout, out> (plain derivatives; GNA page section 5 names training as
  the next step), with ``query_index_lists`` for the queries that attend a
  key.
* ``topk_select`` / ``topk_attend`` -- content-selected block sparsity:
  block-mean importance scores, the top-k KV tiles per Q tile, attention
  over the kept tiles (tutorial section 6; overview page section 2.2).
* ``tile_map`` -- for each query tile, the key tiles it needs, split into
  full and boundary tiles (GNA page, section 1.1 multi-dimensional tiling
  and the perfectly block-sparse case; section 2.1 fine-grained mask only on
  tiles not fully inside the window), by brute-force pair counting.
"""

from .gna import (  # noqa: F401
    validate_geometry,
    window_start,
    window_starts,
    key_set,
    key_index_table,
    attend,
    tile_map,
    tile_pairs_1d,
    tile_map_stats,
    effective_flops,
    sparsity,
)
from .backward import attend_backward, query_index_lists  # noqa: F401
from .topk import (  # noqa: F401
    block_means_f32,
    block_scores_f32,
    kv_tile_is_full,
    select_blocks,
    topk_attend,
    topk_select,
)
