"""CPU oracle for the block-sparse video-attention path (test infrastructure only).

This package is the correctness reference that the HIP library is checked against.  It is
plain, slow NumPy/SciPy in float64 and follows the definitions on the source pages step
by step, with no blocking, fusion or reordering beyond what those definitions state.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import it.
It shares no code with the GPU library and never imports it; the library never imports
this package.

Pages (cited by title and section):
  [SBC]  "Sparse-block compensation" (mlx-arsenal research note): sections "The problem",
         "SVG-EAR -- centroid compensation", "SparsePR -- probe-fitted residual repair",
         "No LSE needed", "Recipe: STA with both repairs", "Deviations from the papers".
  [HMR]  "Dynamic block masks and head-wise mask reuse" (mlx-arsenal research note):
         sections "XAttention -- anti-diagonal block scoring", "HEART -- head-wise temporal
         mask reuse", "What mlx-arsenal ships", "Recipe", "Deviations from the papers",
         "Out of scope, and why" (padding).
  [SPR]  "Partition the Support, Reconstruct the Residual" (paper summary page): the
         paragraphs on Probe-Fitted Residual Reconstruction, group-major permutation and
         grouped-query sharing, and the hard-drop residual statement.
  [BSA]  "Block-sparse attention" (topic page of paper cards): the SVG-EAR card.

Stages (module: function):
  layout.cluster_layout          stable cluster-major order of tokens          [SPR] permutation
  layout.tile_labels             labels of sliding-tile 3-D tiles              [SBC] API table
  centroids.centroids            key/value cluster means and counts            [SBC] SVG-EAR
  scoring.antidiagonal_block_scores  strided antidiagonal block mass          [HMR] XAttention
  topp.top_p_block_mask          per-row top-p keep bits                       [HMR] XAttention
  attention.compensated_attention    softmax over the extended keys            [SBC] No LSE needed
  attention.dense_attention_rows exact dense rows (probes)                     [SPR], [SBC] Recipe
  repair.select_probe_rows       middle-out round-robin probes, |G_a|/m_a      [SBC] API table, Deviations
  repair.ridge_fit               weighted standardized ridge, top-r projection [SPR], [SBC]
  repair.apply_correction        O + dO on every row                           [SPR], [SBC]
  pipeline.run_head              the whole path for one (batch, head)
  reuse.pooled_summary           token means of Q and K per mask head          [HMR] HEART
  reuse.l1_drift                 L1 drift from the anchor (optionally relative) [HMR] HEART, Deviations
  reuse.layer_gate, refresh_decision  per-head refresh with the 40%/80% override [HMR] HEART
  reuse.HeadMaskCache            two-phase cache of masks and anchors          [HMR] ships, Recipe
  static_masks.sliding_tile_block_mask  static sliding-tile (STA) block mask   [SBC] Recipe: STA
  routing.query_centroids        query-cluster means as the routing probes     [BSA] SVG-EAR, [SBC]
  routing.block_compensation_error  first-order output error per block         [BSA] SVG-EAR, [SBC]
  routing.error_aware_route      error-to-cost order under a token budget      [BSA] SVG-EAR

Every function above is pinned by a test under tests/ (test_oracle_*.py) against closed
forms, brute force, library routines or hand-worked fixtures in tests/golden/.
"""

from . import attention, centroids, layout, pipeline, repair, reuse, routing, scoring, static_masks, topp  # noqa: F401
