"""Plain fp64 CPU oracle for RoPE-aware, importance-estimated sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the GPU library.

Sources (web summaries of three papers):

* "Prism: Spectral-Aware Block-Sparse Attention" -- block-sparse prefill
  (sec. 1), mean-pooled block importance (sec. 1), the RoPE x mean-pooling
  analysis (sec. 2), dual-band estimation (sec. 3, item 1) and energy-based
  temperature calibration (sec. 3, item 2).
* "Scaling Attention via Feature Sparsity" -- k-sparse query / key codes
  and scores over the intersection of their active channels (sec. 2),
  ``oracle/feature_sparse.py``.
* "FASA: Frequency-aware Sparse Attention" -- frequency chunks (sec. 2.A),
  the Token Importance Predictor and Focused Attention Computation
  (sec. 2.B), the computation-optimised variant that keeps only a sparse
  subset of key states on the read path (sec. 2.C), and the one-time offline
  calibration of the dominant chunks (sec. 2.B item 1; criterion read here,
  see ``oracle/calibration.py``).

Neither page prints a formula for these steps; the readings taken here are
listed at each function.  Parity of the calibration formula and of the band
combination rule against the original papers is UNPINNED: the pages give no
worked example, so this oracle defines them.
"""
from .sparse_attention import (  # noqa: F401
    rope_frequencies, rope, band_channels, pool_blocks, block_scores, select_row, select_rows,
    prefill_attention, decode_query, token_scores, decode_attention, slab_to_standard,
    standard_to_slab, prefill_pipeline, decode_pipeline, keep_budget,
)
from .calibration import (  # noqa: F401
    calibration_scores, topk_set, overlap_counts, calibrate_dominant,
)
from .feature_sparse import sparsify, intersection_score, sfa_attention  # noqa: F401
