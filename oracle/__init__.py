"""CPU fp64 oracle for KPage-style block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU path never calls
it, and it shares no code with the GPU path (no kernels, headers, helpers or
table generators).

Source: "KPage: Cross-Block Page Compaction for Hardware-Efficient Sparse
Attention" (arXiv 2610.28096), sections 3.2-3.4.

* ``attention``: plain-definition masked softmax attention, forward and
  backward, over exactly the valid token pairs of the block graph.
* ``planner``: the page-table, route, validity, owner, reverse-Q, Q-page and
  adjacency construction, step by step, in integers, plus the pair statistics
  of section 4.4.
* ``selection``: block mean pooling, block scores and top-k selection in a fixed
  fp64 operation order (the selector in front of KPage that produces its graph).
* ``layout``: the oracle's own reading of how a T x H x W token grid is
  flattened into 128-row blocks, used to check block-sparse results against
  dense attention over the original tokens.

Every function here is pinned by a CPU test (tests/test_oracle_*.py) against
closed forms, brute force, dense attention, autograd or finite differences.
"""
from .attention import (  # noqa: F401
    oracle_bwd,
    oracle_fwd,
    oracle_fwd_block,
    brute_force_fwd,
)
from .planner import oracle_plan, PlanTables  # noqa: F401
from .selection import block_means, block_scores, select_top_p, select_topk, top_p_clusters, topk_rows  # noqa: F401
