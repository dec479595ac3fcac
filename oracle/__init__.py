"""Plain fp64 CPU oracle for online log-domain Sinkhorn.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link this package: only the test-suite, the smoke check in
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.
It shares no code with the HIP library and imports nothing from it.

Everything here is written from the pages for readability, not speed:
  * the cost matrix is formed explicitly (in row chunks when large);
  * every log-sum-exp is an explicit max-shifted sum in float64;
  * inputs are the float32 arrays converted exactly to float64.

Sources (cited by page title and section in each module):
  * "FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport" (paper
    summary): the problem, the alternating dual updates, annealing, Morton
    blocks and cells, the coarse lift, the block-pair screen, sparse
    half-steps and the residual certificate.
  * moscot pull request #846, "fix(sparsify): materialize transport-matrix
    rows instead of pushing indicator columns": the entropic row formula,
    the resolved cost scale and the ``min_row`` threshold.
  * POT pull request #868 (N-D convolutional barycenters): the all -inf
    row convention of a log-sum-exp.
  * FlashSinkhorn 2, §A.2 and §A.4: the barycentric projection of plan rows
    and the source-coordinate gradient (``bary``).

Pinning status: every public function is pinned by a CPU test in
``tests/test_oracle_*.py`` (closed forms, brute force on tiny inputs,
invariants). None is "parity unpinned".
"""
from .dense import (  # noqa: F401
    Schedule,
    SolveResult,
    annealing_stages,
    cost_rows,
    halfstep_f,
    halfstep_g,
    logsumexp_rows,
    marginal_residuals,
    materialize_rows,
    mean_sqeuclid,
    min_row,
    plan_rows,
    row_residual_identity,
    solve,
    sparsify,
)
from .morton import interleave, morton_codes, morton_order, quantize  # noqa: F401
from .blocks import (  # noqa: F401
    block_summaries,
    compact_tiles,
    screen,
    screen_transpose,
    sparse_halfstep_f,
    sparse_halfstep_g,
    sparse_residuals,
    tile_shares,
    verify_tiles,
)
from .fs2 import FS2Params, cells, fs2_solve, lift  # noqa: F401
from .bary import barycentric_rows, coordinate_gradient, sparse_barycentric_rows  # noqa: F401
