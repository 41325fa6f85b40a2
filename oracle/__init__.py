"""Plain CPU oracle for the LiLiCorr reranking path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never calls it and shares no code with
it: the two sides meet only on the seeded inputs drawn by ``synth``.

Every function follows the LiLiCorr paper (arXiv 2608.20530) or the SGLang
pull request "[Spec] Add LiLiCorr: a candidate-lattice reranker for DFlash
drafts", as cited in its docstring. Floating point is float64 except at the
stated rounding points, where values are rounded exactly as the method stores
them (bfloat16 GEMM inputs, float32 log-probabilities, scores and walk sums).

Parity status per part (pins live in the test suite, marked ``not gpu``):
  * top-K / log-partition: pinned (brute-force sort, closed forms, scipy).
  * greedy walk: pinned (exhaustive greedy enumeration, alpha = 0 and K = 1
    special cases, hand-computed fixture).
  * pair scores: pinned (unit-norm invariants, duplicated vectors).
  * encoder: pinned by closed-form special cases (zero output projections,
    one-token lattice, uniform attention, one-hot bias tables, rms-norm scale
    invariance, permutation equivariance) and by an independent float64
    torch build from library routines. The trained head of the paper is not
    published, so no printed value pins the encoder's outputs.
  * synthetic weights: pinned to the published SplitMix64 test vector.
  * the paper's own head (drafter hidden state, target fusion, anchor out
    vector): pinned by an independent float64 torch build and closed forms
    (constant fusion output, zero target projection, hand-worked anchor vector,
    the anchor slot's candidates leaving the lattice untouched).
  * exact best path (paper, Appendix E): pinned (brute force over every path
    of tiny lattices, hand-worked fixtures, never below the greedy total).
  * vocabulary-sharded top-K / log-partition: pinned (equal to the unsplit
    definition for any shard count, ties across shard boundaries, constant rows).
  * sampled commit (PR, opt-in sampling): pinned (hand-worked draws at an
    exact boundary, chi-square of draw frequencies against scipy's softmax,
    greedy rows equal to the greedy walk, vanishing temperature).
"""

from .bf16 import round_bf16, bf16_bits_to_f64, f64_to_bf16_bits  # noqa: F401
from .weights import Dims, OracleWeights, weight_table  # noqa: F401
from .topk_lse import topk_lse_row, topk_lse  # noqa: F401
from .encoder import encode_block  # noqa: F401
from .scores import pair_scores  # noqa: F401
from .walk import greedy_walk, WalkResult  # noqa: F401
from .sharded import shard_bounds, shard_partial, merge_partials, topk_lse_sharded_row  # noqa: F401
from .paths import best_path, sample_path, path_total, PathResult, SampleResult  # noqa: F401
from .paper_head import encode_block_paper  # noqa: F401
from .rerank import rerank_block, BlockResult  # noqa: F401
