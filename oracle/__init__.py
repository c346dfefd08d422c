"""Oracle: a plain, slow fp64 CPU definition of Skip-Softmax attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library calls it: only the tests,
the smoke check and the benchmark's CPU-baseline leg import it. It shares no
code with the HIP path; both receive the same inputs from ``synth``.

What it defines (sources: the pages on Skip-Softmax attention):

* ``attention.prefill`` -- FlashAttention-style tiled attention with the
  Skip-Softmax rule ("TRT-LLM sparse attention" page, the three-step
  algorithm: block-local max, comparison with the running max, skip of the
  softmax, the second matmul and the V load; SpargeAttn page, stage two of
  the online filter, threshold lambda < 0).
* ``attention.decode`` -- single-token decode with split-K partials and the
  log-sum-exp combine (same rule; the combine is the standard identity).
* ``attention.replay`` -- the outputs for a given set of skip decisions.
* ``block_mask.block_mask`` -- mean-pooled Q/K block scores with top-k,
  sink block and local window (MInference page, block-sparse pattern and its
  ``block_sparse_attention(..., topk=64)`` call; NOSA page, section 3:
  ``init_blocks=1``, ``window_size=1024``, ``topk=64``).
* ``block_mask.block_scores_compressed`` -- block scores from overlapping
  mean-compressed keys (NOSA page, section 1: kernel_size=32, stride=16),
  fed to the same top-k / sink / window selection.
* ``block_mask.sparge_mask`` -- the SpargeAttn stage-one predictor: block
  self-similarity gate, compressed attention map, top mass selection
  (SpargeAttn page, stage one of the two-stage online filter).
* ``vertical_slash.vertical_slash_mask`` -- the vertical-slash estimator
  (MInference page: the last query rows score every key; the best columns
  and diagonals are kept) and the tiles that cover them.
* ``calibrate.lambda_for_ratio`` -- the threshold that skips a target share
  of tiles, from the margins.
* ``bruteforce`` -- a second, scalar-loop implementation for tiny inputs.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute force and invariants.
"""

from .attention import prefill, decode, replay, combine, visited_tiles, lse_combine_parts
from .block_mask import (pool_blocks, block_scores, block_mask, block_self_similarity, sparge_mask,
                         compress_keys, block_scores_compressed)
from .calibrate import lambda_for_ratio, skip_ratio
from .vertical_slash import vertical_slash_scores, vertical_slash_mask, cover_blocks

__all__ = [
    "prefill", "decode", "replay", "combine", "visited_tiles", "lse_combine_parts",
    "pool_blocks", "block_scores", "block_mask", "block_self_similarity", "sparge_mask",
    "compress_keys", "block_scores_compressed",
    "lambda_for_ratio", "skip_ratio",
    "vertical_slash_scores", "vertical_slash_mask", "cover_blocks",
]
