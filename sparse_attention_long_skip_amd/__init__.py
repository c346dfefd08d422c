"""Skip-Softmax sparse attention for AMD MI355X (gfx950).

Causal GQA prefill with Skip-Softmax tile skipping, single-token split-K
decode with a log-sum-exp combine, N:M sparse softmax prefill, and the
block-sparse prefill predictors (pooled-score top-k, with plain or
overlapping-window key compression; the SpargeAttn stage-one mask; the
vertical-slash estimator). The computation lives in hand-written HIP kernels
behind the C ABI of ``include/ssa.h`` (``libssa.so``); this package is a thin
ctypes binding that marshals torch tensors and the current stream.
"""

from ._lib import (  # noqa: F401
    SSAError, TILE_KEPT, TILE_SKIPPED, SSA_OK, SSA_ERR_INVALID_ARG, SSA_ERR_UNSUPPORTED,
    SSA_ERR_WORKSPACE, SSA_ERR_HIP, SSA_ERR_SCRATCH, DECODE_SCRATCH_BYTES, LIB_PATH, lib,
    status_string, abi_version,
    lambda_from_scale_factor, prefill, decode, decode_workspace_size, block_mask,
    block_mask_compressed_workspace_size,
    block_mask_max_blocks, block_mask_workspace_size, sparge_mask, sparge_mask_workspace_size,
    TAU_MODES, vertical_slash_mask, vertical_slash_workspace_size, lambda_for_ratio,
    calibrate_workspace_size,
)
