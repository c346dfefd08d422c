"""Threshold calibration for a target skip ratio.

The tile margin g_j (the largest row gap of a tile) does not depend on the
threshold: a skipped tile never raises the running max it is compared
with. So the skip set at lambda is {tiles : g_j < lambda}, and one dense
call with margin output (``prefill(..., margins=True)``) gives the skip
ratio of every lambda. The pages call for calibrating the threshold to a
target sparsity (TRT-LLM page, efficiency and accuracy: an automatic
calibration program; ModelOpt tutorial, step 4).

The quantile runs on the device (``ssa_lambda_for_ratio``): among the sorted
margins within +-1% of the target rank, the midpoint of the widest gap
between two finite margins, clamped to <= 0. Nothing is copied to the host
but the four result numbers.
"""

from __future__ import annotations


def calibrate_prefill(q, k, v, target: float, Br: int = 128, Bc: int = 64, causal: bool = True,
                      block_idx=None, block_cnt=None, nm=None, dense_sink: int = 0,
                      dense_recent: int = 0, window: float = 0.01) -> tuple:
    """Run the HIP prefill once densely with margin output and the device
    quantile on the margins; return (lambda, achieved skip ratio at lambda)."""
    from . import _lib
    r = _lib.prefill(q, k, v, float("-inf"), Br=Br, Bc=Bc, causal=causal, block_idx=block_idx,
                     block_cnt=block_cnt, lse=False, margins=True, nm=nm, dense_sink=dense_sink,
                     dense_recent=dense_recent)
    return _lib.lambda_for_ratio(r["tile_margin"], target, window)


def calibrate_decode(q, k_cache, v_cache, seqlens, target: float, split_tiles: int = 32,
                     Bc: int = 64, window: float = 0.01) -> tuple:
    """Decode analogue of calibrate_prefill."""
    from . import _lib
    r = _lib.decode(q, k_cache, v_cache, seqlens, float("-inf"), split_tiles=split_tiles, Bc=Bc,
                    lse=False, margins=True)
    return _lib.lambda_for_ratio(r["tile_margin"], target, window)
