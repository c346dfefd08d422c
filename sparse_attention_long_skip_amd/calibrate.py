"""Threshold calibration for a target skip ratio (host side).

The tile margin g_j (the largest row gap of a tile) does not depend on the
threshold: a skipped tile never raises the running max it is compared
with. So the skip set at lambda is {tiles : g_j < lambda}, and one dense
call with margin output (``prefill(..., margins=True)``) gives the skip
ratio of every lambda. The pages call for calibrating the threshold to a
target sparsity (TRT-LLM page, outlook; ModelOpt tutorial, step 4).

Rule: sort the margins of the visited tiles; among consecutive pairs whose
rank lies within +-window of the target rank, take the widest gap between
two finite margins and put lambda at its midpoint (so few tiles sit near
the threshold); clamp to <= 0.
"""

from __future__ import annotations

import math

import numpy as np


def lambda_for_ratio(margins, target: float, window: float = 0.01) -> float:
    g = np.asarray(margins, dtype=np.float64).reshape(-1)
    g = g[~np.isnan(g)]
    n = g.size
    if n < 2:
        return 0.0
    g.sort()
    want = int(round(target * n))
    lo = min(max(1, int(math.floor((target - window) * n))), max(1, want))
    hi = max(min(n - 1, int(math.ceil((target + window) * n))), min(n - 1, want))
    a, b = g[lo - 1:hi], g[lo:hi + 1]
    ok = np.isfinite(a) & np.isfinite(b)
    if ok.any():
        gaps = np.where(ok, b - a, -1.0)
        r = int(np.argmax(gaps))
        lam = 0.5 * (a[r] + b[r])
    else:
        lam = g[min(max(want, 0), n - 1)]
        if not np.isfinite(lam):
            lam = 0.0
    return float(min(lam, 0.0))


def skip_ratio(margins, lam: float) -> float:
    g = np.asarray(margins, dtype=np.float64).reshape(-1)
    g = g[~np.isnan(g)]
    return float(np.count_nonzero(g < lam)) / max(1, g.size)


def calibrate_prefill(q, k, v, target: float, Br: int = 128, Bc: int = 64, causal: bool = True,
                      block_idx=None, block_cnt=None) -> tuple:
    """Run the HIP prefill once densely with margin output; return
    (lambda, achieved skip ratio at lambda)."""
    from . import _lib
    r = _lib.prefill(q, k, v, float("-inf"), Br=Br, Bc=Bc, causal=causal, block_idx=block_idx,
                     block_cnt=block_cnt, lse=False, margins=True)
    m = r["tile_margin"].cpu().numpy()
    lam = lambda_for_ratio(m, target)
    return lam, skip_ratio(m, lam)


def calibrate_decode(q, k_cache, v_cache, seqlens, target: float, split_tiles: int = 32,
                     Bc: int = 64) -> tuple:
    """Decode analogue of calibrate_prefill."""
    from . import _lib
    r = _lib.decode(q, k_cache, v_cache, seqlens, float("-inf"), split_tiles=split_tiles, Bc=Bc,
                    lse=False, margins=True)
    m = r["tile_margin"].cpu().numpy()
    lam = lambda_for_ratio(m, target)
    return lam, skip_ratio(m, lam)
