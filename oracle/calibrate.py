"""Threshold calibration from tile margins.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Because the running max that a tile is compared with is the max over all
tiles visited before it -- a skipped tile never raises it, since its local
max lies below the running max -- each tile's margin g_j does not depend on
lambda or on earlier decisions. The skip set at lambda is therefore exactly
{tiles : g_j < lambda} and the skip ratio is the empirical distribution of
the margins. The pages describe choosing the threshold for a target
sparsity by calibration (TRT-LLM page, outlook: automatic calibration to a
target sparsity; ModelOpt tutorial, step 4: search for the threshold that
meets a target ratio).
"""

from __future__ import annotations

import numpy as np


def skip_ratio(margins, lam: float) -> float:
    """Share of visited tiles (non-NaN margin) skipped at ``lam``."""
    g = np.asarray(margins, np.float64).ravel()
    g = g[~np.isnan(g)]
    if g.size == 0:
        return 0.0
    return float(np.count_nonzero(g < lam)) / g.size


def lambda_for_ratio(margins, target: float, window: float = 0.01) -> float:
    """A lambda <= 0 that skips about ``target`` of the visited tiles.

    Sort the margins; among the consecutive pairs whose rank lies within
    +-``window`` of the target rank, take the widest gap between finite
    margins and return its midpoint, so that as few tiles as possible lie
    close to lambda. Clamped to <= 0."""
    g = np.asarray(margins, np.float64).ravel()
    g = np.sort(g[~np.isnan(g)])
    n = g.size
    if n < 2:
        return 0.0
    want = int(round(target * n))
    lo = max(1, int(np.floor((target - window) * n)))
    hi = min(n - 1, int(np.ceil((target + window) * n)))
    lo = min(lo, max(1, want))
    hi = max(hi, min(n - 1, want))
    best, lam = -1.0, None
    for r in range(lo, hi + 1):
        a, b = g[r - 1], g[r]
        if not (np.isfinite(a) and np.isfinite(b)):
            continue
        if b - a > best:
            best, lam = b - a, 0.5 * (a + b)
    if lam is None:
        lam = float(g[min(max(want, 0), n - 1)])
        if not np.isfinite(lam):
            lam = 0.0
    return float(min(lam, 0.0))
