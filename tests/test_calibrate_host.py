"""Host-side threshold calibration of the library against the oracle's rule."""

import numpy as np

import oracle
from sparse_attention_long_skip_amd import calibrate


def test_matches_oracle_rule():
    rng = np.random.default_rng(0)
    for t in range(30):
        g = rng.standard_normal(int(rng.integers(10, 5000))) * rng.uniform(0.1, 3) - rng.uniform(0, 2)
        g[rng.random(g.size) < 0.05] = np.inf
        g[rng.random(g.size) < 0.05] = np.nan
        g[rng.random(g.size) < 0.02] = -np.inf
        for target in (0.1, 0.5, 0.8):
            a = calibrate.lambda_for_ratio(g, target)
            b = oracle.lambda_for_ratio(g, target)
            assert a == b, (t, target, a, b)
            assert calibrate.skip_ratio(g, a) == oracle.skip_ratio(g, a)
