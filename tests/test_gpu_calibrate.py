"""GPU parity: the device threshold calibration (``ssa_lambda_for_ratio``)
against the oracle's rule (``oracle.lambda_for_ratio`` / ``oracle.skip_ratio``)
on the same fp32 margins: lambda and the achieved ratio must be identical."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _check(g, target, window=0.01, ws=None):
    import sparse_attention_long_skip_amd as ssa
    g = np.ascontiguousarray(g, dtype=np.float32)
    t = torch.from_numpy(g).cuda() if g.size else torch.empty(0, dtype=torch.float32, device="cuda")
    lam, ratio = ssa.lambda_for_ratio(t, target, window, workspace=ws)
    want = oracle.lambda_for_ratio(g.astype(np.float64), target, window)
    assert lam == want, (g.size, target, window, lam, want)
    assert ratio == oracle.skip_ratio(g.astype(np.float64), lam), (ratio, oracle.skip_ratio(g, lam))
    return lam, ratio


def _random_margins(rng, n):
    kind = rng.integers(0, 5)
    if kind == 0:
        g = rng.standard_normal(n) * rng.uniform(0.01, 3.0) - rng.uniform(0, 1)
    elif kind == 1:   # many ties
        g = np.round(rng.standard_normal(n) * 2, int(rng.integers(0, 3)))
    elif kind == 2:   # wide dynamic range, both signs
        g = rng.choice([-1.0, 1.0], n) * 10.0 ** rng.uniform(-30, 30, n)
    elif kind == 3:   # clustered near zero with exact zeros of both signs
        g = rng.standard_normal(n) * 1e-6
        g[rng.random(n) < 0.1] = 0.0
        g[rng.random(n) < 0.1] = -0.0
    else:             # two separated clusters
        g = np.where(rng.random(n) < 0.5, rng.normal(-3, 0.1, n), rng.normal(0.5, 0.1, n))
    g = g.astype(np.float32)
    g[rng.random(n) < rng.uniform(0, 0.3)] = np.inf
    g[rng.random(n) < rng.uniform(0, 0.3)] = np.nan
    g[rng.random(n) < rng.uniform(0, 0.05)] = -np.inf
    return g


def test_random_margins_match_oracle():
    rng = np.random.default_rng(0)
    for case in range(150):
        n = int(rng.choice([0, 1, 2, 3, 5, 17, 100, 1000, 4099, 65536, 300001]))
        g = _random_margins(rng, n)
        for target in (0.0, 0.1, 0.5, 0.93, 1.0):
            window = float(rng.choice([0.0, 0.01, 0.05, 0.5]))
            _check(g, target, window)


def test_degenerate_inputs():
    _check(np.array([], np.float32), 0.5)
    _check(np.full(10, np.nan, np.float32), 0.5)
    _check(np.array([-1.0], np.float32), 0.5)
    _check(np.full(1000, -0.25, np.float32), 0.5)          # all equal
    _check(np.full(1000, np.inf, np.float32), 0.5)         # all first tiles
    _check(np.full(1000, -np.inf, np.float32), 0.5)
    g = np.concatenate([np.full(600, np.inf), np.full(400, -1.0)]).astype(np.float32)
    for t in (0.3, 0.5, 0.7):
        _check(g, t)
    g = np.linspace(-2, 2, 10001).astype(np.float32)       # evenly spaced: many equal gaps
    for t in (0.25, 0.5):
        _check(g, t)


def test_workspace_reuse_second_call_smaller():
    import sparse_attention_long_skip_amd as ssa
    rng = np.random.default_rng(3)
    big = _random_margins(rng, 200000)
    ws = torch.empty(ssa.calibrate_workspace_size(big.size, 0.01), dtype=torch.uint8, device="cuda")
    _check(big, 0.5, 0.01, ws)
    _check(big[:777], 0.4, 0.01, ws)


@pytest.mark.parametrize("cfg", [1, 3])
def test_real_margins_full_size(cfg):
    """Margins of the dense statistics launch at the 16K and 128K shapes."""
    import sparse_attention_long_skip_amd as ssa
    from parity import dev_bf16
    c = synth.CONFIGS[cfg]
    x = synth.prefill_inputs(cfg, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"], frac=c["frac"])
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    del x
    m = ssa.prefill(q, k, v, -math.inf, Br=c["Br"], Bc=c["Bc"], causal=True, lse=False, margins=True)["tile_margin"]
    g = m.cpu().numpy()
    for target in (0.5, 0.3):
        lam, ratio = ssa.lambda_for_ratio(m, target)
        want = oracle.lambda_for_ratio(g, target)
        assert lam == want, (cfg, target, lam, want)
        assert ratio == oracle.skip_ratio(g, lam)
        print(f"config {cfg} target {target}: lambda {lam:.6f}, ratio {ratio:.4f}")


def test_decode_margins_full_size():
    import sparse_attention_long_skip_amd as ssa
    from parity import dev_bf16
    c = synth.CONFIGS[2]
    y = synth.decode_inputs(2, 0, c["B"], c["Hq"], c["Hkv"], c["S_max"], c["d"], c["len_lo"], c["len_hi"],
                            block=c["Bc"], frac=c["frac"])
    seq = torch.from_numpy(np.asarray(y["seqlens"], np.int32)).cuda()
    r = ssa.decode(dev_bf16(y["q"]), dev_bf16(y["k_cache"]), dev_bf16(y["v_cache"]), seq, -math.inf,
                   split_tiles=c["split_tiles"], lse=False, margins=True)
    m = r["tile_margin"]
    g = m.cpu().numpy()
    lam, ratio = ssa.lambda_for_ratio(m, 0.5)
    assert lam == oracle.lambda_for_ratio(g, 0.5)
    assert ratio == oracle.skip_ratio(g, lam)
