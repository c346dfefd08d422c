"""GPU parity: SpargeAttn stage-one mask (block self-similarity gate,
compressed map, Top-tau selection) and the two-stage pipeline (stage-one
lists, then the skip rule inside block-sparse prefill) against the oracle."""

import math

import numpy as np
import pytest

import oracle
import synth
from parity import prefill_parity, sparge_parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", ["mass", "count"])
@pytest.mark.parametrize("L,theta,tau", [(1000, 0.2, 0.9), (4096, 0.3, 0.5), (333, 0.5, 0.95)])
def test_sparge_small(d, mode, L, theta, tau):
    x = synth.prefill_inputs(600, L + d, 1, 3, 3, L, d, drift=2.0 if d == 64 else 2.8)
    r = sparge_parity(x["q"], x["k"], theta, tau, mode)
    print(f"d={d} L={L} {mode}: rows at a decision band {r['near']}")


@pytest.mark.parametrize("mode", ["mass", "count"])
def test_sparge_long_sequence(mode):
    # nB = 1100 > 1024: one row per workgroup, candidates kept in LDS
    x = synth.prefill_inputs(601, 0, 1, 1, 1, 1100 * 64 - 17, 64, drift=2.0)
    r = sparge_parity(x["q"], x["k"], 0.2, 0.9, mode)
    print(f"{mode}: rows at a decision band {r['near']}")


def test_sparge_limits():
    import torch
    import sparse_attention_long_skip_amd as ssa
    x = synth.prefill_inputs(602, 0, 1, 2, 2, 64 * 37 + 5, 64, drift=2.0)
    q, k = (torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k"))
    nB = 38
    dense = [list(range(b + 1)) for b in range(nB)]
    # theta above every similarity: nothing compressed, dense lists
    g = ssa.sparge_mask(q, k, 2.0, 0.5)
    # theta below every similarity with count mode and tau = 1: every block
    f = ssa.sparge_mask(q, k, -2.0, 1.0, "count")
    # everything compressed, tiny tau: exactly the oracle's argmax block
    t = ssa.sparge_mask(q, k, -2.0, 1e-9, "mass", scores=True)
    torch.cuda.synchronize()
    for res in (g, f):
        idx, cnt = res["block_idx"].cpu().numpy(), res["block_cnt"].cpu().numpy()
        for h in range(2):
            assert [idx[0, h, b, :cnt[0, h, b]].tolist() for b in range(nB)] == dense
    assert np.all(t["block_cnt"].cpu().numpy() == 1)
    ref = oracle.sparge_mask(x["q"], x["k"], 64, -2.0, 1e-9, bits=True)
    gap = np.sort(ref["phat"], axis=-1)
    clear = (gap[..., -1] - gap[..., -2]) > 1e-4
    np.testing.assert_array_equal(t["block_idx"].cpu().numpy()[..., 0][clear],
                                  ref["block_idx"][..., 0][clear])


def test_sparge_two_stage_pipeline():
    # stage one picks the lists, stage two (skip rule) runs inside prefill
    import torch
    import sparse_attention_long_skip_amd as ssa
    from parity import dev_bf16, to_np
    x = synth.prefill_inputs(603, 0, 1, 2, 2, 3000, 64, drift=2.0)
    g = ssa.sparge_mask(dev_bf16(x["q"]), dev_bf16(x["k"]), 0.2, 0.9)
    torch.cuda.synchronize()
    ref = oracle.sparge_mask(x["q"], x["k"], 64, 0.2, 0.9, bits=True)
    gi, gc = to_np(g["block_idx"]), to_np(g["block_cnt"])
    np.testing.assert_array_equal(gc, ref["block_cnt"])
    np.testing.assert_array_equal(gi, ref["block_idx"])
    kept = gc.sum() / (2 * 47 * 48 / 2)
    for lam in (-math.inf, -4.0):
        r = prefill_parity(x["q"], x["k"], x["v"], lam, 64, 64, True,
                           block_idx=ref["block_idx"].astype(np.int32),
                           block_cnt=ref["block_cnt"].astype(np.int32))
        print(f"kept blocks {kept:.2f}, lam={lam}: skipped {r['skipped']}/{r['visited']}")


def test_sparge_batched_heads():
    # B = 2: batch and head indexing of every workspace and output
    x = synth.prefill_inputs(605, 1, 2, 3, 3, 64 * 20 + 9, 64, drift=2.0)
    r = sparge_parity(x["q"], x["k"], 0.25, 0.8, "mass")
    print(f"rows at a decision band {r['near']}")
