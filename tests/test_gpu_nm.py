"""GPU parity: N:M sparse softmax prefill (ssa_prefill_nm) against the oracle."""

import math

import numpy as np
import pytest

import oracle
import synth
from parity import prefill_parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,Br", [(64, 64), (128, 128), (128, 64), (64, 128), (128, 32)])
@pytest.mark.parametrize("n,m", [(2, 4), (1, 4), (3, 4), (1, 2)])
def test_nm_dense_small(d, Br, n, m):
    x = synth.prefill_inputs(500, n * 10 + m, 1, 2, 1, 333, d)
    for causal in (True, False):
        r = prefill_parity(x["q"], x["k"], x["v"], -math.inf, Br, 64, causal, nm=(n, m))
        assert r["skipped"] == 0


@pytest.mark.parametrize("sink,recent", [(4, 0), (0, 100), (64, 256)])
def test_nm_with_dense_sink_and_recent(sink, recent):
    x = synth.prefill_inputs(501, sink + recent, 1, 4, 2, 700, 128)
    prefill_parity(x["q"], x["k"], x["v"], -math.inf, 128, 64, True, nm=(2, 4), dense_sink=sink,
                   dense_recent=recent)


def test_nm_combined_with_skip_rule():
    x = synth.prefill_inputs(502, 0, 1, 4, 2, 1000, 128)
    m = oracle.prefill(x["q"], x["k"], x["v"], -math.inf, 128, 64, True, bits=True, nm=(2, 4),
                       dense_sink=64, dense_recent=128)["margin"]
    lam = oracle.lambda_for_ratio(m, 0.3)
    r = prefill_parity(x["q"], x["k"], x["v"], lam, 128, 64, True, nm=(2, 4), dense_sink=64,
                       dense_recent=128)
    print(f"lambda {lam:.3f}: skipped {r['skipped']}/{r['visited']} exempt {r['exempt']}")


@pytest.mark.parametrize("causal", [True, False])
def test_nm_2of4_exact_ties(causal):
    # duplicated key rows inside groups of 4 give exactly equal scores (the
    # same products in the same order on both sides): two-way ties in every
    # second group and a three-way tie in every fourth, so the lower key
    # index decides which equal score is kept
    x = synth.prefill_inputs(503, 7, 1, 4, 2, 600, 128)
    k = x["k"].copy()
    k[:, :, 1::8, :] = k[:, :, 2::8, :][:, :, : k[:, :, 1::8, :].shape[2], :]
    k[:, :, 3::16, :] = k[:, :, 2::16, :][:, :, : k[:, :, 3::16, :].shape[2], :]
    r = prefill_parity(x["q"], k, x["v"], -math.inf, 128, 64, causal, nm=(2, 4))
    assert r["skipped"] == 0
