"""GPU parity: pooled-score block mask and block-sparse prefill against the oracle."""

import math

import numpy as np
import pytest

import oracle
import synth
from parity import mask_parity, prefill_parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,topk,sink,win", [(1000, 4, 1, 128), (4096, 16, 2, 256), (333, 64, 1, 1024)])
def test_mask_small(d, L, topk, sink, win):
    x = synth.prefill_inputs(400, L, 1, 3, 3, L, d)
    r = mask_parity(x["q"], x["k"], 64, topk, sink, win)
    print(f"d={d} L={L}: near-tie differences {r['ties']}")


def test_block_sparse_prefill_with_oracle_mask():
    x = synth.prefill_inputs(401, 0, 1, 2, 2, 2000, 64)
    m = oracle.block_mask(x["q"], x["k"], 64, 6, 1, 256, bits=True)
    for lam in (-math.inf, -6.0, -0.3):
        r = prefill_parity(x["q"], x["k"], x["v"], lam, 64, 64, True,
                           block_idx=m["block_idx"].astype(np.int32),
                           block_cnt=m["block_cnt"].astype(np.int32))
        print(f"lam={lam}: skipped {r['skipped']}/{r['visited']}")
