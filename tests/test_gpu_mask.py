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


def test_mask_long_sequence_radix_path():
    # nB = 1100 > 1024 exercises the one-row-per-workgroup instance
    x = synth.prefill_inputs(402, 0, 1, 1, 1, 1100 * 64 - 17, 64)
    r = mask_parity(x["q"], x["k"], 64, 64, 1, 1024)
    print(f"near-tie differences {r['ties']}")


def test_mask_ties_prefer_lower_index():
    import torch
    import sparse_attention_long_skip_amd as ssa
    # identical rows everywhere: all pooled scores tie, so the top-k are the lowest indices
    q = torch.ones((1, 1, 64 * 40, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.ones_like(q)
    g = ssa.block_mask(q, k, 64, 5, 0, 0)
    torch.cuda.synchronize()
    idx, cnt = g["block_idx"].cpu().numpy(), g["block_cnt"].cpu().numpy()
    for b in range(40):
        assert idx[0, 0, b, :cnt[0, 0, b]].tolist() == list(range(min(5, b + 1)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,topk,sink,win", [(1000, 4, 1, 128), (4096, 16, 2, 256), (333, 64, 1, 1024),
                                             (64 * 70 + 40, 8, 1, 64)])
def test_compressed_mask(d, L, topk, sink, win):
    # NOSA overlapping key compression: windows of 32 keys every 16
    x = synth.prefill_inputs(403, L, 1, 3, 3, L, d)
    r = mask_parity(x["q"], x["k"], 64, topk, sink, win, compress=(32, 16))
    print(f"d={d} L={L}: near-tie differences {r['ties']}")


def test_compressed_mask_long_sequence():
    x = synth.prefill_inputs(404, 0, 1, 1, 1, 1100 * 64 - 17, 64)
    r = mask_parity(x["q"], x["k"], 64, 64, 1, 1024, compress=(32, 16))
    print(f"near-tie differences {r['ties']}")


def test_masks_batched_heads():
    # B = 2 for the pooled and the compressed mask
    x = synth.prefill_inputs(405, 0, 2, 3, 3, 64 * 25 + 33, 64)
    for compress in (None, (32, 16)):
        r = mask_parity(x["q"], x["k"], 64, 7, 1, 192, compress=compress)
        print(f"compress={compress}: near-tie differences {r['ties']}")
