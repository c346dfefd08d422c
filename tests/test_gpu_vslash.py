"""GPU parity: vertical-slash block estimator (last-query scores, top vertical
keys and slash offsets, tile cover) and block-sparse prefill over its lists."""

import math

import numpy as np
import pytest

import synth
from parity import prefill_parity, vslash_parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,last_q,nv,ns", [(1000, 64, 50, 20), (333, 1, 10, 5), (4096, 17, 300, 64),
                                            (64 * 70 + 40, 64, 0, 30), (500, 64, 600, 600),
                                            (700, 33, 40, 0)])
def test_vslash_small(d, L, last_q, nv, ns):
    x = synth.prefill_inputs(800, L + last_q, 1, 2, 2, L, d)
    r = vslash_parity(x["q"], x["k"], last_q, nv, ns)
    print(f"d={d} L={L} R={last_q} nv={nv} ns={ns}: heads with near-ties {r['tie_heads']}")
    assert r["tie_heads"] == 0


def test_vslash_long_sequence():
    # nB > 1024 and 128 keys per selection thread
    x = synth.prefill_inputs(801, 0, 1, 1, 1, 1100 * 64 - 17, 64)
    r = vslash_parity(x["q"], x["k"], 64, 1000, 64)
    print(f"heads with near-ties {r['tie_heads']}")


def test_vslash_full_size_sampled_heads():
    c = synth.CONFIGS[4]
    x = synth.prefill_inputs(4, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], block=c["Bc"], frac=c["frac"])
    r = vslash_parity(x["q"], x["k"], 64, 1000, 64, heads=[(0, 0), (0, 11)])
    print(f"heads with near-ties {r['tie_heads']}")


def test_vslash_pipeline_prefill():
    x = synth.prefill_inputs(802, 0, 1, 2, 2, 3000, 64)
    r = vslash_parity(x["q"], x["k"], 64, 100, 16)
    assert r["tie_heads"] == 0
    ref = [r["refs"][(0, h)] for h in range(2)]
    bi = np.concatenate([o["block_idx"] for o in ref], axis=1).astype(np.int32)
    bc = np.concatenate([o["block_cnt"] for o in ref], axis=1).astype(np.int32)
    for lam in (-math.inf, -5.0):
        p = prefill_parity(x["q"], x["k"], x["v"], lam, 64, 64, True, block_idx=bi, block_cnt=bc)
        print(f"lam={lam}: skipped {p['skipped']}/{p['visited']}")


@pytest.mark.parametrize("d", [64, 128])
def test_vslash_batched_heads(d):
    # B = 2: batch and head indexing of every workspace section and output
    x = synth.prefill_inputs(803, d, 2, 3, 3, 64 * 30 + 7, d)
    r = vslash_parity(x["q"], x["k"], 48, 90, 20)
    print(f"heads with near-ties {r['tie_heads']}")
