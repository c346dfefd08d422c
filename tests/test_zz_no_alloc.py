"""GPU: the allocation-free decode entry point (``ssa_decode_noalloc``,
static device scratch) against ``ssa_decode`` with a caller workspace, on
two calls in a row, the second smaller, and after the shared scratch was
used by a larger call: outputs, lse and skip counts must be identical."""

import math

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run(cfg_seed, B, Hq, Hkv, S_max, d, lo, hi, T, lam):
    import sparse_attention_long_skip_amd as ssa
    y = synth.decode_inputs(950, cfg_seed, B, Hq, Hkv, S_max, d, lo, hi)
    q, kc, vc = _dev(y["q"]), _dev(y["k_cache"]), _dev(y["v_cache"])
    seq = torch.from_numpy(np.asarray(y["seqlens"], np.int32)).cuda()
    ref = ssa.decode(q, kc, vc, seq, lam, split_tiles=T, counts=True)
    got = ssa.decode(q, kc, vc, seq, lam, split_tiles=T, counts=True, noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(got["out"], ref["out"])
    assert torch.equal(got["lse"], ref["lse"])
    assert torch.equal(got["skip_counts"], ref["skip_counts"])
    return int(ref["skip_counts"].sum())


def test_decode_noalloc_matches_decode_two_calls():
    import sparse_attention_long_skip_amd as ssa
    big = (4, 32, 8, 32768, 128, 16384, 32768, 24)
    assert ssa.decode_workspace_size(4, 32, 32768, 128, 64, 24) <= ssa.DECODE_SCRATCH_BYTES
    s1 = _run(1, *big, -0.5)
    s2 = _run(2, 3, 8, 2, 5000, 64, 100, 5000, 4, -1.0)
    assert s1 > 0 and s2 > 0
    # near the scratch limit (33.0 MB of partials), then small again
    near = (31, 32, 8, 8192, 128, 4096, 8192, 2)
    assert 0.9 * ssa.DECODE_SCRATCH_BYTES < ssa.decode_workspace_size(31, 32, 8192, 128, 64, 2) \
        <= ssa.DECODE_SCRATCH_BYTES
    _run(3, *near, -0.5)
    _run(4, 2, 4, 4, 777, 128, 1, 777, 3, -math.inf)


def test_decode_noalloc_rejects_oversize():
    """A call whose partials exceed the static scratch is refused with
    SSA_ERR_SCRATCH (the buffers are allocated at full size, so the check
    guards nothing out of bounds)."""
    import sparse_attention_long_skip_amd as ssa
    B, Hq, Hkv, S_max, d = 32, 32, 8, 8192, 128
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Hkv, S_max, d), dtype=torch.bfloat16, device="cuda")
    seq = torch.full((B,), S_max, dtype=torch.int32, device="cuda")
    assert ssa.decode_workspace_size(B, Hq, S_max, d, 64, 2) > ssa.DECODE_SCRATCH_BYTES
    with pytest.raises(ssa.SSAError) as e:
        ssa.decode(q, kc, kc, seq, -1.0, split_tiles=2, noalloc=True)
    assert e.value.status == ssa.SSA_ERR_SCRATCH
