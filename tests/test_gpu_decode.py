"""GPU parity: split-K Skip-Softmax decode (HIP, through the C ABI) against the oracle."""

import math

import numpy as np
import pytest

import oracle
import synth
from parity import decode_parity

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 3, 100])
def test_dense_and_calibrated_small(d, T):
    y = synth.decode_inputs(300, d + T, 4, 8, 2, 1000, d, 1, 1000, seqlens=[1, 63, 650, 1000])
    r = decode_parity(y, -math.inf, T)
    assert r["skipped"] == 0
    m = oracle.decode(y["q"], y["k_cache"], y["v_cache"], y["seqlens"], -math.inf, 64, T,
                      bits=True)["margin"]
    lam = oracle.lambda_for_ratio(m, 0.5)
    r = decode_parity(y, lam, T)
    print(f"d={d} T={T} lam={lam:.3f} skipped {r['skipped']}/{r['visited']} exempt {r['exempt']}")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_group_sizes(G, d):
    # every (d, G) instance, including those at one and at two waves per SIMD
    Hkv = 2
    y = synth.decode_inputs(301, G + d, 2, G * Hkv, Hkv, 2048, d, 1500, 2048)
    for lam in (-math.inf, -0.5):
        decode_parity(y, lam, 8)


def test_empty_sequence_and_nan_tail():
    # length 0 -> out 0, lse -inf; the NaN-filled tail must never be read
    y = synth.decode_inputs(302, 0, 3, 4, 1, 512, 128, 0, 512, seqlens=[0, 5, 512])
    r = decode_parity(y, -1.0, 2)
    out = r["gpu"]["out"].float().cpu().numpy()
    assert np.all(out[0] == 0) and np.all(np.isneginf(r["gpu"]["lse"].cpu().numpy()[0]))
    assert np.all(np.isfinite(out))


def test_workspace_reuse_second_call_smaller():
    import torch
    import sparse_attention_long_skip_amd as ssa
    from parity import dev_bf16
    y = synth.decode_inputs(303, 0, 2, 8, 2, 4096, 128, 3000, 4096)
    ws = torch.empty(ssa.decode_workspace_size(2, 8, 4096, 128, 64, 4), dtype=torch.uint8,
                     device="cuda")
    seq = torch.tensor(y["seqlens"], dtype=torch.int32, device="cuda")
    a = ssa.decode(dev_bf16(y["q"]), dev_bf16(y["k_cache"]), dev_bf16(y["v_cache"]), seq, -1.0,
                   split_tiles=4, workspace=ws)
    seq2 = torch.tensor([100, 2000], dtype=torch.int32, device="cuda")
    b = ssa.decode(dev_bf16(y["q"]), dev_bf16(y["k_cache"]), dev_bf16(y["v_cache"]), seq2, -1.0,
                   split_tiles=4, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.decode(y["q"], y["k_cache"], y["v_cache"], [100, 2000], -1.0, 64, 4, bits=True)
    assert np.abs(b["out"].float().cpu().numpy() - ref["out"]).max() < 2e-2


@pytest.mark.parametrize("lens", [[1, 63, 64, 65], [127, 128, 129, 2047]])
def test_length_tile_edges(lens):
    # cache lengths at and around tile and split boundaries (split of 4 tiles)
    y = synth.decode_inputs(302, sum(lens), len(lens), 8, 2, 2048, 128, 1, 2048, seqlens=lens)
    r = decode_parity(y, -0.5, 4)
    print(f"lens={lens}: skipped {r['skipped']}/{r['visited']}")


@pytest.mark.parametrize("lens", [[1535, 1536, 1537, 3072], [64 * 24 * 3 - 1, 1, 64 * 24 + 63, 4100]])
def test_split_boundaries_24(lens):
    # splits of 24 tiles (1536 keys): lengths at and around split ends, the
    # last split partial or a single key long; two query heads per KV head
    y = synth.decode_inputs(304, len(lens), len(lens), 4, 2, 4608, 128, 1, 4608, seqlens=lens)
    for lam in (-math.inf, -0.4):
        r = decode_parity(y, lam, 24)
        print(f"lens={lens} lambda={lam}: skipped {r['skipped']}/{r['visited']}")


@pytest.mark.parametrize("lens", [[1023, 1024, 1025, 2048], [64 * 16 * 3 - 1, 1, 64 * 16 + 63, 4100]])
def test_split_boundaries_16(lens):
    # splits of 16 tiles (1024 keys, the benchmarked split length): lengths at
    # and around split ends; four query heads per KV head
    y = synth.decode_inputs(305, len(lens), len(lens), 8, 2, 4608, 128, 1, 4608, seqlens=lens)
    for lam in (-math.inf, -0.4):
        r = decode_parity(y, lam, 16)
        print(f"lens={lens} lambda={lam}: skipped {r['skipped']}/{r['visited']}")
