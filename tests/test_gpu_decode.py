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
    # every (d, G) instance of the split kernel
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


def test_work_queue_sparse_tickets_and_reuse():
    # The split kernel hands out (sequence, KV head, split) tickets from a work
    # counter. Here a third of the sequences are empty and a third hold under
    # two tiles, so most tickets fall past a sequence's end and the counter
    # jumps; 48 * 4 * 32 = 6144 tickets for 768 waves. Two calls on one
    # workspace (the counter is set by each call), the second with fewer
    # sequences and shorter lengths (rows past the first call's lengths are
    # NaN in these caches).
    import torch
    import sparse_attention_long_skip_amd as ssa
    from parity import dev_bf16
    rng = np.random.default_rng(306)
    B, S = 48, 4096
    i = np.arange(B)
    lens = np.where(i % 3 == 0, 0, np.where(i % 3 == 1, rng.integers(1, 128, B), rng.integers(1000, S + 1, B)))
    y = synth.decode_inputs(306, 0, B, 8, 4, S, 128, 1, S, seqlens=lens)
    r = decode_parity(y, -0.5, 2)
    print(f"skipped {r['skipped']}/{r['visited']}")
    ws = torch.empty(ssa.decode_workspace_size(B, 8, S, 128, 64, 2), dtype=torch.uint8, device="cuda")
    q, kc, vc = dev_bf16(y["q"]), dev_bf16(y["k_cache"]), dev_bf16(y["v_cache"])
    for call, lens_c in enumerate((lens, lens[:40] // 2)):
        Bc = len(lens_c)
        seq = torch.tensor(lens_c, dtype=torch.int32, device="cuda")
        g = ssa.decode(q[:Bc], kc[:Bc], vc[:Bc], seq, -0.5, split_tiles=2, workspace=ws, counts=True)
        torch.cuda.synchronize()
        ref = oracle.decode(y["q"][:Bc], y["k_cache"][:Bc], y["v_cache"][:Bc], lens_c, -0.5, 64, 2,
                            bits=True)
        out = g["out"].float().cpu().numpy()
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(ref["out"])), f"call {call}"
        assert np.abs(out - ref["out"]).max() < 2e-2, f"call {call}"
        sc = g["skip_counts"].cpu().numpy()
        # splits past the end of a sequence report 0; the rest within the band
        for b in range(Bc):
            nsp = -(-(-(-int(lens_c[b]) // 64)) // 2)
            assert np.all(sc[b, :, nsp:] == 0)
        assert abs(int(sc.sum()) - int(ref["skip_counts"].sum())) <= max(2, int(0.01 * ref["skip_counts"].sum()))


def test_work_queue_many_short_sequences():
    # 256 sequences of 1..700 keys, one-tile splits: 256 * 2 * 11 = 5632
    # tickets, many times the wave count, so every wave runs a long chain of
    # splits (including empty ones) from the work counter.
    rng = np.random.default_rng(307)
    B, S = 256, 700
    lens = rng.integers(1, S + 1, B)
    lens[::17] = 0
    y = synth.decode_inputs(307, 0, B, 4, 2, S, 64, 1, S, seqlens=lens)
    for lam in (-math.inf, -0.7):
        r = decode_parity(y, lam, 1)
        print(f"lambda={lam}: skipped {r['skipped']}/{r['visited']}")
