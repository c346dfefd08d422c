"""GPU parity: Skip-Softmax prefill (HIP, through the C ABI) against the oracle."""

import math

import numpy as np
import pytest

import oracle
import synth
from parity import prefill_parity

pytestmark = pytest.mark.gpu


def _inputs(cfg, seed, B, Hq, Hkv, L, d, frac=0.1):
    x = synth.prefill_inputs(cfg, seed, B, Hq, Hkv, L, d, block=64, frac=frac)
    return x["q"], x["k"], x["v"]


@pytest.mark.parametrize("d,Br", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_small_ragged(d, Br, causal):
    # L = 333 spans several tiles of both sizes with a ragged tail.
    q, k, v = _inputs(200, 1, 1, 2, 1, 333, d)
    r = prefill_parity(q, k, v, -math.inf, Br, 64, causal)
    print(f"d={d} Br={Br} causal={causal}: max err {r['max_err_out']:.2e} rel {r['rel_l2_out']:.2e}")
    assert r["skipped"] == 0


@pytest.mark.parametrize("d,Br", [(64, 64), (128, 128), (128, 64)])
def test_skip_small_gqa(d, Br):
    q, k, v = _inputs(201, 2, 2, 8, 2, 1000, d)
    B, Hq, L, _ = q.shape
    m = oracle.prefill(q, k, v, -math.inf, Br, 64, True, bits=True)["margin"]
    lam = oracle.lambda_for_ratio(m, 0.5)
    r = prefill_parity(q, k, v, lam, Br, 64, True)
    print(f"lam={lam:.4f} skipped {r['skipped']}/{r['visited']} exempt {r['exempt']} "
          f"err {r['max_err_out']:.2e}")
    # at this length more than half of the margins are positive (the running
    # max is still growing), so lambda clamps to 0 and fewer tiles skip than
    # asked for: about 20% with 64-row units, 6-7% with 128-row units
    assert r["skipped"] > 0.05 * r["visited"]


def test_config0_full():
    c = synth.CONFIGS[0]
    q, k, v = _inputs(0, 0, c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], c["frac"])
    r = prefill_parity(q, k, v, c["lam"], c["Br"], c["Bc"], c["causal"])
    print(f"config 0: skipped {r['skipped']}/{r['visited']} err {r['max_err_out']:.2e}")


def test_single_row_and_tiny():
    for L in (1, 2, 63, 65):
        q, k, v = _inputs(202, L, 1, 1, 1, L, 64)
        prefill_parity(q, k, v, -2.0, 64, 64, True)


def test_block_list_prefill_small():
    q, k, v = _inputs(203, 0, 1, 2, 2, 700, 64)
    nQ = math.ceil(700 / 64)
    rng = np.random.default_rng(0)
    idx = np.full((1, 2, nQ, 8), -1, np.int32)
    cnt = np.zeros((1, 2, nQ), np.int32)
    for h in range(2):
        for i in range(nQ):
            keep = sorted(set(rng.choice(i + 1, size=min(i + 1, 5), replace=False).tolist()) | {i})[:8]
            idx[0, h, i, :len(keep)] = keep
            cnt[0, h, i] = len(keep)
    # an invalid entry (above the causal limit) is ignored
    idx[0, 0, 0, 1] = 5
    cnt[0, 0, 0] = 2
    for lam in (-math.inf, -1.0):
        prefill_parity(q, k, v, lam, 64, 64, True, block_idx=idx, block_cnt=cnt)


def test_deterministic_repeat():
    import torch
    import sparse_attention_long_skip_amd as ssa
    from parity import dev_bf16
    q, k, v = _inputs(204, 0, 1, 4, 2, 777, 128)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    a = ssa.prefill(qd, kd, vd, -0.5, 128, 64, True, stats=True)
    b = ssa.prefill(qd, kd, vd, -0.5, 128, 64, True, stats=True)
    torch.cuda.synchronize()
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["tile_state"], b["tile_state"])


@pytest.mark.parametrize("d", [64, 128])
def test_wave_granular_votes(d):
    # Br = 32: every 32-row wave decides alone (oracle with 32-row units)
    q, k, v = _inputs(205, d, 2, 4, 2, 1000, d)
    m = oracle.prefill(q, k, v, -math.inf, 32, 64, True, bits=True)["margin"]
    for target in (0.3, 0.6):
        lam = oracle.lambda_for_ratio(m, target)
        r = prefill_parity(q, k, v, lam, 32, 64, True)
        print(f"d={d} lam={lam:.3f}: skipped {r['skipped']}/{r['visited']} exempt {r['exempt']}")
    r = prefill_parity(q, k, v, -math.inf, 32, 64, False)
    assert r["skipped"] == 0


@pytest.mark.parametrize("L", [1, 63, 64, 65, 127, 129, 191])
@pytest.mark.parametrize("d,Br", [(64, 64), (128, 128), (128, 64), (128, 32)])
def test_tile_edges(L, d, Br):
    # lengths at and around tile boundaries, GQA 4/2, a skipping lambda
    q, k, v = _inputs(202, L, 1, 4, 2, L, d)
    r = prefill_parity(q, k, v, -0.2, Br, 64, True)
    print(f"L={L} d={d} Br={Br}: skipped {r['skipped']}/{r['visited']} err {r['max_err_out']:.2e}")


@pytest.mark.parametrize("d,Br", [(64, 64), (128, 128), (128, 32)])
def test_growing_scores_rescale(d, Br):
    # keys scaled up along the sequence: every few tiles a row max exceeds
    # the exponentials' reference by more than 2^8, so O, the row sum and the
    # pending P are rescaled many times per row, with and without skipping
    q, k, v = _inputs(204, 5, 1, 2, 1, 900, d)
    ramp = (1.0 + np.arange(900, dtype=np.float32) / 20.0)[None, None, :, None]
    k = synth.bf16_bits(synth.bf16_to_f32(k) * ramp)
    for lam in (-math.inf, -1.0):
        r = prefill_parity(q, k, v, lam, Br, 64, True)
        print(f"d={d} Br={Br} lambda={lam}: skipped {r['skipped']}/{r['visited']}")


@pytest.mark.parametrize("d,Br", [(64, 64), (128, 128), (128, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_odd_batch_and_group(d, Br, causal):
    # B = 3, G = 3 (B * Hkv = 6 KV heads: the workgroups are dealt to the
    # XCDs in groups of G), a ragged length and a skipping lambda
    q, k, v = _inputs(206, d + causal, 3, 6, 2, 517, d)
    m = oracle.prefill(q, k, v, -math.inf, Br, 64, causal, bits=True)["margin"]
    lam = oracle.lambda_for_ratio(m, 0.4)
    r = prefill_parity(q, k, v, lam, Br, 64, causal)
    print(f"d={d} Br={Br} causal={causal} lam={lam:.3f}: skipped {r['skipped']}/{r['visited']}")


@pytest.mark.parametrize("d,Br", [(64, 64), (128, 64), (128, 128)])
def test_block_list_any_order(d, Br):
    # lists in shuffled and in descending order, with more than 64 entries
    # (the list is read 64 entries per load), invalid entries mixed in: the
    # visit order sets the running max and so the skip decisions
    L = 64 * 90
    q, k, v = _inputs(207, d, 1, 2, 1, L, d)
    nQ = L // Br
    rng = np.random.default_rng(1)
    mb = 96
    idx = np.full((1, 2, nQ, mb), -1, np.int32)
    cnt = np.zeros((1, 2, nQ), np.int32)
    for h in range(2):
        for i in range(nQ):
            tiles = list(range((i + 1) * Br // 64))
            if h == 0:
                rng.shuffle(tiles)
            else:
                tiles = tiles[::-1]
            if i % 7 == 3:
                tiles.insert(len(tiles) // 2, L // 64 + 5)   # out of range
                tiles.insert(1, (i + 1) * Br // 64)          # above the causal limit
            idx[0, h, i, :len(tiles)] = tiles[:mb]
            cnt[0, h, i] = min(len(tiles), mb)
    units = [(0, h, i) for h in range(2) for i in sorted({0, 3, 45, 70, 80, 89, nQ - 1} & set(range(nQ)))]
    m = oracle.prefill(q, k, v, -math.inf, Br, 64, True, bits=True, block_idx=idx, block_cnt=cnt,
                       units=units)["margin"]
    for lam in (-math.inf, oracle.lambda_for_ratio(m, 0.4)):
        r = prefill_parity(q, k, v, lam, Br, 64, True, block_idx=idx, block_cnt=cnt, units=units)
        print(f"d={d} lambda={lam:.3f}: skipped {r['skipped']}/{r['visited']}")
        if lam > -math.inf:
            assert r["skipped"] > 0


@pytest.mark.parametrize("d", [64, 128])
def test_block_lists_of_paired_units(d):
    """64-row units with block lists run two to a 128-row workgroup, their
    lists merged when both are ascending and visited one after the other
    otherwise: ascending pairs, pairs with one shuffled list, disjoint lists,
    entries valid for one unit of the pair only (causal), an empty list, and
    an odd number of units (the last workgroup holds one)."""
    L = 64 * 13 + 5
    q, k, v = _inputs(208, d, 1, 3, 1, L, d)
    nQ = math.ceil(L / 64)
    rng = np.random.default_rng(5)
    mb = 20
    idx = np.full((1, 3, nQ, mb), -1, np.int32)
    cnt = np.zeros((1, 3, nQ), np.int32)
    for h in range(3):
        for i in range(nQ):
            if h == 2 and i % 4 == 1:
                continue                                  # empty list
            pool = list(range(i + 1))
            if h == 1:
                pool = [j for j in pool if (j + i) % 2 == 0] or [i]   # neighbours share few tiles
            keep = sorted(rng.choice(pool, size=min(len(pool), int(rng.integers(1, 9))), replace=False).tolist())
            if i % 2 == 0 and i + 1 < nQ:
                keep.append(i + 1)                        # above this unit's causal limit: ignored
            if h == 0 and i % 6 == 3:
                rng.shuffle(keep)                         # one list of the pair not ascending
            idx[0, h, i, :len(keep)] = keep
            cnt[0, h, i] = len(keep)
    for lam in (-math.inf, -0.5):
        r = prefill_parity(q, k, v, lam, 64, 64, True, block_idx=idx, block_cnt=cnt)
        print(f"d={d} lambda={lam}: skipped {r['skipped']}/{r['visited']} exempt {r['exempt']}")


@pytest.mark.parametrize("d", [64, 128])
def test_block_list_with_repeated_entries(d):
    # a repeated entry is visited again (its keys count twice), in the
    # kernel as in the oracle; with Br = 64 such a list is not strictly
    # ascending, so the two lists of a workgroup are visited one after the
    # other. Skip counts count visits, so they are compared with the
    # oracle's directly (per-tile arrays keep the last visit).
    import torch
    import sparse_attention_long_skip_amd as ssa
    from parity import dev_bf16, to_np, assert_close, BAND
    L = 64 * 9
    q, k, v = _inputs(209, d, 1, 2, 1, L, d)
    nQ = L // 64
    idx = np.full((1, 2, nQ, 12), -1, np.int32)
    cnt = np.zeros((1, 2, nQ), np.int32)
    for h in range(2):
        for i in range(nQ):
            lst = [0, i, i // 2, i] if h == 0 else [i // 3, i // 3, i]
            idx[0, h, i, :len(lst)] = lst
            cnt[0, h, i] = len(lst)
    bi, bc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    for lam in (-math.inf, -1.0):
        ref = oracle.prefill(q, k, v, lam, 64, 64, True, block_idx=idx, block_cnt=cnt, bits=True)
        near = np.abs(ref["margin"] - lam) < BAND
        assert not near.any()
        for kw in (dict(stats=True), dict(counts=True)):
            g = ssa.prefill(qd, kd, vd, lam, Br=64, Bc=64, causal=True, block_idx=bi, block_cnt=bc, **kw)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(to_np(g["skip_counts"]), ref["skip_counts"])
            assert_close("out", to_np(g["out"]), ref["out"])
            assert_close("lse", to_np(g["lse"]), ref["lse"], rtol_l2=1.0)
