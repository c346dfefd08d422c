"""Pins for the decode, combine, block-mask and calibration oracles."""

import math

import numpy as np
import pytest

import oracle
from oracle import bruteforce
from oracle.attention import KEPT, SKIPPED


def _decode_case(seed, B=2, Hq=4, Hkv=2, S_max=40, d=4, spread=None):
    rng = np.random.default_rng(seed)
    spread = spread if spread is not None else float(rng.uniform(0.5, 4.0))
    q = rng.standard_normal((B, Hq, d)) * spread
    kc = rng.standard_normal((B, Hkv, S_max, d)) * spread
    vc = rng.standard_normal((B, Hkv, S_max, d))
    lens = rng.integers(1, S_max + 1, size=B)
    return rng, q, kc, vc, lens


def test_decode_dense_equals_naive_softmax():
    for seed in range(40):
        rng, q, kc, vc, lens = _decode_case(seed)
        Bc = int(rng.choice([1, 3, 4, 8]))
        T = int(rng.choice([1, 2, 3, 100]))
        res = oracle.decode(q, kc, vc, lens, -np.inf, Bc, T)
        G = 2
        for b in range(2):
            n = lens[b]
            for h in range(4):
                kvh = h // G
                o, lse = bruteforce.naive_attention([q[b, h]], kc[b, kvh, :n], vc[b, kvh, :n], False)
                np.testing.assert_allclose(res["out"][b, h], o[0], atol=1e-12)
                np.testing.assert_allclose(res["lse"][b, h], lse[0], atol=1e-12)


def test_split_layout_does_not_change_dense_result():
    for seed in range(20):
        rng, q, kc, vc, lens = _decode_case(seed, S_max=64)
        ref = oracle.decode(q, kc, vc, lens, -np.inf, 4, 10 ** 6)
        for T in (1, 2, 5, 7):
            r = oracle.decode(q, kc, vc, lens, -np.inf, 4, T)
            np.testing.assert_allclose(r["out"], ref["out"], atol=1e-13)
            np.testing.assert_allclose(r["lse"], ref["lse"], atol=1e-13)


def test_decode_skip_set_matches_bruteforce():
    total = 0
    for seed in range(300):
        rng, q, kc, vc, lens = _decode_case(seed, B=1, Hq=(1, 2, 4)[seed % 3], Hkv=1, S_max=48, d=3)
        Bc = int(rng.choice([2, 4, 8]))
        T = int(rng.choice([1, 2, 3, 6]))
        lam = float(rng.uniform(-6, 0))
        res = oracle.decode(q, kc, vc, lens, lam, Bc, T)
        ref = bruteforce.decode_skip_set(q[0], kc[0, 0], int(lens[0]), lam, Bc, T)
        got = set(np.nonzero(res["decision"][0, 0] == SKIPPED)[0].tolist())
        assert got == ref
        total += len(ref)
        # first tile of each split is never skipped
        ntiles = math.ceil(lens[0] / Bc)
        for sp in range(math.ceil(ntiles / T)):
            assert res["decision"][0, 0, sp * T] == KEPT
        assert res["skip_counts"][0, 0].sum() == len(ref)
    assert total > 150


def test_decode_skipped_output_is_softmax_over_kept_tiles():
    for seed in range(30):
        rng, q, kc, vc, lens = _decode_case(seed, B=1, Hq=2, Hkv=1, S_max=30, d=3)
        lam = float(rng.uniform(-4, 0))
        Bc, T = 3, 4
        res = oracle.decode(q, kc, vc, lens, lam, Bc, T)
        n = int(lens[0])
        dec = res["decision"][0, 0]
        cols = [c for c in range(n) if dec[c // Bc] == KEPT]
        for h in range(2):
            o, lse = bruteforce.naive_attention([q[0, h]], kc[0, 0, cols], vc[0, 0, cols], False)
            np.testing.assert_allclose(res["out"][0, h], o[0], atol=1e-12)
            np.testing.assert_allclose(res["lse"][0, h], lse[0], atol=1e-12)


def test_decode_empty_and_overlong_lengths():
    rng, q, kc, vc, _ = _decode_case(1, B=3, S_max=16)
    lens = np.array([0, 16, 99])
    q[2], kc[2], vc[2] = q[1], kc[1], vc[1]
    res = oracle.decode(q, kc, vc, lens, -1.0, 4, 2)
    assert np.all(res["out"][0] == 0) and np.all(res["lse"][0] == -np.inf)
    np.testing.assert_array_equal(res["out"][1], res["out"][2])  # clamped to S_max


def test_lse_combine_identity():
    """Splitting one softmax sum into parts and combining recovers it."""
    rng = np.random.default_rng(0)
    for _ in range(50):
        n, d = int(rng.integers(2, 30)), 3
        s = rng.standard_normal(n) * 5
        v = rng.standard_normal((n, d))
        cuts = np.sort(rng.choice(np.arange(1, n), size=int(rng.integers(0, min(4, n - 1)) + 1), replace=False))
        parts = np.split(np.arange(n), cuts)
        m = [s[p].max() for p in parts]
        l = [np.exp(s[p] - s[p].max()).sum() for p in parts]
        o = [np.exp(s[p] - s[p].max()) @ v[p] for p in parts]
        # an empty part must be ignored
        m.append(-np.inf)
        l.append(0.0)
        o.append(np.zeros(d))
        out, lse = oracle.lse_combine_parts(np.array(m), np.array(l), np.array(o))
        w = np.exp(s - s.max())
        np.testing.assert_allclose(out, w @ v / w.sum(), atol=1e-13)
        np.testing.assert_allclose(lse, s.max() + np.log(w.sum()), atol=1e-13)


def test_pooling_commutes_with_scores():
    """q_bar . k_bar equals the mean of the token scores of the block pair."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 2, 37, 5))
    k = rng.standard_normal((1, 2, 37, 5))
    pool = 8
    sc = oracle.block_scores(q, k, pool)
    S = q @ np.swapaxes(k, -1, -2) / math.sqrt(5)
    nb = 5
    for b in range(nb):
        for c in range(b + 1):
            blk = S[:, :, b * pool:min(37, (b + 1) * pool), c * pool:min(37, (c + 1) * pool)]
            np.testing.assert_allclose(sc[:, :, b, c], blk.mean(axis=(-1, -2)), atol=1e-13)
            assert np.all(np.isneginf(sc[:, :, b, b + 1:]))


def test_block_mask_matches_bruteforce_and_structure():
    for seed in range(40):
        rng = np.random.default_rng(seed)
        L = int(rng.integers(1, 70))
        d = int(rng.integers(1, 5))
        pool = int(rng.choice([2, 4, 8]))
        topk = int(rng.integers(0, 6))
        sink = int(rng.integers(0, 3))
        win = int(rng.integers(0, 20))
        q = rng.standard_normal((1, 1, L, d))
        k = rng.standard_normal((1, 1, L, d))
        res = oracle.block_mask(q, k, pool, topk, sink, win)
        ref = bruteforce.topk_blocks(q[0, 0], k[0, 0], pool, topk, sink, win)
        W = math.ceil(win / pool) if win > 0 else 0
        for b, kept in enumerate(ref):
            cnt = res["block_cnt"][0, 0, b]
            got = res["block_idx"][0, 0, b, :cnt].tolist()
            assert got == kept
            assert all(x == -1 for x in res["block_idx"][0, 0, b, cnt:])
            assert got == sorted(set(got))
            assert set(range(min(sink, b + 1))) <= set(got)
            assert set(range(max(0, b - W + 1), b + 1)) <= set(got)
            assert len(got) <= topk + sink + W
            if b + 1 <= topk:
                assert got == list(range(b + 1))


def test_block_mask_tie_break_prefers_lower_index():
    # identical keys in every block -> all scores tie; topk=2 keeps blocks 0, 1
    q = np.ones((1, 1, 16, 2))
    k = np.ones((1, 1, 16, 2))
    res = oracle.block_mask(q, k, 4, 2, 0, 0)
    for b in range(4):
        assert res["block_idx"][0, 0, b, :res["block_cnt"][0, 0, b]].tolist() == list(range(min(2, b + 1)))


def test_calibrated_lambda_hits_target_ratio():
    rng = np.random.default_rng(4)
    g = rng.standard_normal(20000) * 0.5
    g[:100] = np.inf
    g[100:150] = np.nan
    for target in (0.1, 0.5, 0.7):
        lam = oracle.lambda_for_ratio(g, target)
        assert lam <= 0
        r = oracle.skip_ratio(g, lam)
        if np.quantile(g[np.isfinite(g)], target) < 0:
            assert abs(r - target) <= 0.011
    # a target needing a positive lambda is clamped to 0
    assert oracle.lambda_for_ratio(np.abs(g[150:]), 0.5) == 0.0


def test_calibration_on_oracle_margins_reproduces_ratio():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 2, 64, 4)) * 2
    k = rng.standard_normal((1, 2, 64, 4)) * 2
    v = rng.standard_normal((1, 2, 64, 4))
    m = oracle.prefill(q, k, v, -np.inf, 4, 4, True)["margin"]
    lam = oracle.lambda_for_ratio(m, 0.3)
    res = oracle.prefill(q, k, v, lam, 4, 4, True)
    vis = ~np.isnan(res["margin"])
    got = (res["decision"] == SKIPPED)[vis].mean()
    assert abs(got - oracle.skip_ratio(m, lam)) < 1e-12
    assert abs(got - 0.3) < 0.03


def test_self_similarity_closed_forms():
    # identical rows -> 1; mutually orthogonal rows -> 1/n (self pairs only)
    x = np.zeros((1, 1, 8, 8))
    x[0, 0, :4] = [1, 2, 0, 0, 0, 0, 0, 0]
    for i in range(4):
        x[0, 0, 4 + i, i] = 3.0
    s = oracle.block_self_similarity(x, 4)
    np.testing.assert_allclose(s[0, 0], [1.0, 0.25], atol=1e-15)


def test_sparge_mask_matches_bruteforce():
    for seed in range(30):
        rng = np.random.default_rng(seed)
        L = int(rng.integers(4, 40))
        d = int(rng.integers(2, 5))
        pool = int(rng.choice([2, 4]))
        q = rng.standard_normal((1, 1, L, d)) + rng.uniform(0, 2) * np.ones(d)
        k = rng.standard_normal((1, 1, L, d)) + rng.uniform(0, 2) * np.ones(d)
        theta = float(rng.uniform(0.1, 0.9))
        tau = float(rng.uniform(0.3, 0.99))
        mode = ("mass", "count")[seed % 2]
        res = oracle.sparge_mask(q, k, pool, theta, tau, mode)
        ref = bruteforce.sparge_blocks(q[0, 0], k[0, 0], pool, theta, tau, mode)
        for b, kept in enumerate(ref):
            got = res["block_idx"][0, 0, b, :res["block_cnt"][0, 0, b]].tolist()
            assert got == kept, (seed, b)


def test_sparge_mask_limits():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, 64, 8)) + 2.0
    k = rng.standard_normal((1, 2, 64, 8)) + 2.0
    # theta above every similarity: nothing is compressed -> dense
    d = oracle.sparge_mask(q, k, 8, 1.5, 0.5)
    assert np.array_equal(d["block_cnt"][0, 0], np.arange(1, 9))
    assert np.all(d["phat"] == 0)
    # everything compressed, tau tiny: exactly the argmax block per row
    for mode in ("mass", "count"):
        t = oracle.sparge_mask(q, k, 8, -1.0, 1e-9, mode)
        assert np.all(t["block_cnt"] == 1)
        np.testing.assert_array_equal(t["block_idx"][..., 0], t["phat"].argmax(axis=-1))
        np.testing.assert_allclose(t["phat"].sum(axis=-1), 1.0, rtol=1e-12)
    # count mode with tau = 1 keeps every block
    f = oracle.sparge_mask(q, k, 8, -1.0, 1.0, "count")
    assert np.array_equal(f["block_cnt"][0, 1], np.arange(1, 9))
    # mass mode: the kept mass reaches tau and the set is the smallest such
    r = oracle.sparge_mask(q, k, 8, -1.0, 0.8)
    for h in range(2):
        for b in range(8):
            kept = r["block_idx"][0, h, b, :r["block_cnt"][0, h, b]]
            p = r["phat"][0, h, b]
            assert p[kept].sum() >= 0.8 - 1e-12
            assert r["mass_before"][0, h, b] < 0.8 <= r["mass_at"][0, h, b]
            drop = np.setdiff1d(np.arange(b + 1), kept)
            if len(drop):
                assert p[kept].min() >= p[drop].max()


def test_sparge_mask_uncompressed_key_blocks_always_kept():
    # keys: block 1 is pure noise in alternating directions (similarity 0),
    # blocks 0, 2, 3 are constant rows (similarity 1)
    d, pool = 4, 4
    k = np.zeros((1, 1, 16, d))
    k[0, 0, 0:4] = [1, 0, 0, 0]
    k[0, 0, 4:8] = [[1, 0, 0, 0], [-1, 0, 0, 0], [0, 1, 0, 0], [0, -1, 0, 0]]
    k[0, 0, 8:12] = [0, 0, 1, 0]
    k[0, 0, 12:16] = [0, 0, 0, 1]
    q = np.tile(np.array([0, 0, 0, 5.0]), (1, 1, 16, 1))
    r = oracle.sparge_mask(q, k, pool, 0.5, 1e-6)
    np.testing.assert_allclose(r["sim_k"][0, 0], [1, 0, 1, 1], atol=1e-15)
    # row 3: block 3 (aligned with q) is the top; block 1 is uncompressed
    assert r["block_idx"][0, 0, 3, :r["block_cnt"][0, 0, 3]].tolist() == [1, 3]
    assert r["phat"][0, 0, 3, 1] == 0
    # row 1: compressed candidates {0}; block 1 always kept
    assert r["block_idx"][0, 0, 1, :r["block_cnt"][0, 0, 1]].tolist() == [0, 1]


def test_compressed_keys_closed_forms():
    # keys 0..L-1 along one axis: window m averages m*stride .. m*stride+kernel-1
    L = 50
    k = np.arange(L, dtype=np.float64).reshape(1, 1, L, 1)
    kt = oracle.compress_keys(k, 32, 16)
    assert kt.shape[-2] == 4
    np.testing.assert_allclose(kt[0, 0, :, 0], [15.5, 31.5, (32 + 49) / 2, (48 + 49) / 2])
    # kernel = stride = pool reduces to the plain pooled scores
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 3, 300, 8))
    kk = rng.standard_normal((2, 3, 300, 8))
    np.testing.assert_allclose(oracle.block_scores_compressed(q, kk, 64, 64, 64),
                               oracle.block_scores(q, kk, 64), rtol=1e-12, atol=1e-12)


def test_compressed_block_mask_matches_bruteforce():
    for seed in range(12):
        rng = np.random.default_rng(100 + seed)
        L = int(rng.integers(10, 90))
        d = int(rng.integers(2, 5))
        pool, kernel, stride = [(8, 8, 4), (8, 4, 2), (4, 4, 2), (8, 16, 4)][seed % 4]
        topk, sink, win = int(rng.integers(0, 5)), int(rng.integers(0, 2)), int(rng.integers(0, 20))
        q = rng.standard_normal((1, 1, L, d))
        k = rng.standard_normal((1, 1, L, d))
        sc = oracle.block_scores_compressed(q, k, pool, kernel, stride)
        got = oracle.block_mask(q, k, pool, topk, sink, win, scores=sc)
        ref = bruteforce.topk_blocks(q[0, 0], k[0, 0], pool, topk, sink, win, kernel, stride)
        for b, kept in enumerate(ref):
            assert got["block_idx"][0, 0, b, :got["block_cnt"][0, 0, b]].tolist() == kept, (seed, b)


def test_compressed_scores_see_a_spike_the_block_mean_dilutes():
    # one key block holds a short run of keys aligned with the query: the
    # 32-token windows see it at full strength, the 64-token mean at half
    d, L = 4, 256
    q = np.zeros((1, 1, L, d))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, L, d))
    k[0, 0, 64 + 16:64 + 48, 0] = 2.0   # 32 keys in block 1, exactly window m = 5
    k[0, 0, 128:192, 0] = 1.2           # block 2: a weaker but uniform run
    plain = oracle.block_scores(q, k, 64)
    comp = oracle.block_scores_compressed(q, k, 64, 32, 16)
    assert plain[0, 0, 3, 1] < plain[0, 0, 3, 2]
    assert comp[0, 0, 3, 1] > comp[0, 0, 3, 2]
    np.testing.assert_allclose(comp[0, 0, 3, 1], 2.0 / 2.0, rtol=1e-12)   # 2.0 / sqrt(4)
