"""Pins of the vertical-slash oracle: brute force on tiny inputs, closed
forms and invariants."""

import math

import numpy as np

import oracle
from oracle import bruteforce


def test_matches_bruteforce():
    for seed in range(24):
        rng = np.random.default_rng(700 + seed)
        L = int(rng.integers(3, 45))
        d = int(rng.integers(2, 5))
        pool = int(rng.choice([2, 4, 8]))
        last_q = int(rng.integers(1, L + 1))
        nv, ns = int(rng.integers(0, L + 2)), int(rng.integers(0, L + 2))
        q = rng.standard_normal((1, 1, L, d)) * 1.5
        k = rng.standard_normal((1, 1, L, d)) * 1.5
        r = oracle.vertical_slash_mask(q, k, last_q, nv, ns, pool)
        tiles, vs, ss, v, s = bruteforce.vertical_slash(q[0, 0], k[0, 0], last_q, nv, ns, pool)
        np.testing.assert_allclose(r["v"][0, 0], v, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r["s"][0, 0], s, rtol=1e-12, atol=1e-14)
        assert r["vertical"][(0, 0)].tolist() == vs
        assert r["slash"][(0, 0)].tolist() == ss
        for b, kept in enumerate(tiles):
            assert r["block_idx"][0, 0, b, :r["block_cnt"][0, 0, b]].tolist() == kept, (seed, b)


def test_score_mass_identities():
    # every row's attention sums to one, so both score vectors sum to last_q;
    # with a single query, s is v reversed (offset o = L - 1 - j)
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 3, 70, 8))
    k = rng.standard_normal((2, 3, 70, 8))
    v, s = oracle.vertical_slash_scores(q, k, 5)
    np.testing.assert_allclose(v.sum(-1), 5.0, rtol=1e-12)
    np.testing.assert_allclose(s.sum(-1), 5.0, rtol=1e-12)
    v1, s1 = oracle.vertical_slash_scores(q, k, 1)
    np.testing.assert_allclose(s1, v1[..., ::-1], rtol=1e-12, atol=1e-15)


def test_uniform_attention_closed_form():
    # zero queries: row p attends uniformly to its p + 1 keys
    L, R = 20, 4
    q = np.zeros((1, 1, L, 3))
    k = np.random.default_rng(2).standard_normal((1, 1, L, 3))
    v, s = oracle.vertical_slash_scores(q, k, R)
    rows = range(L - R, L)
    want_v = [sum(1.0 / (p + 1) for p in rows if j <= p) for j in range(L)]
    want_s = [sum(1.0 / (p + 1) for p in rows if o <= p) for o in range(L)]
    np.testing.assert_allclose(v[0, 0], want_v, rtol=1e-12)
    np.testing.assert_allclose(s[0, 0], want_s, rtol=1e-12)


def test_cover_special_cases():
    L, pool = 256, 64
    # only the main diagonal: exactly the diagonal tiles
    lists = oracle.cover_blocks([], [0], L, pool)
    assert lists == [[b] for b in range(4)]
    # one vertical line at key 70 (tile 1): every query tile from 1 on
    lists = oracle.cover_blocks([70], [], L, pool)
    assert lists == [[], [1], [1], [1]]
    # offset 64: row 64b + x meets key 64(b-1) + x, so only tile (b, b-1)
    lists = oracle.cover_blocks([], [64], L, pool)
    assert lists == [[], [0], [1], [2]]
    # offset 1: the diagonal tile and, from the second tile on, the tile to its left
    lists = oracle.cover_blocks([], [1], L, pool)
    assert lists == [[0], [0, 1], [1, 2], [2, 3]]
    # everything chosen: dense causal lists
    lists = oracle.cover_blocks(range(L), range(L), L, pool)
    assert lists == [list(range(b + 1)) for b in range(4)]


def test_topk_ties_and_counts():
    x = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    assert oracle.vertical_slash.top_indices(x, 2).tolist() == [1, 2]
    assert oracle.vertical_slash.top_indices(x, 0).tolist() == []
    assert oracle.vertical_slash.top_indices(x, 9).tolist() == [0, 1, 2, 3, 4]


def test_planted_vertical_is_found():
    # a key aligned with every query takes nearly all the attention mass
    rng = np.random.default_rng(4)
    L, d = 128, 16
    q = rng.standard_normal((1, 1, L, d)) * 0.1
    k = rng.standard_normal((1, 1, L, d)) * 0.1
    q[..., 0] += 6.0
    k[0, 0, 17, 0] += 6.0   # logit 36 / sqrt(16) = 9 against ~0 for the rest
    r = oracle.vertical_slash_mask(q, k, 8, 1, 1, 32)
    assert r["vertical"][(0, 0)].tolist() == [17]
    assert r["v"][0, 0, 17] > 0.9 * 8
    assert math.isfinite(r["v_kth"][0, 0])
