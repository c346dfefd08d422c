"""Pins for the prefill oracle: closed forms, brute force and invariants.

Each test ties ``oracle.prefill`` to something other than itself: the scalar
second implementation in ``oracle.bruteforce``, textbook softmax attention,
or a property that the Skip-Softmax rule (TRT-LLM page, three-step
algorithm; SpargeAttn page, stage two) fixes mathematically.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import bruteforce
from oracle.attention import KEPT, SKIPPED, NOT_VISITED


def _rand(rng, shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _case(seed, B=1, Hq=1, Hkv=1, L=None, d=None, spread=None):
    rng = np.random.default_rng(seed)
    L = L or int(rng.integers(1, 13))
    d = d or int(rng.integers(1, 5))
    spread = spread if spread is not None else float(rng.uniform(0.5, 4.0))
    q = _rand(rng, (B, Hq, L, d), spread)
    k = _rand(rng, (B, Hkv, L, d), spread)
    v = _rand(rng, (B, Hkv, L, d))
    return rng, q, k, v


@pytest.mark.parametrize("causal", [True, False])
def test_dense_equals_naive_softmax(causal):
    for seed in range(60):
        rng, q, k, v = _case(seed)
        Br = int(rng.choice([1, 2, 3, 4, 8]))
        Bc = int(rng.choice([1, 2, 3, 4, 8]))
        res = oracle.prefill(q, k, v, -np.inf, Br, Bc, causal)
        o_ref, lse_ref = bruteforce.naive_attention(q[0, 0], k[0, 0], v[0, 0], causal)
        np.testing.assert_allclose(res["out"][0, 0], np.array(o_ref), rtol=0, atol=1e-12)
        np.testing.assert_allclose(res["lse"][0, 0], np.array(lse_ref), rtol=0, atol=1e-12)
        assert not np.any(res["decision"] == SKIPPED)


def test_skip_rule_matches_bruteforce_1000_seeds():
    n_skips = 0
    for seed in range(1000):
        rng, q, k, v = _case(seed)
        Br = int(rng.choice([1, 2, 4, 8]))
        Bc = int(rng.choice([1, 2, 4, 8]))
        causal = bool(rng.integers(0, 2))
        lam = float(rng.uniform(-8.0, 0.0))
        res = oracle.prefill(q, k, v, lam, Br, Bc, causal)
        o_ref, lse_ref, skipped = bruteforce.skip_attention(q[0, 0], k[0, 0], v[0, 0], lam, Br, Bc, causal)
        got = {(int(i), int(j)) for i, j in zip(*np.nonzero(res["decision"][0, 0] == SKIPPED))}
        assert got == skipped, (seed, Br, Bc, causal, lam)
        n_skips += len(skipped)
        np.testing.assert_allclose(res["out"][0, 0], np.array(o_ref), atol=1e-12, rtol=0)
        lr = np.array(lse_ref)
        np.testing.assert_allclose(res["lse"][0, 0], lr, atol=1e-12, rtol=0)
        assert res["skip_counts"][0, 0].sum() == len(skipped)
    # the cases must actually exercise skipping
    assert n_skips > 500


def test_probabilities_sum_to_one_and_vanish_off_kept():
    for seed in range(40):
        rng, q, k, v = _case(seed, L=int(np.random.default_rng(seed).integers(2, 12)))
        Br, Bc = 2, 2
        lam = -1.0
        causal = bool(seed % 2)
        res = oracle.prefill(q, k, v, lam, Br, Bc, causal, return_probs=True)
        P = res["probs"][0, 0]
        L = P.shape[0]
        np.testing.assert_allclose(P.sum(axis=1), np.ones(L), atol=1e-13)
        assert np.all(P >= 0)
        for r in range(L):
            for c in range(L):
                i, j = r // Br, c // Bc
                allowed = (not causal) or c <= r
                kept = res["decision"][0, 0, i, j] == KEPT
                if not (allowed and kept):
                    assert P[r, c] == 0.0


def test_dominant_key_reproduces_its_value_row():
    rng = np.random.default_rng(7)
    L, d = 16, 8
    q = rng.standard_normal((1, 1, L, d)) * 0.1
    k = rng.standard_normal((1, 1, L, d)) * 0.1
    v = rng.standard_normal((1, 1, L, d))
    # key 3 aligned with every query so that its score beats all others by > 50
    direction = np.ones(d) / math.sqrt(d)
    q[0, 0] += 20 * direction
    k[0, 0, 3] = 20 * direction * 2
    s = q[0, 0] @ k[0, 0].T / math.sqrt(d)
    for r in range(3, L):
        others = np.delete(s[r, :r + 1], 3)
        assert s[r, 3] - others.max() > 50
    for lam in (-np.inf, -6.0, -0.5):
        res = oracle.prefill(q, k, v, lam, 4, 4, True)
        for r in range(3, L):
            np.testing.assert_allclose(res["out"][0, 0, r], v[0, 0, 3], atol=20 * math.exp(-50))


def test_uniform_values_give_that_value():
    rng = np.random.default_rng(3)
    for seed in range(20):
        _, q, k, v = _case(seed, L=10, d=3)
        w = rng.standard_normal(3)
        v[:] = w
        for lam in (-np.inf, -2.0, -0.1, 0.0):
            res = oracle.prefill(q, k, v, lam, 2, 3, bool(seed % 2))
            np.testing.assert_allclose(res["out"][0, 0], np.broadcast_to(w, (10, 3)), atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_heads():
    for seed in range(10):
        rng, q, k, v = _case(seed, B=2, Hq=6, Hkv=2, L=11, d=4)
        G = 3
        krep = np.repeat(k, G, axis=1)
        vrep = np.repeat(v, G, axis=1)
        for lam in (-np.inf, -1.5):
            a = oracle.prefill(q, k, v, lam, 4, 2, True)
            b = oracle.prefill(q, krep, vrep, lam, 4, 2, True)
            np.testing.assert_array_equal(a["out"], b["out"])
            np.testing.assert_array_equal(a["decision"], b["decision"])
        # head hq must read KV head hq // G (not hq % Hkv): heads 1 and 3 differ
        one = oracle.prefill(q[:, 1:2], k[:, 0:1], v[:, 0:1], -np.inf, 4, 2, True)
        a = oracle.prefill(q, k, v, -np.inf, 4, 2, True)
        np.testing.assert_array_equal(a["out"][:, 1:2], one["out"])


def test_monotone_nested_in_lambda():
    for seed in range(50):
        rng, q, k, v = _case(seed, L=12)
        lams = np.sort(rng.uniform(-6, 0, size=4))
        prev = None
        for lam in lams:
            dec = oracle.prefill(q, k, v, lam, 2, 2, True)["decision"] == SKIPPED
            if prev is not None:
                assert np.all(prev <= dec)  # skip(l1) subset of skip(l2) for l1 <= l2
            prev = dec


def test_margins_do_not_depend_on_lambda_and_decide_skips():
    for seed in range(30):
        rng, q, k, v = _case(seed, L=12)
        a = oracle.prefill(q, k, v, -np.inf, 3, 2, True)
        lam = float(rng.uniform(-5, 0))
        b = oracle.prefill(q, k, v, lam, 3, 2, True)
        np.testing.assert_array_equal(a["margin"], b["margin"])
        vis = ~np.isnan(b["margin"])
        np.testing.assert_array_equal((b["decision"] == SKIPPED)[vis], (b["margin"] < lam)[vis])
        np.testing.assert_array_equal(b["decision"] == NOT_VISITED, ~vis)


def test_first_tile_and_argmax_tile_never_skipped():
    for seed in range(200):
        rng, q, k, v = _case(seed, L=int(np.random.default_rng(seed).integers(4, 13)))
        Br, Bc = 2, 2
        causal = bool(seed % 2)
        res = oracle.prefill(q, k, v, float(rng.uniform(-8, 0)), Br, Bc, causal)
        dec = res["decision"][0, 0]
        L = q.shape[2]
        s = q[0, 0] @ k[0, 0].T / math.sqrt(q.shape[3])
        for i in range(dec.shape[0]):
            vis = np.nonzero(dec[i] != NOT_VISITED)[0]
            assert dec[i, vis[0]] == KEPT
        for r in range(L):
            row = s[r, :r + 1] if causal else s[r]
            c = int(np.argmax(row))
            assert dec[r // Br, c // Bc] == KEPT


def test_error_bound_against_dense():
    """|o_skip - o_dense| <= 2 max|v| W_B / (W_A + W_B), weights exp(s - m_r):
    W_A >= 1 since the row max is kept, and every skipped score is below
    m_r + lambda, so W_B <= n_skipped * exp(lambda)."""
    for seed in range(100):
        rng, q, k, v = _case(seed, L=12, d=3)
        lam = float(rng.uniform(-6, -0.5))
        causal = True
        sk = oracle.prefill(q, k, v, lam, 2, 2, causal)
        dn = oracle.prefill(q, k, v, -np.inf, 2, 2, causal)
        dec = sk["decision"][0, 0]
        vmax = np.abs(v).max()
        for r in range(12):
            n_sk = sum(1 for c in range(r + 1) if dec[r // 2, c // 2] == SKIPPED)
            wb = n_sk * math.exp(lam)
            bound = 2 * vmax * wb / (1 + wb)
            err = np.abs(sk["out"][0, 0, r] - dn["out"][0, 0, r]).max()
            assert err <= bound + 1e-12


def test_full_block_list_equals_dense():
    for seed in range(20):
        rng, q, k, v = _case(seed, B=1, Hq=2, Hkv=2, L=13, d=4)
        Br = Bc = 3
        nQ = nK = 5
        idx = np.tile(np.arange(nK), (1, 2, nQ, 1))
        cnt = np.full((1, 2, nQ), nK)
        for lam in (-np.inf, -1.0):
            a = oracle.prefill(q, k, v, lam, Br, Bc, True)
            b = oracle.prefill(q, k, v, lam, Br, Bc, True, block_idx=idx, block_cnt=cnt)
            np.testing.assert_array_equal(a["out"], b["out"])
            np.testing.assert_array_equal(a["decision"], b["decision"])


def test_block_list_restricts_keys_to_kept_blocks():
    """lambda = -inf with a block list equals softmax over the allowed keys of
    the listed blocks (written out with scalar loops)."""
    for seed in range(30):
        rng, q, k, v = _case(seed, L=12, d=3)
        Br = Bc = 3
        nQ = 4
        idx = np.full((1, 1, nQ, 4), -1)
        cnt = np.zeros((1, 1, nQ), int)
        for i in range(nQ):
            cand = [j for j in range(i + 1)]
            keep = sorted(set(rng.choice(cand, size=int(rng.integers(1, len(cand) + 1)), replace=False)) | {i})
            idx[0, 0, i, :len(keep)] = keep
            cnt[0, 0, i] = len(keep)
        res = oracle.prefill(q, k, v, -np.inf, Br, Bc, True, block_idx=idx, block_cnt=cnt)
        for r in range(12):
            i = r // Br
            keep = set(idx[0, 0, i, :cnt[0, 0, i]].tolist())
            cols = [c for c in range(r + 1) if c // Bc in keep]
            s = [sum(q[0, 0, r, t] * k[0, 0, c, t] for t in range(3)) / math.sqrt(3) for c in cols]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            o = [sum(w[a] * v[0, 0, c, e] for a, c in enumerate(cols)) / sum(w) for e in range(3)]
            np.testing.assert_allclose(res["out"][0, 0, r], o, atol=1e-12)


def test_ragged_last_tiles_and_single_row():
    rng, q, k, v = _case(5, L=1, d=2)
    res = oracle.prefill(q, k, v, -3.0, 4, 4, True)
    np.testing.assert_allclose(res["out"][0, 0, 0], v[0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(res["lse"][0, 0, 0], q[0, 0, 0] @ k[0, 0, 0] / math.sqrt(2), atol=1e-15)


def test_bf16_bit_inputs_widen_exactly():
    from synth import bf16_bits, bf16_to_f32
    rng = np.random.default_rng(11)
    x = [rng.standard_normal((1, 1, 9, 4)).astype(np.float32) for _ in range(3)]
    bits = [bf16_bits(a) for a in x]
    vals = [bf16_to_f32(b).astype(np.float64) for b in bits]
    a = oracle.prefill(*bits, -1.0, 2, 2, True, bits=True)
    b = oracle.prefill(*vals, -1.0, 2, 2, True)
    np.testing.assert_array_equal(a["out"], b["out"])


def test_strict_comparison_keeps_exact_ties_at_zero():
    """Tile 1 repeats tile 0's keys, so every row's gap is exactly 0; with
    lambda = 0 the strict rule keeps it (0 < 0 is false)."""
    rng = np.random.default_rng(2)
    d = 4
    kt = rng.standard_normal((2, d))
    k = np.concatenate([kt, kt])[None, None]
    q = rng.standard_normal((1, 1, 4, d))
    v = rng.standard_normal((1, 1, 4, d))
    res = oracle.prefill(q, k, v, 0.0, 4, 2, False)
    assert res["margin"][0, 0, 0, 1] == 0.0
    assert res["decision"][0, 0, 0, 1] == KEPT
    res = oracle.prefill(q, k, v, 1e-300, 4, 2, False)
    assert res["decision"][0, 0, 0, 1] == SKIPPED


def test_nm_sparse_softmax_matches_bruteforce():
    for seed in range(60):
        rng, q, k, v = _case(seed, L=int(np.random.default_rng(seed).integers(2, 14)))
        m = int(rng.choice([2, 4]))
        n = int(rng.integers(1, m))
        causal = bool(seed % 2)
        sink = int(rng.integers(0, 3))
        recent = int(rng.integers(0, 4))
        res = oracle.prefill(q, k, v, -np.inf, 4, 4, causal, nm=(n, m), dense_sink=sink, dense_recent=recent)
        o_ref, lse_ref = bruteforce.nm_attention(q[0, 0], k[0, 0], v[0, 0], n, m, causal, sink, recent)
        np.testing.assert_allclose(res["out"][0, 0], np.array(o_ref), atol=1e-12)
        np.testing.assert_allclose(res["lse"][0, 0], np.array(lse_ref), atol=1e-12)


def test_nm_keeps_at_most_n_per_group_and_n_equal_m_is_dense():
    rng, q, k, v = _case(3, L=16, d=4)
    res = oracle.prefill(q, k, v, -np.inf, 4, 8, False, nm=(2, 4), return_probs=True)
    P = res["probs"][0, 0]
    for r in range(16):
        for g0 in range(0, 16, 4):
            assert np.count_nonzero(P[r, g0:g0 + 4]) == 2
    a = oracle.prefill(q, k, v, -1.0, 4, 8, True, nm=(4, 4))
    b = oracle.prefill(q, k, v, -1.0, 4, 8, True)
    np.testing.assert_array_equal(a["out"], b["out"])
    # exemptions covering every key give dense attention
    c = oracle.prefill(q, k, v, -np.inf, 4, 8, True, nm=(1, 4), dense_recent=16)
    d = oracle.prefill(q, k, v, -np.inf, 4, 8, True)
    np.testing.assert_allclose(c["out"], d["out"], atol=1e-14)
