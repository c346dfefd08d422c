"""Pins for the oracle's forced-decision mode (``oracle.replay`` and the
``forced=`` argument of ``oracle.prefill`` / ``oracle.decode``).

The GPU parity harness scores a decision unit whose GPU decisions differ
from the oracle's inside the 1e-3 band against the oracle's outputs for the
GPU's own decisions. These tests fix what that mode means, independently of
the rule's arithmetic (TRT-LLM page, three-step algorithm: a skipped tile
adds no exponentials, no row sum and no P.V; so the output is softmax
attention over the keys of the kept tiles only):

* replaying the rule's own decisions reproduces the rule's result exactly;
* forcing every visited tile kept gives dense attention;
* a random forced mask gives textbook softmax attention (the scalar
  ``bruteforce.naive_attention``) over exactly the keys of the tiles the
  mask keeps in that unit -- different masks per batch, head, query tile and
  split, so a flipped flag or a mask read at the wrong unit fails.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import bruteforce
from oracle.attention import KEPT, SKIPPED, NOT_VISITED


def _prefill_case(seed, B=2, Hq=4, Hkv=2, L=None, d=3):
    rng = np.random.default_rng(seed)
    L = L or int(rng.integers(5, 23))
    spread = float(rng.uniform(0.5, 3.0))
    q = rng.standard_normal((B, Hq, L, d)) * spread
    k = rng.standard_normal((B, Hkv, L, d)) * spread
    v = rng.standard_normal((B, Hkv, L, d))
    return rng, q, k, v


def _forced_random(rng, decision, p_skip):
    """Random KEPT/SKIPPED over the visited tiles of ``decision``."""
    f = np.where(rng.random(decision.shape) < p_skip, SKIPPED, KEPT).astype(np.int8)
    f[decision == NOT_VISITED] = NOT_VISITED
    return f


def _kept_columns(forced_row, Bc, r, L, causal, tiles):
    cols = []
    for j in tiles:
        if forced_row[j] != KEPT:
            continue
        for c in range(j * Bc, min(L, (j + 1) * Bc)):
            if not causal or c <= r:
                cols.append(c)
    return cols


@pytest.mark.parametrize("causal", [True, False])
def test_replay_of_own_decisions_is_bit_identical(causal):
    for seed in range(40):
        rng, q, k, v = _prefill_case(seed)
        Br = int(rng.choice([1, 2, 3, 4]))
        Bc = int(rng.choice([1, 2, 3, 4]))
        lam = float(rng.uniform(-3.0, 0.0))
        ref = oracle.prefill(q, k, v, lam, Br, Bc, causal)
        rep = oracle.replay(q, k, v, ref["decision"], Br, Bc, causal)
        for key in ("out", "lse", "decision", "skip_counts"):
            np.testing.assert_array_equal(rep[key], ref[key], err_msg=f"{key} seed {seed}")
        # margins are the rule's own quantity and do not depend on the decisions
        np.testing.assert_array_equal(np.isnan(rep["margin"]), np.isnan(ref["margin"]))
        ok = ~np.isnan(ref["margin"])
        np.testing.assert_array_equal(rep["margin"][ok], ref["margin"][ok])


def test_replay_all_kept_equals_dense():
    for seed in range(30):
        rng, q, k, v = _prefill_case(100 + seed)
        Br, Bc = int(rng.choice([1, 2, 4])), int(rng.choice([1, 3, 4]))
        causal = bool(seed % 2)
        dense = oracle.prefill(q, k, v, -np.inf, Br, Bc, causal)
        forced = np.where(dense["decision"] != NOT_VISITED, KEPT, NOT_VISITED).astype(np.int8)
        rep = oracle.replay(q, k, v, forced, Br, Bc, causal)
        np.testing.assert_array_equal(rep["out"], dense["out"])
        np.testing.assert_array_equal(rep["lse"], dense["lse"])
        assert not np.any(rep["skip_counts"])


@pytest.mark.parametrize("causal", [True, False])
def test_replay_random_mask_is_softmax_over_kept_columns(causal):
    """Every row against the scalar brute force over its unit's kept keys."""
    n_checked = n_empty = 0
    for seed in range(25):
        rng, q, k, v = _prefill_case(200 + seed, B=2, Hq=4, Hkv=2)
        B, Hq, L, _ = q.shape
        G = Hq // k.shape[1]
        Br, Bc = int(rng.choice([2, 3, 4])), int(rng.choice([1, 2, 3]))
        base = oracle.prefill(q, k, v, -np.inf, Br, Bc, causal)
        forced = _forced_random(rng, base["decision"], float(rng.uniform(0.2, 0.8)))
        rep = oracle.replay(q, k, v, forced, Br, Bc, causal)
        np.testing.assert_array_equal(rep["decision"], forced)
        np.testing.assert_array_equal(rep["skip_counts"], (forced == SKIPPED).sum(axis=-1))
        for b in range(B):
            for h in range(Hq):
                for r in range(L):
                    i = r // Br
                    tiles = oracle.visited_tiles(i, Br, Bc, L, causal)
                    cols = _kept_columns(forced[b, h, i], Bc, r, L, causal, tiles)
                    if not cols:
                        assert np.all(rep["out"][b, h, r] == 0) and rep["lse"][b, h, r] == -np.inf
                        n_empty += 1
                        continue
                    o, lse = bruteforce.naive_attention([q[b, h, r]], k[b, h // G, cols],
                                                        v[b, h // G, cols], False)
                    np.testing.assert_allclose(rep["out"][b, h, r], o[0], atol=1e-12, rtol=0)
                    assert abs(rep["lse"][b, h, r] - lse[0]) <= 1e-12
                    n_checked += 1
    assert n_checked > 1000 and n_empty > 0


def test_replay_with_block_list_uses_list_and_mask():
    """Forced decisions on top of a block list: only listed, kept tiles count."""
    for seed in range(15):
        rng, q, k, v = _prefill_case(300 + seed, B=1, Hq=2, Hkv=1, L=18, d=2)
        Br = Bc = 3
        nQ = nK = 6
        idx = np.full((1, 2, nQ, nK), -1, np.int32)
        cnt = np.zeros((1, 2, nQ), np.int32)
        for h in range(2):
            for i in range(nQ):
                lst = [j for j in range(i + 1) if rng.random() < 0.6] or [i]
                rng.shuffle(lst)
                idx[0, h, i, :len(lst)] = lst
                cnt[0, h, i] = len(lst)
        base = oracle.prefill(q, k, v, -np.inf, Br, Bc, True, block_idx=idx, block_cnt=cnt)
        forced = _forced_random(rng, base["decision"], 0.4)
        rep = oracle.replay(q, k, v, forced, Br, Bc, True, block_idx=idx, block_cnt=cnt)
        for h in range(2):
            for r in range(18):
                i = r // Br
                tiles = [int(j) for j in idx[0, h, i, :cnt[0, h, i]]]
                cols = _kept_columns(forced[0, h, i], Bc, r, 18, True, tiles)
                if not cols:
                    assert rep["lse"][0, h, r] == -np.inf
                    continue
                o, lse = bruteforce.naive_attention([q[0, h, r]], k[0, 0, cols], v[0, 0, cols], False)
                np.testing.assert_allclose(rep["out"][0, h, r], o[0], atol=1e-12, rtol=0)


def _decode_case(seed, B=3, Hq=4, Hkv=2, S_max=37, d=3):
    rng = np.random.default_rng(seed)
    spread = float(rng.uniform(0.5, 3.0))
    q = rng.standard_normal((B, Hq, d)) * spread
    kc = rng.standard_normal((B, Hkv, S_max, d)) * spread
    vc = rng.standard_normal((B, Hkv, S_max, d))
    lens = rng.integers(1, S_max + 1, size=B)
    return rng, q, kc, vc, lens


def test_decode_forced_own_decisions_bit_identical():
    for seed in range(40):
        rng, q, kc, vc, lens = _decode_case(seed)
        Bc, T = int(rng.choice([2, 3, 4])), int(rng.choice([1, 2, 3, 5]))
        lam = float(rng.uniform(-3.0, 0.0))
        ref = oracle.decode(q, kc, vc, lens, lam, Bc, T)
        rep = oracle.decode(q, kc, vc, lens, lam, Bc, T, forced=ref["decision"])
        for key in ("out", "lse", "decision", "skip_counts", "m_parts", "l_parts", "o_parts"):
            np.testing.assert_array_equal(rep[key], ref[key], err_msg=f"{key} seed {seed}")


def test_decode_forced_all_kept_equals_dense():
    for seed in range(30):
        rng, q, kc, vc, lens = _decode_case(50 + seed)
        Bc, T = int(rng.choice([2, 3, 4])), int(rng.choice([1, 2, 3]))
        dense = oracle.decode(q, kc, vc, lens, -np.inf, Bc, T)
        forced = np.where(dense["decision"] != NOT_VISITED, KEPT, NOT_VISITED).astype(np.int8)
        rep = oracle.decode(q, kc, vc, lens, 0.0, Bc, T, forced=forced)
        np.testing.assert_array_equal(rep["out"], dense["out"])
        np.testing.assert_array_equal(rep["lse"], dense["lse"])


def test_decode_forced_random_mask_is_softmax_over_kept_columns():
    """Per split: the split partial is the softmax sum over its kept keys;
    overall: softmax over every kept key of the sequence."""
    n_checked = 0
    for seed in range(40):
        rng, q, kc, vc, lens = _decode_case(100 + seed)
        B, Hq, d = q.shape
        Hkv = kc.shape[1]
        G = Hq // Hkv
        Bc, T = int(rng.choice([2, 3, 4])), int(rng.choice([1, 2, 3]))
        base = oracle.decode(q, kc, vc, lens, -np.inf, Bc, T)
        forced = _forced_random(rng, base["decision"], float(rng.uniform(0.2, 0.8)))
        rep = oracle.decode(q, kc, vc, lens, 0.0, Bc, T, forced=forced)
        np.testing.assert_array_equal(rep["decision"], forced)
        for b in range(B):
            n = int(lens[b])
            ntiles = math.ceil(n / Bc)
            for h in range(Hq):
                kvh = h // G
                kept = [c for c in range(n) if forced[b, kvh, c // Bc] == KEPT]
                if kept:
                    o, lse = bruteforce.naive_attention([q[b, h]], kc[b, kvh, kept], vc[b, kvh, kept], False)
                    np.testing.assert_allclose(rep["out"][b, h], o[0], atol=1e-12, rtol=0)
                    assert abs(rep["lse"][b, h] - lse[0]) <= 1e-12
                    n_checked += 1
                else:
                    assert np.all(rep["out"][b, h] == 0) and rep["lse"][b, h] == -np.inf
                # the split partials: l_s and o_s over the split's kept keys
                for sp in range(math.ceil(ntiles / T)):
                    cs = [c for c in kept if sp * T <= c // Bc < (sp + 1) * T]
                    if not cs:
                        assert rep["l_parts"][b, h, sp] == 0
                        continue
                    s = [float(np.dot(q[b, h], kc[b, kvh, c])) / math.sqrt(d) for c in cs]
                    m = max(s)
                    w = [math.exp(x - m) for x in s]
                    assert abs(rep["m_parts"][b, h, sp] - m) <= 1e-12
                    assert abs(rep["l_parts"][b, h, sp] - sum(w)) <= 1e-12 * max(1.0, sum(w))
                    ov = sum(wt * vc[b, kvh, c] for wt, c in zip(w, cs))
                    np.testing.assert_allclose(rep["o_parts"][b, h, sp], ov, atol=1e-12, rtol=0)
    assert n_checked > 300
