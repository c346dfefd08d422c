"""Host-side arithmetic of the benchmark: algorithmic byte and tile counts
(checked against hand counts and against the oracle's visit rule)."""

import math

import numpy as np

import bench
import oracle


def test_decode_loaded_bytes_hand_count():
    # B=2, Hq=4, Hkv=2, d=8, Bc=64, splits of T=2 tiles, lengths 100 and 200,
    # 5 kept tiles:
    #   K   2 B * 8 * 2 heads * (100 + 200) keys          = 9600
    #   V   2 B * 8 * 64 keys * 5 tiles                    = 5120
    #   q + out  2 * (2 B * 2 seq * 4 heads * 8)           = 256
    #   lse 4 B * 2 * 4                                    = 32
    #   partials: ceil(ceil(100/64)/2) + ceil(ceil(200/64)/2) = 1 + 2 = 3 splits
    #             per sequence-head, written and read: 2 * 4 B * 4 heads * 3 * (8 + 2) = 960
    assert bench.decode_loaded_bytes([100, 200], 2, 4, 2, 8, 64, 2, 5) == 9600 + 5120 + 256 + 32 + 960


def test_decode_loaded_bytes_workspace_counts_batch_once():
    # the split partials grow with the sum of the splits over sequences, not
    # with B times that sum: doubling the batch with copies of the same
    # sequences doubles every term
    one = bench.decode_loaded_bytes([1000, 3000], 2, 8, 2, 128, 64, 4, 17)
    two = bench.decode_loaded_bytes([1000, 3000] * 2, 4, 8, 2, 128, 64, 4, 34)
    assert two == 2 * one


def test_visited_tiles_count_dense_hand_count():
    # L=333, Br=128, Bc=64: query tiles end at rows 127, 255, 332 -> 2, 4, 6
    # causal tiles; 6 tiles each without the mask; two heads
    assert bench.visited_tiles_count(1, 2, 333, 128, 64, True) == 24
    assert bench.visited_tiles_count(1, 2, 333, 128, 64, False) == 36


def test_visited_tiles_count_matches_visit_rule():
    rng = np.random.default_rng(0)
    for _ in range(20):
        L = int(rng.integers(1, 700))
        Br = int(rng.choice([32, 64, 128]))
        Bc = 64
        B, H = 2, 3
        nQ, nK = math.ceil(L / Br), math.ceil(L / Bc)
        causal = bool(rng.integers(2))
        want = sum(len(oracle.visited_tiles(i, Br, Bc, L, causal)) for i in range(nQ)) * B * H
        assert bench.visited_tiles_count(B, H, L, Br, Bc, causal) == want
        mb = 6
        idx = rng.integers(-2, nK + 3, size=(B, H, nQ, mb)).astype(np.int32)
        cnt = rng.integers(-1, mb + 2, size=(B, H, nQ)).astype(np.int32)
        want = sum(len(oracle.visited_tiles(i, Br, Bc, L, causal,
                                            idx[b, h, i, :max(0, min(int(cnt[b, h, i]), mb))]))
                   for b in range(B) for h in range(H) for i in range(nQ))
        assert bench.visited_tiles_count(B, H, L, Br, Bc, causal, idx, cnt) == want
