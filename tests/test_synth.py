"""The seeded generator: determinism, per-piece seeding and planted structure."""

import math

import numpy as np

import synth


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, np.inf, 1e-40], np.float32)
    b = synth.bf16_bits(x)
    back = synth.bf16_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                 # tie -> even (mantissa 0)
    assert back[2] == 1.0 + 2 ** -6       # tie -> even (rounds up)
    assert back[3] == -2.5 and np.isinf(back[4])
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    rb = synth.bf16_to_f32(synth.bf16_bits(r))
    assert np.max(np.abs(rb - r) / np.abs(r)) <= 2 ** -8  # unit roundoff, 8-bit significand


def test_prefill_generator_deterministic_and_parallel_equal():
    a = synth.prefill_inputs(100, 1, 1, 4, 2, 300, 8, workers=1)
    b = synth.prefill_inputs(100, 1, 1, 4, 2, 300, 8, workers=3)
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(a[key], b[key])
    c = synth.prefill_inputs(100, 2, 1, 4, 2, 300, 8, workers=1)
    assert not np.array_equal(a["q"], c["q"])


def test_planted_direction_structure():
    L, d, blk = 4096, 64, 64
    x = synth.prefill_inputs(101, 0, 1, 2, 1, L, d, block=blk, frac=0.1, workers=1)
    q = synth.bf16_to_f32(x["q"]).astype(np.float64)
    k = synth.bf16_to_f32(x["k"]).astype(np.float64)
    planted = x["planted"][0][0]
    assert len(planted) == round(0.1 * math.ceil(L / blk))
    # recover u from the mean query row: mean(q) ~ 4u
    u = q[0].mean(axis=(0, 1))
    u /= np.linalg.norm(u)
    proj = k[0, 0] @ u
    blocks = proj.reshape(-1, blk).mean(axis=1)
    is_p = np.zeros(L // blk, bool)
    is_p[planted] = True
    assert blocks[is_p].mean() > 3.5 and abs(blocks[~is_p].mean()) < 0.5
    assert proj[0] > 6.0                                # sink key
    # both query heads share the group's direction
    u1 = q[0, 1].mean(axis=0)
    assert u1 @ u / np.linalg.norm(u1) > 0.99


def test_decode_generator_lengths_and_tail():
    x = synth.decode_inputs(102, 0, 3, 4, 2, 256, 16, 100, 200, workers=1)
    lens = x["seqlens"]
    assert np.all((lens >= 100) & (lens <= 200))
    for b in range(3):
        assert np.all(x["k_cache"][b, :, lens[b]:] == synth.TAIL_FILL)
        assert not np.any(x["k_cache"][b, :, :lens[b]] == synth.TAIL_FILL)
    y = synth.decode_inputs(102, 0, 3, 4, 2, 256, 16, 100, 200, workers=2)
    np.testing.assert_array_equal(x["k_cache"], y["k_cache"])
