"""Seeded synthetic inputs for Skip-Softmax attention (prefill and decode).

This module only draws and rounds input tensors. It holds none of the
attention arithmetic and is shared by the tests, the benchmark and the
oracle checks, so that both sides see bit-identical inputs.

Recipe (the planted-direction workload of the Skip-Softmax pages: a
shared direction added to the queries and to a fraction of key blocks,
plus a sink key):

* Q, K, V entries are standard normal draws (numpy PCG64, float32).
* One unit direction ``u`` (a normalised Gaussian vector of length d) is
  drawn per (batch, KV head); every query head of that group shares it.
* ``plant`` * u is added to every query row.
* ``round(frac * nblocks)`` key blocks of ``block`` tokens are drawn without
  replacement; ``plant`` * u is added to every key row in them.
* ``sink`` * u is added to key 0 (on top of any planting).
* Optional block drift (``drift`` > 0, for the block-similarity predictor
  of the SpargeAttn page, whose premise is that neighbouring tokens are
  alike): every block of ``block`` rows of Q (per query head) and of K gets
  one shared vector a_j * w_j added to all its rows, with w_j a standard
  normal vector and a_j uniform in [0, drift], so blocks range from
  unrelated tokens (a_j near 0) to nearly identical ones.
* Every value is rounded to bfloat16 with round-to-nearest-even.

Every piece is drawn from its own ``numpy.random.SeedSequence`` keyed by
(config id, seed, batch, KV head, stream, sub-index, chunk), so any head or
row chunk can be regenerated alone and pieces can be drawn in parallel.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

CHUNK_ROWS = 4096

# stream ids inside one (config, seed, batch, kv head) key
_S_U, _S_PLANT, _S_Q, _S_K, _S_V, _S_DQ = 0, 1, 2, 3, 4, 5
_S_LENS = 6
_S_DRIFT = 7


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the
    16-bit patterns as uint16. NaN maps to a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16/int16) to exact float32 values."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(x) for x in key])))


def _direction(cfg, seed, b, kvh, d) -> np.ndarray:
    u = _rng(cfg, seed, b, kvh, _S_U).standard_normal(d)
    return (u / np.linalg.norm(u)).astype(np.float32)


def _planted_blocks(cfg, seed, b, kvh, nblocks, frac) -> np.ndarray:
    n = int(round(frac * nblocks))
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(cfg, seed, b, kvh, _S_PLANT).choice(nblocks, size=n, replace=False))


def _normal_rows(key, rows, d) -> np.ndarray:
    """Draw ``rows`` x ``d`` standard normals, chunk by chunk, each chunk from
    its own seed (key + (chunk,))."""
    out = np.empty((rows, d), dtype=np.float32)
    for c in range(0, max(1, math.ceil(rows / CHUNK_ROWS))):
        r0, r1 = c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS)
        if r1 > r0:
            out[r0:r1] = _rng(*key, c).standard_normal((r1 - r0, d), dtype=np.float32)
    return out


def _add_drift(x, key, block, drift):
    """Add a_j * w_j to every row of block j (see the module docstring)."""
    if drift <= 0:
        return
    L, d = x.shape
    nb = math.ceil(L / block)
    rng = _rng(*key)
    amp = rng.uniform(0.0, drift, nb).astype(np.float32)
    w = rng.standard_normal((nb, d), dtype=np.float32)
    for j in range(nb):
        x[j * block:min(L, (j + 1) * block)] += amp[j] * w[j]


def _prefill_piece(args):
    cfg, seed, b, kvh, G, L, d, block, frac, plant, sink, drift, what, g = args
    u = _direction(cfg, seed, b, kvh, d)
    if what == "q":
        x = _normal_rows((cfg, seed, b, kvh, _S_Q, g), L, d)
        x += np.float32(plant) * u
        _add_drift(x, (cfg, seed, b, kvh, _S_DRIFT, 1 + g), block, drift)
        return bf16_bits(x)
    if what == "k":
        x = _normal_rows((cfg, seed, b, kvh, _S_K), L, d)
        _add_drift(x, (cfg, seed, b, kvh, _S_DRIFT, 0), block, drift)
        nb = math.ceil(L / block)
        for blk in _planted_blocks(cfg, seed, b, kvh, nb, frac):
            x[blk * block:min(L, (blk + 1) * block)] += np.float32(plant) * u
        if L > 0:
            x[0] += np.float32(sink) * u
        return bf16_bits(x)
    x = _normal_rows((cfg, seed, b, kvh, _S_V), L, d)
    return bf16_bits(x)


def _pool(n_tasks, workers):
    if workers is None:
        workers = int(os.environ.get("SYNTH_WORKERS", "0")) or min(16, os.cpu_count() or 1)
    return max(1, min(workers, n_tasks))


def _run(fn, tasks, workers):
    w = _pool(len(tasks), workers)
    if w == 1 or len(tasks) <= 2:
        return [fn(t) for t in tasks]
    with ProcessPoolExecutor(max_workers=w) as ex:
        return list(ex.map(fn, tasks, chunksize=1))


def prefill_inputs(cfg: int, seed: int, B: int, Hq: int, Hkv: int, L: int, d: int,
                   block: int = 64, frac: float = 0.1, plant: float = 4.0, sink: float = 8.0,
                   drift: float = 0.0, workers: int | None = None) -> dict:
    """Q [B,Hq,L,d], K and V [B,Hkv,L,d] as bfloat16 bit patterns (uint16).

    Query head hq belongs to KV head hq // (Hq // Hkv)."""
    assert Hq % Hkv == 0
    G = Hq // Hkv
    tasks = []
    for b in range(B):
        for kvh in range(Hkv):
            for g in range(G):
                tasks.append((cfg, seed, b, kvh, G, L, d, block, frac, plant, sink, drift, "q", g))
            tasks.append((cfg, seed, b, kvh, G, L, d, block, frac, plant, sink, drift, "k", 0))
            tasks.append((cfg, seed, b, kvh, G, L, d, block, frac, plant, sink, drift, "v", 0))
    res = _run(_prefill_piece, tasks, workers)
    q = np.empty((B, Hq, L, d), np.uint16)
    k = np.empty((B, Hkv, L, d), np.uint16)
    v = np.empty((B, Hkv, L, d), np.uint16)
    it = iter(res)
    for b in range(B):
        for kvh in range(Hkv):
            for g in range(G):
                q[b, kvh * G + g] = next(it)
            k[b, kvh] = next(it)
            v[b, kvh] = next(it)
    planted = [[_planted_blocks(cfg, seed, b, kvh, math.ceil(L / block), frac)
                for kvh in range(Hkv)] for b in range(B)]
    return {"q": q, "k": k, "v": v, "planted": planted}


def decode_seqlens(cfg: int, seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence cache lengths, uniform integers in [lo, hi]."""
    return _rng(cfg, seed, _S_LENS).integers(lo, hi + 1, size=B).astype(np.int32)


def _decode_piece(args):
    cfg, seed, b, kvh, G, n, S_max, d, block, frac, plant, sink, what = args
    u = _direction(cfg, seed, b, kvh, d)
    if what == "q":
        x = _rng(cfg, seed, b, kvh, _S_DQ).standard_normal((G, d), dtype=np.float32)
        x += np.float32(plant) * u
        return bf16_bits(x)
    if what == "k":
        x = _normal_rows((cfg, seed, b, kvh, _S_K), n, d)
        nb = math.ceil(n / block)
        for blk in _planted_blocks(cfg, seed, b, kvh, nb, frac):
            x[blk * block:min(n, (blk + 1) * block)] += np.float32(plant) * u
        if n > 0:
            x[0] += np.float32(sink) * u
        return bf16_bits(x)
    return bf16_bits(_normal_rows((cfg, seed, b, kvh, _S_V), n, d))


# bfloat16 pattern written into cache slots past a sequence's length: a
# quiet NaN, so that any read of them shows up in the outputs.
TAIL_FILL = 0x7FC0


def decode_inputs(cfg: int, seed: int, B: int, Hq: int, Hkv: int, S_max: int, d: int,
                  len_lo: int, len_hi: int, block: int = 64, frac: float = 0.1,
                  plant: float = 4.0, sink: float = 8.0, seqlens=None,
                  tail_fill: int = TAIL_FILL, workers: int | None = None) -> dict:
    """One query token per sequence: q [B,Hq,d]; caches [B,Hkv,S_max,d]
    with the first seqlens[b] rows valid and the rest set to ``tail_fill``."""
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if seqlens is None:
        seqlens = decode_seqlens(cfg, seed, B, len_lo, len_hi)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    tasks = []
    for b in range(B):
        n = int(min(max(seqlens[b], 0), S_max))
        for kvh in range(Hkv):
            for what in ("q", "k", "v"):
                tasks.append((cfg, seed, b, kvh, G, n, S_max, d, block, frac, plant, sink, what))
    res = _run(_decode_piece, tasks, workers)
    q = np.empty((B, Hq, d), np.uint16)
    kc = np.full((B, Hkv, S_max, d), tail_fill, np.uint16)
    vc = np.full((B, Hkv, S_max, d), tail_fill, np.uint16)
    it = iter(res)
    for b in range(B):
        n = int(min(max(seqlens[b], 0), S_max))
        for kvh in range(Hkv):
            q[b, kvh * G:(kvh + 1) * G] = next(it)
            kc[b, kvh, :n] = next(it)
            vc[b, kvh, :n] = next(it)
    return {"q": q, "k_cache": kc, "v_cache": vc, "seqlens": seqlens}


# The five seeded workloads: shapes and generator settings.
CONFIGS = {
    0: dict(kind="prefill", B=1, Hq=1, Hkv=1, L=1024, d=64, Br=64, Bc=64, causal=True,
            frac=0.10, lam=-6.0),
    1: dict(kind="prefill", B=1, Hq=32, Hkv=8, L=16384, d=128, Br=128, Bc=64, causal=True,
            frac=0.10, target_skip=0.5),
    # split_tiles: 16 key tiles per split (6368 splits for these lengths):
    # 2% faster than 24 tiles and 3% faster than 12 at ~50% skip with the
    # persistent split kernel
    2: dict(kind="decode", B=32, Hq=32, Hkv=8, S_max=32768, d=128, Bc=64, len_lo=16384,
            len_hi=32768, split_tiles=16, frac=0.10, target_skip=0.5),
    3: dict(kind="prefill", B=1, Hq=8, Hkv=1, L=131072, d=128, Br=128, Bc=64, causal=True,
            frac=0.05, lam_sweep=[-3.0, -4.0, -5.0, -6.0, -7.0, -8.0, -9.0]),
    4: dict(kind="sparse", B=1, Hq=16, Hkv=16, L=32768, d=64, Br=64, Bc=64, causal=True,
            frac=0.10, pool=64, topk=64, sink_blocks=1, window_tokens=1024, lam=-6.0),
}

# SpargeAttn two-stage workload: the block-sparse shape above with drifting
# blocks, stage one (theta, tau) then the skip rule (lam) over its lists.
SPARGE = dict(kind="sparge", cfg_id=5, B=1, Hq=16, Hkv=16, L=32768, d=64, Br=64, Bc=64,
              causal=True, frac=0.10, drift=2.0, pool=64, theta=0.2, tau=0.9, lam=-6.0)
