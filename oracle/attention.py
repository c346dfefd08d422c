"""fp64 oracle for Skip-Softmax tiled attention (prefill and split-K decode).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions (pages: "TRT-LLM sparse attention, 1.4x" -- the three-step
algorithm and the benefits section; "SpargeAttn" -- stage two of the
two-stage online filter):

* score s[r, c] = q_r . k_c / sqrt(d), in natural-log units; entries that are
  not allowed (c > r under the causal mask, c >= len in decode, key tile
  not in the block list) are -inf.
* Work is split into decision units. Prefill: the Br consecutive query rows
  of one query head (query tile i). Decode: the G query heads that share one
  KV head, one row each, over one split of ``split_tiles`` key tiles.
* Inside a unit the key tiles (Bc keys each) are visited in ascending order
  (block list order in the sparse case). For tile j and row r:
  m_loc = max of the row's scores in the tile, m_prev = max over the tiles
  visited before j in the unit (-inf if none). The row gap is m_loc - m_prev,
  with gap = -inf when the row has no allowed key in the tile and gap = +inf
  when m_prev = -inf but m_loc is finite (the first tile). The tile margin is
  g_j = max over rows of the gap, and the tile is skipped iff g_j < lambda
  (strict, lambda <= 0).
* A skipped tile contributes nothing: no exponentials, no row-sum, no P.V.
  The output is softmax attention renormalised over the kept tiles:
  m = row max, l = sum exp(s - m), o = sum exp(s - m) v / l, lse = m + ln l.
  A row with no kept allowed key gets o = 0, lse = -inf.

Inputs may be float arrays or bfloat16 bit patterns (uint16, ``bits=True``);
slices are widened to float64 one unit at a time.
"""

from __future__ import annotations

import math

import numpy as np

NOT_VISITED, KEPT, SKIPPED = 0, 1, 2


def _widen(x, bits: bool) -> np.ndarray:
    """float64 view of a slice; bfloat16 bit patterns are placed in the top
    half of a float32 word (the bfloat16 format definition)."""
    if bits:
        w = np.asarray(x).view(np.uint16).astype(np.uint32) << 16
        return w.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def visited_tiles(i: int, Br: int, Bc: int, L: int, causal: bool, block_list=None) -> list:
    """Key tiles visited by query tile i, in visit order.

    Dense: every tile 0..nK-1; causal keeps tiles with j*Bc <= last row of
    the query tile (at least one allowed entry). With a block list, its
    entries are taken in the given order and entries outside [0, nK) or
    above the causal limit are ignored."""
    nK = math.ceil(L / Bc)
    last_row = min((i + 1) * Br, L) - 1
    cand = range(nK) if block_list is None else [int(j) for j in block_list]
    out = []
    for j in cand:
        if j < 0 or j >= nK:
            continue
        if causal and j * Bc > last_row:
            continue
        out.append(j)
    return out


def _row_gaps(m_loc: np.ndarray, m_prev: np.ndarray) -> np.ndarray:
    gap = np.empty_like(m_loc)
    none = m_loc == -np.inf
    first = (~none) & (m_prev == -np.inf)
    rest = ~(none | first)
    gap[none] = -np.inf
    gap[first] = np.inf
    gap[rest] = m_loc[rest] - m_prev[rest]
    return gap


def _softmax_out(s_list, v_list, nrows, d):
    """Renormalised softmax over the kept score blocks: (o, lse, m, l, p)."""
    if not s_list:
        return (np.zeros((nrows, d)), np.full(nrows, -np.inf), np.full(nrows, -np.inf),
                np.zeros(nrows), np.zeros((nrows, 0)))
    s = np.concatenate(s_list, axis=1)
    vv = np.concatenate(v_list, axis=0)
    m = s.max(axis=1)
    ok = m > -np.inf
    p = np.zeros_like(s)
    p[ok] = np.exp(s[ok] - m[ok, None])
    l = p.sum(axis=1)
    o = np.zeros((nrows, d))
    o[ok] = (p[ok] @ vv) / l[ok, None]
    lse = np.full(nrows, -np.inf)
    lse[ok] = m[ok] + np.log(l[ok])
    return o, lse, m, l, p


def nm_mask(s: np.ndarray, rows: np.ndarray, cols: np.ndarray, n: int, m: int,
            dense_sink: int = 0, dense_recent: int = 0) -> np.ndarray:
    """N:M sparse softmax mask (Model Optimizer tutorial, step 2: in every M
    consecutive key positions only the top-N scores are kept, the others are
    set to -inf; FAQ: sink tokens and recent tokens stay dense).

    s [nrows, ncols] holds scores with -inf where not allowed; rows/cols are
    the absolute positions. Groups are aligned: key c is in group c // m.
    Within a group, allowed positions are ranked by score (ties: lower c
    first) and the top n are kept; positions c < dense_sink or
    row - dense_recent < c <= row are kept as well. Returns the masked copy."""
    out = np.full_like(s, -np.inf)
    for a, r in enumerate(rows):
        for g0 in range(0, s.shape[1], m):
            idx = list(range(g0, min(g0 + m, s.shape[1])))
            allowed = [i for i in idx if s[a, i] > -np.inf]
            ranked = sorted(allowed, key=lambda i: (-s[a, i], cols[i]))
            keep = set(ranked[:n])
            for i in allowed:
                c = cols[i]
                if c < dense_sink or r - dense_recent < c <= r:
                    keep.add(i)
            for i in keep:
                out[a, i] = s[a, i]
    return out


def prefill(q, k, v, lam: float, Br: int, Bc: int, causal: bool = True,
            block_idx=None, block_cnt=None, units=None, forced=None,
            bits: bool = False, return_probs: bool = False, nm=None,
            dense_sink: int = 0, dense_recent: int = 0) -> dict:
    """Skip-Softmax prefill. q [B,Hq,L,d]; k, v [B,Hkv,L,d]; query head hq
    reads KV head hq // (Hq/Hkv).

    ``block_idx`` [B,Hq,nQ,max] / ``block_cnt`` [B,Hq,nQ] restrict each query
    tile to a list of key tiles. ``nm`` = (N, M) applies N:M sparse softmax
    (``nm_mask``, with ``dense_sink`` / ``dense_recent`` exemptions) to the
    scores before the tile rule. ``units`` limits the work to a list of
    (b, hq, i). ``forced`` [B,Hq,nQ,nK] (KEPT/SKIPPED) replaces the rule's
    decisions (replay). Returns a dict with out [B,Hq,L,d], lse [B,Hq,L],
    decision and margin [B,Hq,nQ,nK] (margin NaN where not visited),
    skip_counts [B,Hq,nQ], and the probabilities [B,Hq,L,L] if asked."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0 and k.shape == (B, Hkv, L, d) and v.shape == k.shape
    G = Hq // Hkv
    nQ, nK = math.ceil(L / Br), math.ceil(L / Bc)
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, L, d))
    lse = np.full((B, Hq, L), -np.inf)
    decision = np.zeros((B, Hq, nQ, nK), np.int8)
    margin = np.full((B, Hq, nQ, nK), np.nan)
    skip_counts = np.zeros((B, Hq, nQ), np.int64)
    probs = np.zeros((B, Hq, L, L)) if return_probs else None
    if units is None:
        units = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nQ)]
    with np.errstate(invalid="ignore", over="ignore"):
        for (b, hq, i) in units:
            kvh = hq // G
            r0, r1 = i * Br, min(L, (i + 1) * Br)
            rows = np.arange(r0, r1)
            blist = None
            if block_idx is not None:
                blist = block_idx[b, hq, i, :int(block_cnt[b, hq, i])]
            tiles = visited_tiles(i, Br, Bc, L, causal, blist)
            qi = _widen(q[b, hq, r0:r1], bits)
            m_prev = np.full(r1 - r0, -np.inf)
            s_kept, v_kept, c_kept = [], [], []
            for j in tiles:
                c0, c1 = j * Bc, min(L, (j + 1) * Bc)
                s = (qi @ _widen(k[b, kvh, c0:c1], bits).T) * scale
                if causal:
                    s[np.arange(c0, c1)[None, :] > rows[:, None]] = -np.inf
                if nm is not None:
                    s = nm_mask(s, rows, np.arange(c0, c1), nm[0], nm[1], dense_sink, dense_recent)
                m_loc = s.max(axis=1)
                g = _row_gaps(m_loc, m_prev).max()
                margin[b, hq, i, j] = g
                if forced is None:
                    skip = g < lam
                else:
                    skip = forced[b, hq, i, j] == SKIPPED
                decision[b, hq, i, j] = SKIPPED if skip else KEPT
                m_prev = np.maximum(m_prev, m_loc)
                if skip:
                    skip_counts[b, hq, i] += 1
                else:
                    s_kept.append(s)
                    v_kept.append(_widen(v[b, kvh, c0:c1], bits))
                    c_kept.append(np.arange(c0, c1))
            o, ls, _, l, p = _softmax_out(s_kept, v_kept, r1 - r0, d)
            out[b, hq, r0:r1] = o
            lse[b, hq, r0:r1] = ls
            if probs is not None and c_kept:
                cols = np.concatenate(c_kept)
                ok = l > 0
                probs[b, hq, r0:r1][np.ix_(ok, cols)] = p[ok] / l[ok, None]
    res = {"out": out, "lse": lse, "decision": decision, "margin": margin,
           "skip_counts": skip_counts}
    if probs is not None:
        res["probs"] = probs
    return res


def replay(q, k, v, forced, Br: int, Bc: int, causal: bool = True, **kw) -> dict:
    """Prefill outputs for given skip decisions (KEPT/SKIPPED per tile):
    the outputs that a kernel taking exactly those decisions must produce."""
    return prefill(q, k, v, 0.0, Br, Bc, causal, forced=forced, **kw)


def lse_combine_parts(m_parts, l_parts, o_parts):
    """Log-sum-exp combine of partial softmax sums over disjoint key sets.

    Part s holds m_s (its max), l_s = sum exp(x - m_s) and the unnormalised
    o_s = sum exp(x - m_s) v. Then lse = log sum_s l_s exp(m_s) and
    out = sum_s exp(m_s - lse) o_s. Parts with l_s = 0 are empty. Arrays
    carry the part index on axis -1 (m, l) and -2 (o)."""
    m_parts = np.asarray(m_parts, np.float64)
    l_parts = np.asarray(l_parts, np.float64)
    o_parts = np.asarray(o_parts, np.float64)
    live = l_parts > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        lse_s = np.where(live, m_parts + np.log(np.where(live, l_parts, 1.0)), -np.inf)
    top = lse_s.max(axis=-1, keepdims=True)
    finite = np.isfinite(top)
    top_safe = np.where(finite, top, 0.0)
    w = np.where(live, np.exp(lse_s - top_safe), 0.0)
    tot = w.sum(axis=-1, keepdims=True)
    lse = np.where(finite, top_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    scale = np.where(live, np.exp(np.where(live, m_parts, 0.0) - np.where(finite, lse, 0.0)), 0.0)
    out = (scale[..., :, None] * o_parts).sum(axis=-2)
    return out, lse[..., 0]


combine = lse_combine_parts


def decode(q, k_cache, v_cache, seqlens, lam: float, Bc: int, split_tiles: int,
           units=None, forced=None, bits: bool = False) -> dict:
    """Skip-Softmax single-token decode with split-K partials.

    q [B,Hq,d]; caches [B,Hkv,S_max,d] of which the first seqlens[b] rows are
    valid (lengths are clamped to [0, S_max]). The new token attends all valid
    keys. The unit is (b, KV head, split): the G query heads of that KV head
    over key tiles [s*T, (s+1)*T) of the sequence; the running max restarts
    at each split. Partials (m, l, unnormalised o) per split are combined with
    the log-sum-exp identity. ``units`` limits work to a list of (b, kvh).
    ``forced`` [B,Hkv,nTiles] replaces the rule's decisions. Returns out
    [B,Hq,d], lse [B,Hq], decision/margin [B,Hkv,nTiles], skip_counts
    [B,Hkv,nSplits], and the partials."""
    B, Hq, d = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    assert Hq % Hkv == 0
    G = Hq // Hkv
    T = int(split_tiles)
    nT = math.ceil(S_max / Bc)
    nS = math.ceil(nT / T)
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    decision = np.zeros((B, Hkv, nT), np.int8)
    margin = np.full((B, Hkv, nT), np.nan)
    skip_counts = np.zeros((B, Hkv, nS), np.int64)
    m_parts = np.full((B, Hq, nS), -np.inf)
    l_parts = np.zeros((B, Hq, nS))
    o_parts = np.zeros((B, Hq, nS, d))
    if units is None:
        units = [(b, h) for b in range(B) for h in range(Hkv)]
    seqlens = np.asarray(seqlens)
    with np.errstate(invalid="ignore", over="ignore"):
        for (b, kvh) in units:
            n = int(min(max(int(seqlens[b]), 0), S_max))
            rows = _widen(q[b, kvh * G:(kvh + 1) * G], bits)
            ntiles = math.ceil(n / Bc)
            for sp in range(math.ceil(ntiles / T)):
                m_prev = np.full(G, -np.inf)
                s_kept, v_kept = [], []
                for j in range(sp * T, min(ntiles, (sp + 1) * T)):
                    c0, c1 = j * Bc, min(n, (j + 1) * Bc)
                    s = (rows @ _widen(k_cache[b, kvh, c0:c1], bits).T) * scale
                    m_loc = s.max(axis=1)
                    g = _row_gaps(m_loc, m_prev).max()
                    margin[b, kvh, j] = g
                    skip = (g < lam) if forced is None else (forced[b, kvh, j] == SKIPPED)
                    decision[b, kvh, j] = SKIPPED if skip else KEPT
                    m_prev = np.maximum(m_prev, m_loc)
                    if skip:
                        skip_counts[b, kvh, sp] += 1
                    else:
                        s_kept.append(s)
                        v_kept.append(_widen(v_cache[b, kvh, c0:c1], bits))
                if s_kept:
                    s = np.concatenate(s_kept, axis=1)
                    vv = np.concatenate(v_kept, axis=0)
                    m = s.max(axis=1)
                    p = np.exp(s - m[:, None])
                    hs = slice(kvh * G, (kvh + 1) * G)
                    m_parts[b, hs, sp] = m
                    l_parts[b, hs, sp] = p.sum(axis=1)
                    o_parts[b, hs, sp] = p @ vv
            hs = slice(kvh * G, (kvh + 1) * G)
            o, ls = lse_combine_parts(m_parts[b, hs], l_parts[b, hs], o_parts[b, hs])
            out[b, hs] = o
            lse[b, hs] = ls
    return {"out": out, "lse": lse, "decision": decision, "margin": margin,
            "skip_counts": skip_counts, "m_parts": m_parts, "l_parts": l_parts,
            "o_parts": o_parts}
