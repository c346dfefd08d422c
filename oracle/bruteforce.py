"""Scalar-loop second implementation for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written with plain Python loops and ``math`` so that it shares no array code
with ``oracle.attention``; the tests compare the two on many random tiny
cases. Rule and output as in ``oracle.attention`` (Skip-Softmax three-step
algorithm of the TRT-LLM page; SpargeAttn stage two).
"""

from __future__ import annotations

import math


def _dot(a, b):
    t = 0.0
    for x, y in zip(a, b):
        t += float(x) * float(y)
    return t


def naive_attention(q, k, v, causal):
    """softmax(q k^T / sqrt(d)) v for one head: q [Lq][d], k/v [Lk][d]."""
    d = len(q[0])
    out, lses = [], []
    for r, qr in enumerate(q):
        cols = [c for c in range(len(k)) if (not causal or c <= r)]
        s = [_dot(qr, k[c]) / math.sqrt(d) for c in cols]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = sum(w)
        out.append([sum(w[t] * float(v[c][e]) for t, c in enumerate(cols)) / tot
                    for e in range(len(v[0]))])
        lses.append(m + math.log(tot))
    return out, lses


def skip_attention(q, k, v, lam, Br, Bc, causal):
    """One head, prefill. Returns (out, lse, skipped) where skipped is the set
    of (query tile, key tile) pairs the rule skips."""
    L, d = len(q), len(q[0])
    nQ = (L + Br - 1) // Br
    nK = (L + Bc - 1) // Bc
    skipped = set()
    out = [[0.0] * len(v[0]) for _ in range(L)]
    lses = [-math.inf] * L
    for i in range(nQ):
        rows = list(range(i * Br, min(L, (i + 1) * Br)))
        runmax = {r: -math.inf for r in rows}
        kept_cols = {r: [] for r in rows}
        for j in range(nK):
            cols = list(range(j * Bc, min(L, (j + 1) * Bc)))
            if causal and cols[0] > rows[-1]:
                continue
            worst = -math.inf
            locs = {}
            for r in rows:
                loc = -math.inf
                for c in cols:
                    if causal and c > r:
                        continue
                    loc = max(loc, _dot(q[r], k[c]) / math.sqrt(d))
                locs[r] = loc
                if loc == -math.inf:
                    gap = -math.inf
                elif runmax[r] == -math.inf:
                    gap = math.inf
                else:
                    gap = loc - runmax[r]
                worst = max(worst, gap)
            skip = worst < lam
            if skip:
                skipped.add((i, j))
            for r in rows:
                runmax[r] = max(runmax[r], locs[r])
                if not skip:
                    kept_cols[r].extend(c for c in cols if not (causal and c > r))
        for r in rows:
            cs = kept_cols[r]
            if not cs:
                continue
            s = [_dot(q[r], k[c]) / math.sqrt(d) for c in cs]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            out[r] = [sum(w[t] * float(v[c][e]) for t, c in enumerate(cs)) / tot
                      for e in range(len(v[0]))]
            lses[r] = m + math.log(tot)
    return out, lses, skipped


def decode_skip_set(q_rows, k, n, lam, Bc, T):
    """Decode, one KV head: q_rows [G][d], k [n][d]. Skipped tile indices."""
    d = len(q_rows[0])
    ntiles = (n + Bc - 1) // Bc
    skipped = set()
    for sp in range((ntiles + T - 1) // T):
        runmax = [-math.inf] * len(q_rows)
        for j in range(sp * T, min(ntiles, (sp + 1) * T)):
            worst = -math.inf
            locs = []
            for g, qr in enumerate(q_rows):
                loc = max(_dot(qr, k[c]) / math.sqrt(d) for c in range(j * Bc, min(n, (j + 1) * Bc)))
                locs.append(loc)
                gap = math.inf if runmax[g] == -math.inf else loc - runmax[g]
                worst = max(worst, gap)
            if worst < lam:
                skipped.add(j)
            runmax = [max(a, b) for a, b in zip(runmax, locs)]
    return skipped


def topk_blocks(q, k, pool, topk, sink_blocks, window_tokens, kernel=None, stride=None):
    """Block mask for one head by explicit loops: q, k [L][d]. With kernel
    and stride, a key block's score is the best score of the overlapping
    compressed windows (kernel tokens, every stride tokens) starting in it."""
    L, d = len(q), len(q[0])
    nb = (L + pool - 1) // pool

    def mean(rows):
        return [sum(float(x[e]) for x in rows) / len(rows) for e in range(d)]

    qb = [mean(q[b * pool:min(L, (b + 1) * pool)]) for b in range(nb)]
    if kernel is None:
        kw = [[mean(k[c * pool:min(L, (c + 1) * pool)])] for c in range(nb)]
    else:
        kw = [[mean(k[s:min(L, s + kernel)]) for s in range(c * pool, min(L, (c + 1) * pool), stride)]
              for c in range(nb)]
    W = -(-window_tokens // pool) if window_tokens > 0 else 0
    res = []
    for b in range(nb):
        scored = [(-max(_dot(qb[b], w) for w in kw[c]) / math.sqrt(d), c) for c in range(b + 1)]
        scored.sort()
        keep = {c for _, c in scored[:topk]}
        keep |= {c for c in range(min(sink_blocks, b + 1))}
        keep |= {c for c in range(max(0, b - W + 1), b + 1)}
        res.append(sorted(keep))
    return res


def nm_attention(q, k, v, n, m, causal, dense_sink=0, dense_recent=0):
    """One head, N:M sparse softmax without tile skipping, by explicit loops:
    for each row and each aligned group of m keys, keep the n allowed keys
    with the highest scores (ties: lower index), plus sink / recent keys."""
    L, d = len(q), len(q[0])
    out, lses = [], []
    for r in range(L):
        kept = []
        for g0 in range(0, L, m):
            grp = [c for c in range(g0, min(g0 + m, L)) if not (causal and c > r)]
            sc = [(-_dot(q[r], k[c]) / math.sqrt(d), c) for c in grp]
            sc.sort()
            chosen = {c for _, c in sc[:n]}
            chosen |= {c for c in grp if c < dense_sink or r - dense_recent < c <= r}
            kept.extend(sorted(chosen))
        s = [_dot(q[r], k[c]) / math.sqrt(d) for c in kept]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = sum(w)
        out.append([sum(w[t] * float(v[c][e]) for t, c in enumerate(kept)) / tot for e in range(len(v[0]))])
        lses.append(mx + math.log(tot))
    return out, lses


def sparge_blocks(q, k, pool, theta, tau, tau_mode="mass"):
    """SpargeAttn stage-one mask for one head by explicit loops: pairwise
    cosine similarities, explicit block means, a softmax over the compressed
    key blocks, then a greedy pick of the most probable blocks."""
    L, d = len(q), len(q[0])
    nb = (L + pool - 1) // pool

    def blk(x, b):
        return x[b * pool:min(L, (b + 1) * pool)]

    def sim(rows):
        n = len(rows)
        tot = 0.0
        for a in rows:
            for c in rows:
                na = math.sqrt(sum(float(t) * float(t) for t in a))
                nc = math.sqrt(sum(float(t) * float(t) for t in c))
                if na > 0 and nc > 0:
                    tot += _dot(a, c) / (na * nc)
        return tot / (n * n)

    def mean(rows):
        return [sum(float(x[e]) for x in rows) / len(rows) for e in range(d)]

    simk = [sim(blk(k, c)) for c in range(nb)]
    res = []
    for b in range(nb):
        if sim(blk(q, b)) <= theta:
            res.append(list(range(b + 1)))
            continue
        comp = [c for c in range(b + 1) if simk[c] > theta]
        keep = [c for c in range(b + 1) if simk[c] <= theta]
        if comp:
            qb = mean(blk(q, b))
            sc = {c: _dot(qb, mean(blk(k, c))) / math.sqrt(d) for c in comp}
            mx = max(sc.values())
            w = {c: math.exp(sc[c] - mx) for c in comp}
            tot = sum(w.values())
            left = list(comp)
            picked, acc = [], 0.0
            want = math.ceil(tau * len(comp)) if tau_mode == "count" else None
            while left:
                if want is not None and len(picked) == want:
                    break
                if want is None and acc >= tau:
                    break
                best = left[0]
                for c in left:
                    if w[c] > w[best]:
                        best = c
                left.remove(best)
                picked.append(best)
                acc += w[best] / tot
            keep += picked
        res.append(sorted(keep))
    return res


def vertical_slash(q, k, last_q, n_vertical, n_slash, pool):
    """Vertical-slash estimate and tile cover for one head by explicit loops:
    the attention rows of the last queries, column and diagonal sums, greedy
    picks, then every allowed entry (r, j) on a chosen line marks its tile."""
    L, d = len(q), len(q[0])
    v = [0.0] * L
    s = [0.0] * L
    for p in range(L - last_q, L):
        sc = [_dot(q[p], k[j]) / math.sqrt(d) for j in range(p + 1)]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        tot = sum(w)
        for j in range(p + 1):
            v[j] += w[j] / tot
            s[p - j] += w[j] / tot

    def pick(x, n):
        left, out = list(range(L)), []
        while left and len(out) < n:
            best = left[0]
            for i in left:
                if x[i] > x[best]:
                    best = i
            left.remove(best)
            out.append(best)
        return set(out)

    vs, ss = pick(v, n_vertical), pick(s, n_slash)
    nb = (L + pool - 1) // pool
    tiles = [set() for _ in range(nb)]
    for r in range(L):
        for j in range(r + 1):
            if j in vs or (r - j) in ss:
                tiles[r // pool].add(j // pool)
    return [sorted(t) for t in tiles], sorted(vs), sorted(ss), v, s
