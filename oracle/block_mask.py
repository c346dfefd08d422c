"""fp64 oracle for the pooled-score block mask (block-sparse prefill).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition (MInference page, block-sparse pattern: mean-pool Q and K over
blocks and use the fact that pooling commutes with the matrix product to
score whole blocks, then run block-sparse FlashAttention over the chosen
blocks; its ``block_sparse_attention(q, k, v, topk=64)`` call; NOSA page,
section 3: keep ``init_blocks=1`` leading block(s) and a ``window_size=1024``
token local window besides the top-k):

* q_bar[b] = mean of the query rows of block b (``pool`` tokens; the last
  block may be short), k_bar[c] likewise for keys.
* score[b, c] = q_bar[b] . k_bar[c] / sqrt(d) for causal candidates c <= b.
* kept(b) = top-``topk`` candidates by score (ties: lower c first)
  union {0 .. sink_blocks-1} union {b - W + 1 .. b} with
  W = ceil(window_tokens / pool), restricted to 0 <= c <= b, listed in
  ascending order.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _widen


def pool_blocks(x, pool: int, bits: bool = False) -> np.ndarray:
    """Mean over consecutive blocks of ``pool`` rows along axis -2 (fp64)."""
    x = _widen(x, bits)
    L = x.shape[-2]
    nb = math.ceil(L / pool)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]))
    for blk in range(nb):
        out[..., blk, :] = x[..., blk * pool:min(L, (blk + 1) * pool), :].mean(axis=-2)
    return out


def block_scores(q, k, pool: int, bits: bool = False) -> np.ndarray:
    """Pooled block scores [..., nB, nB] = q_bar k_bar^T / sqrt(d); entries
    above the diagonal (c > b) are -inf."""
    qb = pool_blocks(q, pool, bits)
    kb = pool_blocks(k, pool, bits)
    d = qb.shape[-1]
    s = (qb @ np.swapaxes(kb, -1, -2)) / math.sqrt(d)
    nb = s.shape[-1]
    s[..., np.triu_indices(nb, 1)[0], np.triu_indices(nb, 1)[1]] = -np.inf
    return s


def compress_keys(k, kernel: int, stride: int, bits: bool = False) -> np.ndarray:
    """Overlapping mean compression of the keys (NOSA page, section 1, the
    CompressK module: a sliding window of kernel_size=32 tokens moved by
    stride=16, each window averaged into one compressed key). Window m
    averages keys [m*stride, min(L, m*stride + kernel)); windows start at
    every multiple of stride below L (the last ones may be short)."""
    k = _widen(k, bits)
    L = k.shape[-2]
    nw = math.ceil(L / stride)
    out = np.empty(k.shape[:-2] + (nw, k.shape[-1]))
    for m in range(nw):
        out[..., m, :] = k[..., m * stride:min(L, m * stride + kernel), :].mean(axis=-2)
    return out


def block_scores_compressed(q, k, pool: int, kernel: int, stride: int,
                            bits: bool = False) -> np.ndarray:
    """Block scores from overlapping compressed keys (NOSA page, sections 1
    and 3: attention over the compressed keys picks the candidate blocks).
    Reading: key block c (pool tokens) is represented by the compressed
    windows that start inside it, m in [c*pool/stride, (c+1)*pool/stride),
    and its score against query block b is the best of them:
    score[b, c] = max_m q_bar[b] . k_tilde[m] / sqrt(d), for c <= b (-inf
    above the diagonal). With kernel = stride = pool this is block_scores."""
    if pool % stride:
        raise ValueError("stride must divide pool")
    qb = pool_blocks(q, pool, bits)
    kt = compress_keys(k, kernel, stride, bits)
    d = qb.shape[-1]
    s = (qb @ np.swapaxes(kt, -1, -2)) / math.sqrt(d)  # [..., nB, nW]
    nb, nw = qb.shape[-2], kt.shape[-2]
    per = pool // stride
    out = np.full(qb.shape[:-2] + (nb, nb), -np.inf)
    for c in range(nb):
        out[..., c] = s[..., c * per:min(nw, (c + 1) * per)].max(axis=-1)
    out[..., np.triu_indices(nb, 1)[0], np.triu_indices(nb, 1)[1]] = -np.inf
    return out


def block_mask(q, k, pool: int, topk: int, sink_blocks: int, window_tokens: int,
               bits: bool = False, scores=None) -> dict:
    """Kept key blocks per query block. q, k [B,H,L,d]. Returns block_idx
    [B,H,nB,max_blocks] (ascending, padded with -1), block_cnt [B,H,nB],
    the scores, and the score of the topk-th candidate per row (``kth``),
    which tests use to locate near-ties."""
    if scores is None:
        scores = block_scores(q, k, pool, bits)
    B, H, nb, _ = scores.shape
    W = math.ceil(window_tokens / pool) if window_tokens > 0 else 0
    max_blocks = min(nb, topk + sink_blocks + W)
    idx = np.full((B, H, nb, max_blocks), -1, np.int64)
    cnt = np.zeros((B, H, nb), np.int64)
    kth = np.full((B, H, nb), -np.inf)
    for b_ in range(B):
        for h in range(H):
            for qb in range(nb):
                cand = scores[b_, h, qb, :qb + 1]
                order = np.argsort(-cand, kind="stable")
                top = order[:topk]
                if len(order) > topk:
                    kth[b_, h, qb] = cand[order[topk - 1]] if topk > 0 else np.inf
                keep = set(int(c) for c in top)
                keep.update(c for c in range(min(sink_blocks, qb + 1)))
                keep.update(c for c in range(max(0, qb - W + 1), qb + 1))
                kept = sorted(keep)
                cnt[b_, h, qb] = len(kept)
                idx[b_, h, qb, :len(kept)] = kept
    return {"block_idx": idx, "block_cnt": cnt, "scores": scores, "kth": kth,
            "max_blocks": max_blocks}


def block_self_similarity(x, pool: int, bits: bool = False) -> np.ndarray:
    """Mean cosine similarity of the tokens of each block (SpargeAttn page,
    stage one: blocks whose tokens are similar enough are compressed to one
    mean token). Read as the mean over ALL ordered token pairs (i, j) of the
    block, self pairs included: sim = || mean_i x_i / |x_i| ||^2. A zero row
    counts as a zero vector."""
    x = _widen(x, bits)
    L = x.shape[-2]
    nb = math.ceil(L / pool)
    out = np.empty(x.shape[:-2] + (nb,))
    for blk in range(nb):
        xb = x[..., blk * pool:min(L, (blk + 1) * pool), :]
        nrm = np.linalg.norm(xb, axis=-1, keepdims=True)
        xh = np.where(nrm > 0, xb / np.where(nrm > 0, nrm, 1.0), 0.0)
        mean = xh.mean(axis=-2)
        out[..., blk] = (mean * mean).sum(axis=-1)
    return out


def sparge_mask(q, k, pool: int, theta: float, tau: float, tau_mode: str = "mass",
                bits: bool = False) -> dict:
    """SpargeAttn stage-one mask (SpargeAttn page, two-stage online filter,
    stage one "sparse block online prediction"), causal. Readings:

    * a query or key block is *compressed* when its self-similarity
      (``block_self_similarity``) is above theta; it is then represented by
      its mean token;
    * the compressed map of query block b is P_hat[b, c] =
      softmax over the compressed key blocks c <= b of
      q_bar[b] . k_bar[c] / sqrt(d); uncompressed key blocks have no token,
      take no part in the softmax and are always computed;
    * Top-tau selection over the compressed candidates, ranked by P_hat
      (ties: lower c first): ``tau_mode="mass"`` keeps the smallest top set
      whose P_hat mass reaches tau; ``tau_mode="count"`` keeps the
      ceil(tau * n) best of the n compressed candidates (ceil in fp64);
    * an uncompressed query block keeps every causal block;
    * lists are ascending.

    Returns block_idx [B,H,nB,nB] (-1 padded), block_cnt, P_hat (0 outside
    the compressed candidates), sim_q, sim_k and, per row, what decides the
    cut for near-tie tests: ``mass_before`` / ``mass_at`` (the mass before and
    after the last kept block, mass mode) and ``score_gap`` (score of the last
    kept minus that of the first dropped candidate, inf when none drops)."""
    if tau_mode not in ("mass", "count"):
        raise ValueError(tau_mode)
    scores = block_scores(q, k, pool, bits)
    sim_q = block_self_similarity(q, pool, bits)
    sim_k = block_self_similarity(k, pool, bits)
    B, H, nb, _ = scores.shape
    idx = np.full((B, H, nb, nb), -1, np.int64)
    cnt = np.zeros((B, H, nb), np.int64)
    phat = np.zeros_like(scores)
    mass_before = np.full((B, H, nb), np.nan)
    mass_at = np.full((B, H, nb), np.nan)
    score_gap = np.full((B, H, nb), np.inf)
    for b_ in range(B):
        for h in range(H):
            for qb in range(nb):
                comp = [c for c in range(qb + 1) if sim_k[b_, h, c] > theta]
                keep = set(c for c in range(qb + 1) if sim_k[b_, h, c] <= theta)
                if sim_q[b_, h, qb] <= theta:
                    keep = set(range(qb + 1))
                elif comp:
                    row = scores[b_, h, qb, comp]
                    p = np.exp(row - row.max())
                    p /= p.sum()
                    phat[b_, h, qb, comp] = p
                    order = sorted(range(len(comp)), key=lambda j: (-p[j], comp[j]))
                    if tau_mode == "count":
                        n_keep = math.ceil(tau * len(comp))
                    else:
                        acc, n_keep = 0.0, 0
                        for j in order:
                            if acc >= tau:
                                break
                            mass_before[b_, h, qb] = acc
                            acc += p[j]
                            n_keep += 1
                        mass_at[b_, h, qb] = acc
                    keep.update(comp[j] for j in order[:n_keep])
                    if 0 < n_keep < len(comp):
                        score_gap[b_, h, qb] = row[order[n_keep - 1]] - row[order[n_keep]]
                kept = sorted(keep)
                cnt[b_, h, qb] = len(kept)
                idx[b_, h, qb, :len(kept)] = kept
    return {"block_idx": idx, "block_cnt": cnt, "phat": phat, "sim_q": sim_q, "sim_k": sim_k,
            "mass_before": mass_before, "mass_at": mass_at, "score_gap": score_gap}
