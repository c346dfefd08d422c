"""fp64 oracle for the vertical-slash block estimator.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition (MInference page: of its three patterns, vertical-slash is
estimated by attending from the last query vector(s) to every key, which
gives the best vertical lines (key columns) and slash lines (diagonals);
its ``vertical_slash_sparse_attention(q, k, v, vertical_topk=32, slash=0.2)``
call). Readings:

* the last ``last_q`` query rows i (positions p_i = L - last_q + i) attend
  causally: A[i, j] = softmax over j <= p_i of q_i . k_j / sqrt(d);
  ``last_q = 1`` is the page's single last query;
* vertical score v[j] = sum_i A[i, j]; slash score s[o] = sum_i A[i, p_i - o]
  over the rows with p_i - o >= 0 (o = 0 is the main diagonal);
* the top ``n_vertical`` keys by v and the top ``n_slash`` offsets by s are
  chosen (ties: lower index first; a count at or above L takes all);
* the attention that follows runs on blocks of ``pool`` x ``pool`` tiles:
  tile (b, c), c <= b, is kept iff it holds an allowed entry (r, j), j <= r,
  with j a chosen vertical or r - j a chosen slash. For rows r in
  [r_lo, r_hi] and keys j in [j_lo, j_hi] this is: a chosen vertical lies in
  [j_lo, j_hi] (every key of a tile c <= b precedes the tile's last row), or a
  chosen slash lies in [max(0, r_lo - j_hi), r_hi - j_lo].
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _widen


def vertical_slash_scores(q, k, last_q: int, bits: bool = False):
    """(v, s) for one or more heads: q, k [..., L, d] -> v, s [..., L]."""
    q = _widen(q, bits)
    k = _widen(k, bits)
    L, d = q.shape[-2], q.shape[-1]
    if not 1 <= last_q <= L:
        raise ValueError("need 1 <= last_q <= L")
    lead = q.shape[:-2]
    v = np.zeros(lead + (L,))
    s = np.zeros(lead + (L,))
    for idx in np.ndindex(*lead):
        for i in range(last_q):
            p = L - last_q + i
            sc = k[idx][:p + 1] @ q[idx][p] / math.sqrt(d)
            a = np.exp(sc - sc.max())
            a /= a.sum()
            v[idx][:p + 1] += a
            s[idx][:p + 1] += a[::-1]      # offset o = p - j
    return v, s


def top_indices(x: np.ndarray, n: int) -> np.ndarray:
    """Indices of the n largest entries of a 1-D array (ties: lower index
    first), returned in ascending order."""
    order = np.lexsort((np.arange(len(x)), -x))
    return np.sort(order[:min(n, len(x))])


def cover_blocks(verticals, slashes, L: int, pool: int):
    """Block lists (ascending, per query block) of the tiles that hold a
    chosen vertical or slash entry, by the interval rule above."""
    nb = math.ceil(L / pool)
    vflag = np.zeros(L, bool)
    vflag[np.asarray(verticals, np.int64)] = True
    sflag = np.zeros(L, bool)
    sflag[np.asarray(slashes, np.int64)] = True
    lists = []
    for b in range(nb):
        r_lo, r_hi = b * pool, min(L, (b + 1) * pool) - 1
        kept = []
        for c in range(b + 1):
            j_lo, j_hi = c * pool, min(L, (c + 1) * pool) - 1
            if vflag[j_lo:j_hi + 1].any() or sflag[max(0, r_lo - j_hi):r_hi - j_lo + 1].any():
                kept.append(c)
        lists.append(kept)
    return lists


def vertical_slash_mask(q, k, last_q: int, n_vertical: int, n_slash: int, pool: int = 64,
                        bits: bool = False) -> dict:
    """q, k [B,H,L,d]. Returns block_idx [B,H,nB,nB] (-1 padded), block_cnt,
    the chosen vertical / slash indices (ascending) per head, the scores v, s
    and the n-th largest score of each (``v_kth``, ``s_kth``; -inf when
    everything is taken) for near-tie tests."""
    B, H, L, _ = q.shape
    nb = math.ceil(L / pool)
    v, s = vertical_slash_scores(q, k, last_q, bits)
    idx = np.full((B, H, nb, nb), -1, np.int64)
    cnt = np.zeros((B, H, nb), np.int64)
    vert, sl = {}, {}
    v_kth = np.full((B, H), -np.inf)
    s_kth = np.full((B, H), -np.inf)
    for b in range(B):
        for h in range(H):
            vi = top_indices(v[b, h], n_vertical)
            si = top_indices(s[b, h], n_slash)
            vert[(b, h)], sl[(b, h)] = vi, si
            if 0 < n_vertical < L:
                v_kth[b, h] = np.sort(v[b, h])[::-1][n_vertical - 1]
            if 0 < n_slash < L:
                s_kth[b, h] = np.sort(s[b, h])[::-1][n_slash - 1]
            for qb, kept in enumerate(cover_blocks(vi, si, L, pool)):
                cnt[b, h, qb] = len(kept)
                idx[b, h, qb, :len(kept)] = kept
    return {"block_idx": idx, "block_cnt": cnt, "vertical": vert, "slash": sl, "v": v, "s": s,
            "v_kth": v_kth, "s_kth": s_kth}
