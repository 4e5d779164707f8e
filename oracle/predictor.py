"""Pooled-Q / pooled-K tile-mask predictor by its plain definition (test
infrastructure only).

The FG-Attn abstract ("FG-Attn: Leveraging Fine-Grained Sparse Attention in
Video Diffusion Models", section Abstract) takes the tile mask as given; the
predictor that produces one is the pooled-score thresholding recipe of this
library's mask-prediction call:

  * Qbar_i = mean of the rows of query tile i, Kbar_j = mean of the keys of
    key tile j (valid rows only, so a partial last tile averages fewer rows);
  * s_ij = Qbar_i . Kbar_j;
  * row i keeps the k largest s_ij, k = T_k - 1 - floor(p * (T_k - 1) / 100)
    for sparsity p percent: with distinct scores these are exactly the tiles
    strictly above numpy's linear-interpolated p-th percentile of the row;
  * equal scores are ordered by ascending j (a stable sort of -s).
"""
from __future__ import annotations

import numpy as np

from .sparse_attention import _f64


def topk_count(T_k: int, sparsity_percent: int) -> int:
    return T_k - 1 - (int(sparsity_percent) * (T_k - 1)) // 100


def _pool(x: np.ndarray, size: int) -> np.ndarray:
    """Mean of each run of `size` consecutive rows (the last run may be shorter)."""
    L = x.shape[0]
    T = -(-L // size)
    out = np.empty((T, x.shape[1]))
    for t in range(T):
        out[t] = x[t * size:min(t * size + size, L)].mean(axis=0)
    return out


def pooled_scores(q_bh, k_bh, M: int, N: int, rows=None) -> np.ndarray:
    """s[i, j] = mean(Q rows of tile i) . mean(K rows of tile j) for one (b, h)."""
    q_bh, k_bh = _f64(q_bh), _f64(k_bh)
    qb = _pool(q_bh, M)
    kb = _pool(k_bh, N)
    if rows is not None:
        qb = qb[np.asarray(rows)]
    return qb @ kb.T


def _pack(keep: np.ndarray) -> np.ndarray:
    T_k = keep.shape[-1]
    nw = -(-T_k // 32)
    out = np.zeros(keep.shape[:-1] + (nw,), dtype=np.uint64)
    for j in range(T_k):
        out[..., j // 32] |= keep[..., j].astype(np.uint64) << np.uint64(j % 32)
    return out.astype(np.uint32)


def predict_keep(scores: np.ndarray, sparsity_percent: int) -> np.ndarray:
    """bool [R, T_k]: top-k of each row, ties to the smaller key-tile index."""
    R, T_k = scores.shape
    k = topk_count(T_k, sparsity_percent)
    keep = np.zeros((R, T_k), dtype=bool)
    for r in range(R):
        order = np.argsort(-scores[r], kind="stable")
        keep[r, order[:k]] = True
    return keep


def predict_mask(q, k, M: int, N: int, sparsity_percent: int, tiles=None):
    """q, k: [B, H, L, d] -> uint32 bitmap [B, H, T_q, words] (or, with `tiles`
    given as [B, H, n], only those query-tile rows: [B, H, n, words])."""
    q, k = _f64(q), _f64(k)
    B, H, L, _ = q.shape
    out = []
    for b in range(B):
        for h in range(H):
            rows = None if tiles is None else np.asarray(tiles)[b, h]
            s = pooled_scores(q[b, h], k[b, h], M, N, rows=rows)
            out.append(_pack(predict_keep(s, sparsity_percent)))
    return np.stack(out).reshape(B, H, -1, out[0].shape[-1])
