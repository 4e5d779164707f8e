"""Tile-sparse softmax attention, backward, by its plain definition (float64).

Test infrastructure only (see the package docstring).

The pages define only the forward pass: "FG-Attn: Leveraging Fine-Grained
Sparse Attention in Video Diffusion Models", section Abstract, skips the
scores of whole M x N tiles, and skipped scores take no part in the softmax.
The gradients here are the derivative of exactly that forward (the one in
sparse_attention.py) with respect to Q, K and V, for an upstream gradient dO
of the output.  Writing the forward as S = scale Q K^T, P = softmax of the
kept entries of each row of S (skipped entries 0), O = P V, the chain rule
gives, row by row:

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - D),   D[r] = sum_c P[r,c] dP[r,c]   (elementwise product)
    dQ = scale dS K,     dK = scale dS^T Q

Skipped entries have P = 0, so their dS is 0 whatever dP is; a row with no
kept key has P = 0 everywhere and contributes nothing.  D is computed here
as the row sum of P * dP, its definition.  (It equals the row sum of
dO * O; the GPU library uses that form, and the tests check the two agree.)
"""
from __future__ import annotations

import numpy as np

from .sparse_attention import _f64, keep_matrix, tile_rows


def _probs(s: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """Row softmax of s over the kept entries; skipped entries and empty rows give 0."""
    s = np.where(keep, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    p = np.exp(s - np.where(empty, 0.0, m)[:, None])      # exp(-inf) = 0
    l = p.sum(axis=1)
    p /= np.where(empty, 1.0, l)[:, None]
    p[empty] = 0.0
    return p


def _head_bwd(q, k, v, do, keep, sc):
    """Gradients of one (b, h) with the full keep matrix [L, L]."""
    p = _probs(sc * (q @ k.T), keep)
    dv = p.T @ do
    dp = do @ v.T
    dsum = (p * dp).sum(axis=1)
    ds = p * (dp - dsum[:, None])
    dq = sc * (ds @ k)
    dk = sc * (ds.T @ q)
    return dq, dk, dv


def attention_bwd(q, k, v, do, mask_bits, M: int, N: int, scale: float):
    """Gradients of the tile-sparse attention output with respect to q, k, v.

    q, k, v, do: [B, H, L, d]; mask_bits: uint32 [B, H, ceil(L/M), words].
    Returns (dQ, dK, dV), float64 [B, H, L, d] each.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, L, d = q.shape
    sc = float(np.float32(scale))
    mask_bits = np.asarray(mask_bits)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            keep = keep_matrix(mask_bits[b, h], L, M, N)
            dq[b, h], dk[b, h], dv[b, h] = _head_bwd(q[b, h], k[b, h], v[b, h], do[b, h], keep, sc)
    return dq, dk, dv


def attention_bwd_rows(q_bh, k_bh, v_bh, do_bh, mask_bits_bh, M: int, N: int, scale: float,
                       q_tiles=None, k_rows=None, group: int = 1024):
    """Selected gradient rows of one (b, h), for sequences too long for L x L.

    dQ rows of the query tiles `q_tiles` (all their rows, clipped to L) and dK,
    dV rows of the key rows `k_rows`.  q_bh, k_bh, v_bh, do_bh: [L, d];
    mask_bits_bh: uint32 [T_q, words].  Returns (q_rows, dQ [nq, d], k_rows,
    dK [nk, d], dV [nk, d]) in float64.  dK and dV are sums over every query
    row; they are accumulated `group` query rows at a time to bound memory,
    which changes only the order of that float64 sum.
    """
    q_bh, k_bh, v_bh, do_bh = _f64(q_bh), _f64(k_bh), _f64(v_bh), _f64(do_bh)
    L, d = q_bh.shape
    sc = float(np.float32(scale))
    q_rows = tile_rows(L, M, q_tiles) if q_tiles is not None else np.zeros(0, dtype=np.int64)
    k_rows = np.asarray(k_rows if k_rows is not None else [], dtype=np.int64)

    dq = np.zeros((len(q_rows), d))
    for g0 in range(0, len(q_rows), group):
        rows = q_rows[g0:g0 + group]
        keep = keep_matrix(mask_bits_bh, L, M, N, rows=rows)
        p = _probs(sc * (q_bh[rows] @ k_bh.T), keep)
        dp = do_bh[rows] @ v_bh.T
        ds = p * (dp - (p * dp).sum(axis=1)[:, None])
        dq[g0:g0 + len(rows)] = sc * (ds @ k_bh)

    dk = np.zeros((len(k_rows), d))
    dv = np.zeros((len(k_rows), d))
    if len(k_rows):
        for r0 in range(0, L, group):
            rows = np.arange(r0, min(r0 + group, L))
            keep = keep_matrix(mask_bits_bh, L, M, N, rows=rows)
            p = _probs(sc * (q_bh[rows] @ k_bh.T), keep)       # full rows: D needs every key
            dp = do_bh[rows] @ v_bh.T
            dsum = (p * dp).sum(axis=1)
            ps = p[:, k_rows]
            ds = ps * (dp[:, k_rows] - dsum[:, None])
            dk += sc * (ds.T @ q_bh[rows])
            dv += ps.T @ do_bh[rows]
    return q_rows, dq, k_rows, dk, dv
