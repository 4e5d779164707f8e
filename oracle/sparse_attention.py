"""Tile-sparse softmax attention, forward, by its plain definition (float64).

Test infrastructure only (see the package docstring).

Definition followed (FG-Attn abstract, "FG-Attn: Leveraging Fine-Grained
Sparse Attention in Video Diffusion Models", section Abstract): the score
matrix S = scale * Q K^T is partitioned into tiles of M queries by N keys;
a tile whose mask bit is 0 has its scores skipped.  Skipped scores take no
part in the softmax, which is the same as setting them to -inf.  Then
P = softmax(S) row by row and O = P V.

Readings where the page is silent:
  * bit = 1 keeps a tile; bitmap words are uint32, LSB first, row-major
    [B][H][T_q][words]; padding bits past T_k are ignored.
  * the last query / key tile may be partial; rows and keys past L do not exist.
  * a row with no kept key gives O = 0 and LSE = -inf.
  * `scale` is the float32 value the caller passes, widened to float64.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):          # a torch tensor (possibly bf16): exact widening
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def unpack_mask(bits, T_k: int) -> np.ndarray:
    """uint32 words [..., words] -> bool [..., T_k]: bit (j % 32) of word j // 32."""
    bits = np.asarray(bits, dtype=np.uint64)
    j = np.arange(T_k)
    words = bits[..., j // 32]
    return ((words >> (j % 32).astype(np.uint64)) & np.uint64(1)).astype(bool)


def keep_matrix(mask_bits_head, L: int, M: int, N: int, rows=None) -> np.ndarray:
    """Per-score keep flags for one (b, h): keep[r, c] = bit(floor(r/M), floor(c/N)).

    mask_bits_head: uint32 [T_q, words].  rows: query rows to expand (default all).
    """
    T_k = -(-L // N)
    r = np.arange(L) if rows is None else np.asarray(rows)
    c = np.arange(L)
    # only the bitmap rows of the requested query rows are unpacked
    tiles = unpack_mask(np.asarray(mask_bits_head)[r // M], T_k)   # [len(r), T_k]
    return tiles[:, c // N]


def _softmax_pv(s: np.ndarray, keep: np.ndarray, v: np.ndarray):
    """Rows of softmax(s with skipped entries at -inf) @ v; empty rows -> 0, lse -inf."""
    s = np.where(keep, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])                        # exp(-inf) = 0 for skipped scores
    l = p.sum(axis=1)
    o = (p @ v) / np.where(empty, 1.0, l)[:, None]
    o[empty] = 0.0
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return o, lse


def attention(q, k, v, mask_bits, M: int, N: int, scale: float):
    """Full tile-sparse attention.

    q, k, v: [B, H, L, d]; mask_bits: uint32 [B, H, ceil(L/M), words].
    Returns (O float64 [B, H, L, d], LSE float64 [B, H, L]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, d = q.shape
    sc = float(np.float32(scale))
    mask_bits = np.asarray(mask_bits)
    o = np.zeros((B, H, L, d))
    lse = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            s = sc * (q[b, h] @ k[b, h].T)                 # [L, L]
            keep = keep_matrix(mask_bits[b, h], L, M, N)
            o[b, h], lse[b, h] = _softmax_pv(s, keep, v[b, h])
    return o, lse


def tile_rows(L: int, M: int, tiles) -> np.ndarray:
    """Query rows of the given query tiles, in tile order, clipped to L."""
    rows = [np.arange(t * M, min(t * M + M, L)) for t in np.asarray(tiles).ravel()]
    return np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)


def attention_rows(q_bh, k_bh, v_bh, mask_bits_bh, M: int, N: int, scale: float, tiles,
                   group: int = 32):
    """Tile-sparse attention for selected query tiles of one (b, h).

    q_bh, k_bh, v_bh: [L, d]; mask_bits_bh: uint32 [T_q, words].
    Returns (rows, O rows float64 [n, d], LSE float64 [n]).  Output rows are
    independent of each other by definition, so they are evaluated `group`
    tiles at a time only to bound memory; no arithmetic is reordered.
    """
    q_bh, k_bh, v_bh = _f64(q_bh), _f64(k_bh), _f64(v_bh)
    L = k_bh.shape[0]
    sc = float(np.float32(scale))
    tiles = np.asarray(tiles).ravel()
    rows_all, o_all, lse_all = [], [], []
    for g0 in range(0, len(tiles), group):
        rows = tile_rows(L, M, tiles[g0:g0 + group])
        s = sc * (q_bh[rows] @ k_bh.T)
        keep = keep_matrix(mask_bits_bh, L, M, N, rows=rows)
        o, lse = _softmax_pv(s, keep, v_bh)
        rows_all.append(rows)
        o_all.append(o)
        lse_all.append(lse)
    return np.concatenate(rows_all), np.concatenate(o_all), np.concatenate(lse_all)
