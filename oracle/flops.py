"""Kept-tile FLOP count (test infrastructure only).

Two matrix products per kept tile (S = Q K^T on the tile, then P V), each
2 FLOP per multiply-add, over the tile's real extent: 4 * d * m_i * n_j with
m_i = min(M, L - i*M) and n_j = min(N, L - j*N).  Softmax work is not counted.
"""
from __future__ import annotations

import numpy as np

from .sparse_attention import unpack_mask


def kept_flops(mask_bits, L: int, M: int, N: int, d: int) -> int:
    mask_bits = np.asarray(mask_bits)
    T_q, T_k = -(-L // M), -(-L // N)
    m = np.minimum(M, L - np.arange(T_q) * M).astype(np.int64)
    n = np.minimum(N, L - np.arange(T_k) * N).astype(np.int64)
    total = 0
    flat = mask_bits.reshape(-1, T_q, mask_bits.shape[-1])
    for head in flat:
        keep = unpack_mask(head, T_k)
        total += int((m[:, None] * keep * n[None, :]).sum())
    return 4 * d * total
