"""Mask compaction by its plain definition (test infrastructure only).

FG-Attn ("FG-Attn: Leveraging Fine-Grained Sparse Attention in Video Diffusion
Models", section Abstract) decides per M x N tile whether its scores are
computed.  Compaction turns one query tile's row of keep bits into the
ascending list of kept key tiles, i.e. the indices whose bit is 1.

Output is CSR over rows ordered (b, h, i) row-major: row_ptr int64
[B*H*T_q + 1], col_idx int32 [nnz] holding key-tile indices j < T_k.
"""
from __future__ import annotations

import numpy as np

from .sparse_attention import unpack_mask


def compact(mask_bits, T_k: int):
    """uint32 [B, H, T_q, words] -> (row_ptr int64, col_idx int32)."""
    mask_bits = np.asarray(mask_bits)
    rows = unpack_mask(mask_bits.reshape(-1, mask_bits.shape[-1]), T_k)   # [R, T_k]
    lists = [np.flatnonzero(r) for r in rows]
    counts = np.array([len(x) for x in lists], dtype=np.int64)
    row_ptr = np.zeros(len(lists) + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = (np.concatenate(lists) if lists else np.zeros(0)).astype(np.int32)
    return row_ptr, col_idx
