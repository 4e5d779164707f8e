"""Difference of two tile masks, by its plain definition (test infrastructure only).

FG-Attn ("FG-Attn: Leveraging Fine-Grained Sparse Attention in Video
Diffusion Models", section Abstract) makes one keep decision per M x N tile.
When a mask predicted at one denoising step is reused at later steps, the
quantity that says how far two masks are apart is the number of tiles whose
decision differs.  Per bitmap row (b, h, i) that is the count of key tiles
j < T_k whose keep bit differs between the two masks (padding bits past T_k
are not decisions and are ignored); per head it is the sum over the head's
rows.
"""
from __future__ import annotations

import numpy as np

from .sparse_attention import unpack_mask


def mask_diff(a_bits, b_bits, T_k: int):
    """(per-row counts int64 [B, H, T_q], per-head counts int64 [B, H]) of
    differing keep decisions between two uint32 bitmaps [B, H, T_q, words]."""
    a = unpack_mask(np.asarray(a_bits), T_k)
    b = unpack_mask(np.asarray(b_bits), T_k)
    rows = (a != b).sum(axis=-1).astype(np.int64)
    return rows, rows.sum(axis=-1)
