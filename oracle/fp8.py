"""FP8 (e4m3) quantisation of Q and K with per-tile scales, by definition
(test infrastructure only).

The pages define tile-sparse attention in no particular precision.  The FP8
variant of the path reads Q and K as 8-bit floats: each value is the
e4m3 number nearest (ties to even) to x / s, where s is the scale of the
value's tile, and the attention then uses x ~ e4m3 * s.  Readings:
  * e4m3 is the OCP 8-bit format with 4 exponent bits (bias 7), 3 mantissa
    bits, subnormals, largest finite value 448 and no infinities;
  * Q has one scale per 16-row tile of a (b, h) and K one scale per (b, h);
    a scale is (largest |x| of its tile) / 448 computed in float32, or 1 for
    an all-zero tile, so the largest value of every tile maps to 448;
  * x / s is computed in float32, then rounded to e4m3.
The attention of the quantised inputs is the plain definition applied to the
dequantised values (sparse_attention.attention), V staying in its own type.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
Q_TILE_ROWS = 16


def round_e4m3(x) -> np.ndarray:
    """float32 values -> the nearest e4m3 values (float64), ties to even.
    Magnitudes of 464 and above have no e4m3 neighbour and give NaN."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    # exponent of the binade (normal numbers from 2^-6); below it the spacing is 2^-9
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    quantum = np.exp2(e - 3)
    r = np.round(a / quantum) * quantum          # np.round: half to even; a / quantum is exact
    r = np.where(a >= 464.0, np.nan, np.minimum(r, E4M3_MAX))
    return np.copysign(r, x)


def tile_scales(x, rows: int) -> np.ndarray:
    """float32 scales of consecutive `rows`-row tiles along axis -2 of
    x [..., L, d]: max |x| over the tile (rows past L absent) / 448."""
    x = np.asarray(x, dtype=np.float32)
    L = x.shape[-2]
    n = -(-L // rows)
    out = np.empty(x.shape[:-2] + (n,), dtype=np.float32)
    for t in range(n):
        amax = np.abs(x[..., t * rows:min(L, t * rows + rows), :]).max(axis=(-2, -1))
        out[..., t] = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0))
    return out


def quantize(x, rows: int):
    """(e4m3 values float64 [..., L, d], float32 scales [..., ceil(L/rows)])."""
    x = np.asarray(x, dtype=np.float32)
    s = tile_scales(x, rows)
    s_rows = np.repeat(s, rows, axis=-1)[..., :x.shape[-2]]
    return round_e4m3(x / s_rows[..., None]), s


def dequantize(values, scales, rows: int) -> np.ndarray:
    values = np.asarray(values, dtype=np.float64)
    s_rows = np.repeat(np.asarray(scales, dtype=np.float64), rows, axis=-1)[..., :values.shape[-2]]
    return values * s_rows[..., None]


def quantize_qk(q, k):
    """The FP8 path's inputs: Q per 16-row tile, K per (b, h).
    Returns (q8, q_scale [B, H, ceil(L/16)], k8, k_scale [B, H])."""
    q = np.asarray(q.float().numpy() if hasattr(q, "float") else q, dtype=np.float32)
    k = np.asarray(k.float().numpy() if hasattr(k, "float") else k, dtype=np.float32)
    q8, qs = quantize(q, Q_TILE_ROWS)
    k8, ks = quantize(k, k.shape[-2])
    return q8, qs, k8, ks[..., 0]
