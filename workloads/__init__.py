"""Seeded synthetic workloads for tile-sparse attention.

This package produces inputs only: Q/K/V tensors, keep-bitmaps and the
sampled query tiles used for parity checks.  It holds none of the attention
arithmetic, so both the GPU path and the CPU oracle can be fed from it
without sharing any of the method's code.
"""
from .gen import (  # noqa: F401
    Workload, MaskRecipe, CONFIGS, HEADLINE, get, splitmix64, pack_bits,
    mask_bits, mask_rows_bool, make_qkv, make_do, sample_tiles, row_words, diag_tiles,
    frame_thresholds, hash_params, prob_threshold, structured_params,
)
