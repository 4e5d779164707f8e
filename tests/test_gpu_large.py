"""Attention parity at the full benchmark shapes, on sampled query tiles.

Inputs are the seeded workload tensors at their real size; the GPU computes
every row, the oracle the sampled query tiles (tile 0, the last, partial
tile, and 254 random ones per head) of every head for the headline 16x8
workload and of a spread of heads for the others (all heads with
TSA_PARITY_ALL_HEADS=1).  Oracle inputs never come from the GPU: masks of
the sampled rows come from the host generators (the GPU generator's rows are
checked equal to them first) or, for the predicted mask, from the oracle's
own predictor.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import mask_to_np, sampled_compare, say, to_dev_mask, torch_or_skip
from oracle import predictor as opred

pytestmark = pytest.mark.gpu


# The headline workload (16x8 tiles at 70% sparsity) is checked on every head.
# The others take a spread of four heads to bound the fp64 oracle's time: at
# 256 sampled tiles per head one head costs 6.9e10 (wan480), 1.6e11 (wan720)
# and 2.4e11 (hunyuan720) dense fp64 FLOPs.
ALL_HEADS = {"wan480_fine"}


def _heads(w):
    if w.name in ALL_HEADS or os.environ.get("TSA_PARITY_ALL_HEADS") == "1":
        return list(range(w.H))
    return sorted({0, w.H // 3, w.H // 2, w.H - 1})


def _attn(w, q, k, v, mask_dev):
    import torch

    import tile_sparse_attention_amd as T
    o, lse = T.attention_fwd(q, k, v, mask_dev, w.M, w.N, w.scale, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def _head_bits_from_rows(w, h, tiles):
    """Bitmap [T_q, words] of head h holding the host generator's rows for
    `tiles` (other rows are never read by the oracle)."""
    out = np.zeros((w.T_q, w.words), dtype=np.uint32)
    out[tiles] = W.pack_bits(W.mask_rows_bool(w, [(0, h, int(i)) for i in tiles]))
    return out


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["wan480_fine", "wan720_n1", "wan480_struct"])
def test_hash_mask_configs(name):
    torch_or_skip()
    import tile_sparse_attention_amd as T
    w = W.get(name)
    say(f"large {name}: generating inputs")
    q, k, v = W.make_qkv(w)
    if w.mask.kind == "structured":
        mask = T.maskgen_structured(w.B, w.H, w.L, w.M, w.N, **W.structured_params(w))
    else:
        mask = T.maskgen_hash(w.B, w.H, w.L, w.M, w.N, **W.hash_params(w))
    say(f"large {name}: attention on GPU")
    o, lse = _attn(w, q.cuda(), k.cuda(), v.cuda(), mask)
    tiles = W.sample_tiles(w)
    heads = _heads(w)
    if w.mask.kind == "structured":  # one head of every pattern, skipped heads included
        heads = sorted(set(heads) | {w.mask.patterns.index(t) for t in set(w.mask.patterns)})
    bits_cache = {}
    mnp = mask_to_np(mask)
    for h in heads:
        bits_cache[h] = _head_bits_from_rows(w, h, tiles[0, h])
        assert np.array_equal(mnp[0, h, tiles[0, h]], bits_cache[h][tiles[0, h]])
    say(f"large {name}: oracle on {len(heads)} heads x {tiles.shape[2]} tiles")
    sampled_compare(w, q, k, v, o, lse, lambda b, h: bits_cache[h], tiles, heads, name)


def test_exact_drop_config():
    torch_or_skip()
    w = W.get("wan480_coarse")
    say("large wan480_coarse: generating inputs")
    q, k, v = W.make_qkv(w)
    bits = W.mask_bits(w)
    o, lse = _attn(w, q.cuda(), k.cuda(), v.cuda(), to_dev_mask(bits))
    tiles = W.sample_tiles(w)
    heads = _heads(w)
    say(f"large wan480_coarse: oracle on {len(heads)} heads")
    sampled_compare(w, q, k, v, o, lse, lambda b, h: bits[b, h], tiles, heads, "wan480_coarse")


def test_predicted_mask_config():
    """Predictor on the GPU, then attention on a bitmap whose sampled rows are
    the oracle predictor's rows, so the oracle's mask input is its own."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    w = W.get("hunyuan720")
    say("large hunyuan720: generating inputs")
    q, k, v = W.make_qkv(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mask = T.predict_mask(qd, kd, w.M, w.N, w.mask.sparsity_percent)
    tiles = W.sample_tiles(w)
    heads = _heads(w)
    rows = {}
    for h in heads:
        s = opred.pooled_scores(q[0, h], k[0, h], w.M, w.N, rows=tiles[0, h])
        rows[h] = opred._pack(opred.predict_keep(s, w.mask.sparsity_percent))
        mask[0, h, torch.from_numpy(tiles[0, h]).cuda()] = torch.from_numpy(rows[h].view(np.int32)).cuda()
    o, lse = _attn(w, qd, kd, vd, mask)

    def head_bits(b, h):
        out = np.zeros((w.T_q, w.words), dtype=np.uint32)
        out[tiles[0, h]] = rows[h]
        return out
    say(f"large hunyuan720: oracle on {len(heads)} heads")
    sampled_compare(w, q, k, v, o, lse, head_bits, tiles, heads, "hunyuan720")


@pytest.mark.timeout(600)
def test_long_sequence_past_the_chunk_skip_limit():
    """L = 300007 (2344 key chunks, above the 2048 the chunk-skipping path
    handles, so only the plain kernel runs), 16x8 tiles, i.i.d. 10% keep with
    the diagonal kept: 256 sampled query tiles of both heads, including the
    last, partial one."""
    torch_or_skip()
    w = W.Workload("long", 1, 2, 300007, 128, 16, 8, "bf16",
                   W.MaskRecipe("hash", p_near=0.1, p_far=0.1), 1234)
    say("large L=300007 16x8: generating inputs")
    q, k, v = W.make_qkv(w)
    import tile_sparse_attention_amd as T
    mask = T.maskgen_hash(w.B, w.H, w.L, w.M, w.N, **W.hash_params(w))
    say("large L=300007 16x8: attention on GPU")
    o, lse = _attn(w, q.cuda(), k.cuda(), v.cuda(), mask)
    tiles = W.sample_tiles(w)
    mnp = mask_to_np(mask)
    bits = {}
    for h in range(w.H):
        bits[h] = _head_bits_from_rows(w, h, tiles[0, h])
        assert np.array_equal(mnp[0, h, tiles[0, h]], bits[h][tiles[0, h]])
    say("large L=300007 16x8: oracle on 2 heads x 256 tiles")
    sampled_compare(w, q, k, v, o, lse, lambda b, h: bits[h], tiles, list(range(w.H)), "long L=300007")
