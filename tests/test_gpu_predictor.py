"""GPU pooled-Q/pooled-K tile-mask predictor against the CPU oracle.

The GPU scores in fp32 and the oracle in fp64, so decisions may differ only
for scores within a small band around a row's threshold.  Checked per row:
exactly k tiles kept; every tile whose oracle score is above the oracle's
k-th largest score by more than delta is kept, every tile below it by more
than delta is dropped, delta = 1e-4 * max|s| + 1e-6.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import mask_to_np, say, torch_or_skip
from oracle import predictor as opred

pytestmark = pytest.mark.gpu


def _check_rows(gpu_bits, scores, sp):
    T_k = scores.shape[1]
    k = opred.topk_count(T_k, sp)
    keep = oracle.unpack_mask(gpu_bits, T_k)
    assert np.all(keep.sum(axis=1) == k), "wrong number of kept tiles"
    if k == 0:
        return 0
    srt = -np.sort(-scores, axis=1)
    thr = srt[:, k - 1]
    delta = 1e-4 * np.abs(scores).max(axis=1) + 1e-6
    above = scores > (thr + delta)[:, None]
    below = scores < (thr - delta)[:, None]
    assert np.all(keep[above]), "a clearly-above tile was dropped"
    assert not np.any(keep[below]), "a clearly-below tile was kept"
    exact = oracle.unpack_mask(opred._pack(opred.predict_keep(scores, sp)), T_k)
    return int((exact != keep).sum())


def _run(q, k, M, N, sp):
    import tile_sparse_attention_amd as T
    return mask_to_np(T.predict_mask(q.cuda(), k.cuda(), M, N, sp))


@pytest.mark.parametrize("dtype,d,L,M,N,sp", [
    ("bf16", 128, 1000, 16, 16, 85), ("bf16", 128, 777, 16, 8, 70), ("f32", 64, 512, 16, 16, 50),
    ("bf16", 64, 300, 32, 1, 90), ("bf16", 128, 16, 16, 16, 85), ("f32", 128, 2000, 64, 64, 0),
    ("bf16", 128, 4100, 16, 4, 99),
    ("bf16", 64, 9000, 64, 1, 85)])   # 9000 key tiles: rows too long to be held in LDS
def test_predictor_small(dtype, d, L, M, N, sp):
    torch_or_skip()
    w = W.Workload("p", 2, 2, L, d, M, N, dtype, W.MaskRecipe("predicted", sparsity_percent=sp),
                   31 + L, offset_frame_tokens=max(1, L // 5), offset_sigma=0.5)
    say(f"predictor {dtype} d={d} L={L} {M}x{N} sp={sp}")
    q, k, _ = W.make_qkv(w)
    bits = _run(q, k, M, N, sp)
    for b in range(w.B):
        for h in range(w.H):
            s = opred.pooled_scores(q[b, h], k[b, h], M, N)
            _check_rows(bits[b, h], s, sp)


@pytest.mark.parametrize("L,M,N", [(256, 16, 16), (8320, 64, 1)])  # row in LDS / row too long for it
def test_predictor_ties_go_to_smaller_tile(L, M, N):
    torch = torch_or_skip()
    say(f"predictor ties L={L} {M}x{N}")
    d = 64
    g = torch.Generator().manual_seed(L + N)
    q = torch.randn(1, 1, L, d, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 1, N, d, generator=g).repeat(1, 1, L // N, 1).to(torch.bfloat16)   # all key tiles equal
    bits = _run(q, k, M, N, 50)
    keep = oracle.unpack_mask(bits[0, 0], L // N)
    kk = opred.topk_count(L // N, 50)
    assert np.all(keep[:, :kk]) and not np.any(keep[:, kk:])


def test_predictor_hunyuan_sampled_rows():
    """The 24-head, 118800-token shape with per-frame offsets: sampled rows."""
    torch_or_skip()
    w = W.get("hunyuan720").replace(H=4)
    say("predictor hunyuan720 (4 heads) sampled rows")
    q, k, _ = W.make_qkv(w)
    bits = _run(q, k, w.M, w.N, 85)
    tiles = W.sample_tiles(w, per_head=64)
    mism = 0
    for h in range(w.H):
        s = opred.pooled_scores(q[0, h], k[0, h], w.M, w.N, rows=tiles[0, h])
        mism += _check_rows(bits[0, h, tiles[0, h]], s, 85)
    print(f"[predictor] near-threshold decisions differing from fp64: {mism}", flush=True)


@pytest.mark.parametrize("L,M,N,sp", [(4096, 16, 16, 85), (6000, 16, 4, 70)])
def test_predictor_rows_with_a_spike_of_equal_scores(L, M, N, sp):
    """Most key tiles are copies of one tile, so every row holds a run of
    equal scores: where the k-th largest falls in that run the row's bin
    overflows and the row is finished by the exact per-row select, elsewhere
    the run lies clear of the threshold.  Both kinds of rows keep exactly k,
    respect the threshold band, and keep the equal scores of the run in
    ascending j order (ties to the smaller tile)."""
    torch = torch_or_skip()
    say(f"predictor spike L={L} {M}x{N} sp={sp}")
    d = 64
    T_k = L // N
    g = torch.Generator().manual_seed(L + sp)
    q = torch.randn(1, 2, L, d, generator=g)
    k = torch.randn(1, 2, L, d, generator=g)
    copies = torch.rand(T_k, generator=g) < 0.6          # key tiles replaced by tile 0
    kt = k.view(1, 2, T_k, N, d)
    kt[:, :, copies] = kt[:, :, :1]
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    bits = _run(q, k, M, N, sp)
    kk = opred.topk_count(T_k, sp)
    run_rows = 0
    for h in range(2):
        s = opred.pooled_scores(q[0, h], k[0, h], M, N)
        _check_rows(bits[0, h], s, sp)
        keep = oracle.unpack_mask(bits[0, h], T_k)
        srt = -np.sort(-s, axis=1)
        for i in range(s.shape[0]):
            same = np.flatnonzero(s[i] == s[i, 0])       # the copies of tile 0 (and tile 0)
            kept = keep[i, same]
            # kept members of the run form a prefix in j order
            assert not np.any(~kept[:-1] & kept[1:]), f"row {i}: equal scores not kept by smaller j"
            if srt[i, kk - 1] == s[i, 0] and 0 < kept.sum() < same.size:
                run_rows += 1
    print(f"[predictor] spike rows split inside the run: {run_rows}", flush=True)
    assert run_rows > 0, "no row has its threshold inside the run of equal scores"


def test_predictor_rows_longer_than_65535_tiles():
    """Rows of 70000 key tiles (L = 70000, 64x1 tiles): the fused kernel's
    histograms switch from 16-bit to 32-bit counts past 65535 tiles.  Every
    row of both heads against the oracle (exact k, threshold band)."""
    torch_or_skip()
    w = W.Workload("p_wide", 1, 2, 70000, 64, 64, 1, "bf16", W.MaskRecipe("predicted", sparsity_percent=85),
                   77, offset_frame_tokens=14000, offset_sigma=0.5)
    say("predictor rows of 70000 key tiles")
    q, k, _ = W.make_qkv(w)
    bits = _run(q, k, w.M, w.N, 85)
    mism = 0
    for h in range(w.H):
        s = opred.pooled_scores(q[0, h], k[0, h], w.M, w.N)
        assert s.shape[1] > 65535
        mism += _check_rows(bits[0, h], s, 85)
    print(f"[predictor] 70000-tile rows: near-threshold decisions differing from fp64: {mism}", flush=True)
