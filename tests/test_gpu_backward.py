"""GPU parity of the tile-sparse attention backward (dQ, dK, dV) against the
float64 CPU oracle (oracle/backward.py), through the C ABI, on seeded inputs.

The forward that feeds the backward (O and LSE) is the library's own, as in
training; the oracle recomputes everything from Q, K, V, dO and the mask.

Tolerance, from the arithmetic: the probabilities and dS are rounded to bf16
for the matrix cores and the gradients are stored in bf16, each a relative
error of at most 2^-9 per term, with fp32 accumulation in between.  So the
check is relative to the size of the reference: max-abs error at most 2% of
max(1, max |ref|) and mean-abs error at most 1% of mean |ref| plus 1e-5, the
fp32 rounding of dP - D where the reference is exactly zero (one kept key
per row); observed: about 0.4% and 0.25%.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import say, small_workload, to_dev_mask, torch_or_skip

pytestmark = pytest.mark.gpu

MAX_REL, MEAN_REL = 2e-2, 1e-2


def _check(case, got, ref):
    g = got.float().cpu().numpy()
    assert np.all(np.isfinite(g)), f"{case}: non-finite gradient"
    err = np.abs(g - ref)
    mx, mean = float(err.max()), float(err.mean())
    bound_max = MAX_REL * max(1.0, float(np.abs(ref).max()))
    bound_mean = MEAN_REL * float(np.abs(ref).mean()) + 1e-5
    print(f"[parity] {case}: max_abs={mx:.3e} (<= {bound_max:.3e}) mean_abs={mean:.3e} "
          f"(<= {bound_mean:.3e})", flush=True)
    assert mx <= bound_max, f"{case}: max-abs {mx} > {bound_max}"
    assert mean <= bound_mean, f"{case}: mean-abs {mean} > {bound_mean}"


def _run(w, bits, case, q=None, k=None, v=None, do=None, scale=None):
    import tile_sparse_attention_amd as T
    torch = torch_or_skip()
    say(f"{case}: B={w.B} H={w.H} L={w.L} d={w.d} M={w.M} N={w.N} seed={w.seed}")
    if q is None:
        q, k, v = W.make_qkv(w)
        do = W.make_do(w)
    scale = w.scale if scale is None else scale
    qd, kd, vd, dod, md = q.cuda(), k.cuda(), v.cuda(), do.cuda(), to_dev_mask(bits)
    o, lse = T.attention_fwd(qd, kd, vd, md, w.M, w.N, scale, return_lse=True)
    dq, dk, dv = T.attention_bwd(qd, kd, vd, o, dod, lse, md, w.M, w.N, scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, bits, w.M, w.N, scale)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        _check(f"{case} {name}", got, ref)
    return dq, dk, dv


@pytest.mark.parametrize("M", [16, 32, 64])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 32, 64])
def test_bwd_tile_grid_ragged(M, N):
    # L = 1000: partial last 128-row chunk, 16-row unit and key tile (N >= 16)
    w = small_workload(f"bwd_{M}x{N}", 1000, 128, M, N, p=0.3, seed=300 + M + N)
    _run(w, W.mask_bits(w), f"bwd d128 {M}x{N} L=1000")


@pytest.mark.parametrize("N", [1, 8])
def test_bwd_kept_counts_at_pass_boundaries(N):
    # kept key tiles per (query tile, 128-key chunk) cycled over the counts a
    # dQ pass (32 keys, one score block when <= 16 remain) or a dK/dV unit
    # pair can end on; the dK/dV side sees the same tiles from the key side
    counts = {1: (0, 1, 15, 16, 17, 31, 32, 33, 48, 49, 128), 8: (0, 1, 2, 3, 4, 5, 8, 15, 16)}[N]
    L = 1024 + 45
    w = small_workload(f"bwd_passes_{N}", L, 128, 16, N, seed=300 + N)
    tpc = 128 // N
    rng = np.random.default_rng(100 + N)
    keep = np.zeros((1, w.H, w.T_q, w.T_k), dtype=bool)
    for h in range(w.H):
        for i in range(w.T_q):
            for c in range(-(-w.T_k // tpc)):
                j0, j1 = c * tpc, min(c * tpc + tpc, w.T_k)
                n = min(counts[(i + 3 * c + h) % len(counts)], j1 - j0)
                keep[0, h, i, j0 + rng.choice(j1 - j0, n, replace=False)] = True
    _run(w, W.pack_bits(keep), f"bwd 16x{N} kept counts at pass boundaries")


@pytest.mark.parametrize("M,N,L", [(16, 8, 777), (64, 4, 1029), (16, 1, 500), (32, 64, 300)])
def test_bwd_head_dim_64(M, N, L):
    w = small_workload(f"bwd64_{M}x{N}", L, 64, M, N, p=0.3, seed=400 + M + N + L)
    _run(w, W.mask_bits(w), f"bwd d64 {M}x{N} L={L}")


@pytest.mark.parametrize("L", [1, 13, 16, 127, 129, 256])
def test_bwd_short_and_boundary_lengths(L):
    w = small_workload(f"bwd_len{L}", L, 128, 16, 8, p=0.5, seed=500 + L)
    _run(w, W.mask_bits(w), f"bwd 16x8 L={L}")


def test_bwd_all_ones_mask():
    w = small_workload("bwd_ones", 640, 128, 16, 8, seed=61)
    bits = W.pack_bits(np.ones((1, 2, w.T_q, w.T_k), dtype=bool))
    _run(w, bits, "bwd 16x8 all kept")


def test_bwd_empty_rows_and_heads():
    # head 0: every third query tile keeps nothing; head 1 keeps nothing at all
    w = small_workload("bwd_empty", 600, 128, 16, 8, seed=62)
    keep = W.mask_rows_bool(w, np.array([(0, h, i) for h in range(2) for i in range(w.T_q)]))
    keep = keep.reshape(1, 2, w.T_q, w.T_k)
    keep[0, 0, ::3] = False
    keep[0, 1] = False
    dq, dk, dv = _run(w, W.pack_bits(keep), "bwd 16x8 empty rows / head")
    assert float(dq[0, 1].abs().max()) == 0.0 and float(dk[0, 1].abs().max()) == 0.0
    assert float(dv[0, 1].abs().max()) == 0.0
    assert float(dq[0, 0, 0:16].abs().max()) == 0.0


def test_bwd_negative_scale_and_batch():
    w = W.Workload("bwd_neg", 2, 3, 500, 128, 16, 16, "bf16",
                   W.MaskRecipe("hash", p_near=0.4, p_far=0.4, force_diag=True), 63)
    _run(w, W.mask_bits(w), "bwd 16x16 B=2 H=3 scale<0", scale=-w.scale)


def test_bwd_large_logits():
    # Q scaled by 8: sharp softmax rows, probabilities near 0 and 1
    torch = torch_or_skip()
    w = small_workload("bwd_big", 600, 128, 16, 8, p=0.5, seed=64)
    q, k, v = W.make_qkv(w)
    q = (q.float() * 8).to(torch.bfloat16)
    _run(w, W.mask_bits(w), "bwd 16x8 large logits", q=q, k=k, v=v, do=W.make_do(w))
