"""GPU parity of the FP8 path: the e4m3 quantisation of Q and K is bit-exact
against the oracle's (oracle/fp8.py), and FP8-score attention matches the
float64 oracle applied to the dequantised Q and K (V in bf16) within the
bf16 path's tolerance: the arithmetic after quantisation is the bf16 path's
(fp32 accumulation, probabilities rounded to bf16, O stored in bf16).

The quantisation's own error, against the float64 oracle on the unquantised
inputs, is bounded for N(0,1) Q, K, V at scale 1/sqrt(d) by this arithmetic:
rounding to e4m3 (3 mantissa bits) leaves a relative error of at most 2^-4
per element, RMS at most 2^-4/sqrt(3) = 0.036; a score q.k*scale then moves by
sigma_s = scale * sqrt(2 d E[q^2 k^2]) * 0.036 = 0.051 RMS (d = 128).  An
output element sum_j p_j v_j moves by about sigma_s * sqrt(sum_j p_j^2) *
sigma_v <= sigma_s, since sum_j p_j^2 <= 1 and sigma_v = 1.  So max-abs
<= 6 sigma_s = 0.31 and mean-abs <= 0.8 sigma_s = 0.041 (the mean-abs of a
normal of that RMS).  Sharper logits (the x8 case) are outside this bound
and only printed."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL, say, small_workload, to_dev_mask, torch_or_skip
from oracle import fp8

pytestmark = pytest.mark.gpu


def _quantize_gpu(q, k):
    import tile_sparse_attention_amd as T
    torch = torch_or_skip()
    q8, qs, k8, ks = T.quantize_qk_fp8(q.cuda(), k.cuda())
    torch.cuda.synchronize()
    return q8, qs, k8, ks


def _e4m3_values(bytes_u8):
    import torch
    return bytes_u8.cpu().view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


@pytest.mark.parametrize("L", [1000, 13, 256, 4099, 1])
def test_quantize_bit_exact(L):
    torch = torch_or_skip()
    w = small_workload(f"q8_{L}", L, 128, 16, 8, seed=700 + L)
    q, k, _ = W.make_qkv(w)
    if L == 1000:
        q[0, 1, 32:48] = 0                        # an all-zero Q tile: scale 1, zero bytes
    say(f"fp8 quantise L={L}")
    q8, qs, k8, ks = _quantize_gpu(q, k)
    rq, rqs, rk, rks = fp8.quantize_qk(q, k)
    assert np.array_equal(qs.cpu().numpy(), rqs) and np.array_equal(ks.cpu().numpy(), rks)
    assert np.array_equal(_e4m3_values(q8), rq) and np.array_equal(_e4m3_values(k8), rk)


UNQUANTISED_TOL = dict(max_abs=0.31, mean_abs=0.041)


def _run(w, bits, case, scale=None, q=None, k=None, v=None, normal_inputs=True):
    import tile_sparse_attention_amd as T
    torch = torch_or_skip()
    say(f"{case}: B={w.B} H={w.H} L={w.L} M={w.M} N={w.N} seed={w.seed}")
    if q is None:
        q, k, v = W.make_qkv(w)
    scale = w.scale if scale is None else scale
    q8, qs, k8, ks = _quantize_gpu(q, k)
    o, lse = T.attention_fwd_fp8(q8, k8, qs, ks, v.cuda(), to_dev_mask(bits), w.M, w.N, scale, return_lse=True)
    torch.cuda.synchronize()
    # the oracle's own quantisation (bit-exact with the GPU's, tested above), dequantised
    rq, rqs, rk, rks = fp8.quantize_qk(q, k)
    qd = fp8.dequantize(rq, rqs, 16)
    kd = fp8.dequantize(rk, rks[..., None], w.L)
    ro, rl = oracle.attention(qd, kd, v, bits, w.M, w.N, scale)
    got = o.float().cpu().numpy()
    err = np.abs(got - ro)
    mx, mean = float(err.max()), float(err.mean())
    exact, _ = oracle.attention(q, k, v, bits, w.M, w.N, scale)
    qerr = np.abs(got - exact)
    print(f"[parity] {case}: vs dequantised oracle max_abs={mx:.3e} mean_abs={mean:.3e}; "
          f"vs unquantised oracle max_abs={qerr.max():.3e} mean_abs={qerr.mean():.3e}", flush=True)
    assert np.all(np.isfinite(got))
    assert mx <= TOL["bf16"]["max_abs"] and mean <= TOL["bf16"]["mean_abs"]
    if normal_inputs:
        assert qerr.max() <= UNQUANTISED_TOL["max_abs"] and qerr.mean() <= UNQUANTISED_TOL["mean_abs"]
    fin = np.isfinite(rl)
    gl = lse.cpu().numpy()
    assert np.array_equal(np.isfinite(gl), fin)
    if fin.any():
        assert float(np.abs(gl[fin] - rl[fin]).max()) <= 2e-2


@pytest.mark.parametrize("M,N,L", [(16, 8, 1000), (16, 16, 1003), (32, 32, 777), (64, 64, 1029), (16, 8, 13),
                                   (32, 8, 4099), (16, 1, 1000), (16, 2, 777), (16, 4, 1003), (32, 1, 300),
                                   (64, 2, 515), (16, 1, 13)])
def test_fp8_attention_parity(M, N, L):
    w = small_workload(f"f8_{M}x{N}", L, 128, M, N, p=0.3, seed=800 + M + N + L)
    _run(w, W.mask_bits(w), f"fp8 {M}x{N} L={L}")


# kept tiles per (query tile, 128-key chunk) cycling through every count a
# pass can end on: 32 keys per pass with a short last pass at 16 or fewer
# (N < 8), four octets per pass with a short last pass at one or two (N >= 8)
_PASS_COUNTS = {1: (0, 1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 100, 127, 128),
                4: (0, 1, 3, 4, 5, 7, 8, 9, 15, 16, 17, 24, 31, 32),
                8: (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 15, 16), 16: (0, 1, 2, 3, 4, 5, 6, 7, 8)}


@pytest.mark.parametrize("N", [1, 4, 8, 16])
def test_fp8_kept_counts_at_pass_boundaries(N):
    L = 2048 + 77   # 16 whole chunks and a partial one
    w = small_workload(f"f8_passes_{N}", L, 128, 16, N, seed=840 + N)
    tpc = 128 // N
    counts = _PASS_COUNTS[N]
    rng = np.random.default_rng(40 + N)
    keep = np.zeros((1, w.H, w.T_q, w.T_k), dtype=bool)
    for h in range(w.H):
        for i in range(w.T_q):
            for c in range(-(-w.T_k // tpc)):
                j0, j1 = c * tpc, min(c * tpc + tpc, w.T_k)
                n = min(counts[(i + 3 * c + h) % len(counts)], j1 - j0)
                keep[0, h, i, j0 + rng.choice(j1 - j0, n, replace=False)] = True
    _run(w, W.pack_bits(keep), f"fp8 16x{N} kept counts at pass boundaries")


@pytest.mark.parametrize("N", [16, 1])
def test_fp8_attention_negative_scale_and_batch(N):
    w = W.Workload(f"f8_neg_{N}", 2, 3, 600, 128, 16, N, "bf16",
                   W.MaskRecipe("hash", p_near=0.4, p_far=0.4, force_diag=True), 81 + N)
    _run(w, W.mask_bits(w), f"fp8 16x{N} B=2 H=3 scale<0", scale=-w.scale)


@pytest.mark.parametrize("N", [8, 1])
def test_fp8_attention_large_logits_and_empty_rows(N):
    torch = torch_or_skip()
    w = small_workload(f"f8_big_{N}", 700, 128, 16, N, p=0.5, seed=82 + N)
    q, k, v = W.make_qkv(w)
    q = (q.float() * 8).to(torch.bfloat16)
    keep = W.mask_rows_bool(w, np.array([(0, h, i) for h in range(2) for i in range(w.T_q)]))
    keep = keep.reshape(1, 2, w.T_q, w.T_k)
    keep[0, 1, ::4] = False
    _run(w, W.pack_bits(keep), f"fp8 16x{N} logits x8, empty rows", q=q, k=k, v=v, normal_inputs=False)


def test_fp8_rejects_unsupported_shapes():
    """d = 64 has no FP8 path (one 16x16x128 step would be half padding): the
    call is refused before any kernel runs."""
    import tile_sparse_attention_amd as T
    torch = torch_or_skip()
    B, H, L, d = 1, 2, 300, 64
    q8 = torch.zeros((B, H, L, d), dtype=torch.uint8, device="cuda")
    k8 = torch.zeros_like(q8)
    qs = torch.ones((B, H, -(-L // 16)), dtype=torch.float32, device="cuda")
    ks = torch.ones((B, H), dtype=torch.float32, device="cuda")
    v = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device="cuda")
    mask = torch.zeros((B, H, -(-L // 16), T.mask_row_words(L, 8)), dtype=torch.int32, device="cuda")
    with pytest.raises(T.TsaError) as e:
        T.attention_fwd_fp8(q8, k8, qs, ks, v, mask, 16, 8)
    assert e.value.status == T.ERR_UNSUPPORTED
    torch.cuda.synchronize()
