"""GPU parity of the FP8 path: the e4m3 quantisation of Q and K is bit-exact
against the oracle's (oracle/fp8.py), and FP8-score attention matches the
float64 oracle applied to the dequantised Q and K (V in bf16) within the
bf16 path's tolerance: the arithmetic after quantisation is the bf16 path's
(fp32 accumulation, probabilities rounded to bf16, O stored in bf16)."""
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


def _run(w, bits, case, scale=None, q=None, k=None, v=None):
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
    fin = np.isfinite(rl)
    gl = lse.cpu().numpy()
    assert np.array_equal(np.isfinite(gl), fin)
    if fin.any():
        assert float(np.abs(gl[fin] - rl[fin]).max()) <= 2e-2


@pytest.mark.parametrize("M,N,L", [(16, 8, 1000), (16, 16, 1003), (32, 32, 777), (64, 64, 1029), (16, 8, 13),
                                   (32, 8, 4099)])
def test_fp8_attention_parity(M, N, L):
    w = small_workload(f"f8_{M}x{N}", L, 128, M, N, p=0.3, seed=800 + M + N + L)
    _run(w, W.mask_bits(w), f"fp8 {M}x{N} L={L}")


def test_fp8_attention_negative_scale_and_batch():
    w = W.Workload("f8_neg", 2, 3, 600, 128, 16, 16, "bf16",
                   W.MaskRecipe("hash", p_near=0.4, p_far=0.4, force_diag=True), 81)
    _run(w, W.mask_bits(w), "fp8 16x16 B=2 H=3 scale<0", scale=-w.scale)


def test_fp8_attention_large_logits_and_empty_rows():
    torch = torch_or_skip()
    w = small_workload("f8_big", 700, 128, 16, 8, p=0.5, seed=82)
    q, k, v = W.make_qkv(w)
    q = (q.float() * 8).to(torch.bfloat16)
    keep = W.mask_rows_bool(w, np.array([(0, h, i) for h in range(2) for i in range(w.T_q)]))
    keep = keep.reshape(1, 2, w.T_q, w.T_k)
    keep[0, 1, ::4] = False
    _run(w, W.pack_bits(keep), "fp8 16x8 logits x8, empty rows", q=q, k=k, v=v)


def test_fp8_rejects_unsupported_shapes():
    import tile_sparse_attention_amd as T
    torch = torch_or_skip()
    w = small_workload("f8_n4", 300, 128, 16, 4, seed=83)
    q, k, v = W.make_qkv(w)
    q8, qs, k8, ks = _quantize_gpu(q, k)
    with pytest.raises(T.TsaError) as e:
        T.attention_fwd_fp8(q8, k8, qs, ks, v.cuda(), to_dev_mask(W.mask_bits(w)), 16, 4)
    assert e.value.status == T.ERR_UNSUPPORTED
    torch.cuda.synchronize()
