"""Parity of the backward and of the FP8 path at the full 16x8 benchmark shape
(1 x 40 x 32760 x 128), and of the FP8 path at the 16x1 shape (1 x 40 x
75600 x 128), on sampled outputs the oracle computes one by one.

The GPU computes everything; the oracle the sampled rows of two heads (0 and
H-1): dQ of 16 sampled query tiles, dK and dV of 64 sampled keys (which needs
every query row of the head), the FP8 quantisation of the whole head, and the
FP8 attention of the sampled query tiles.  Masks of those heads come from the
host generator, checked equal to the GPU generator's first.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL, compare, mask_to_np, say, torch_or_skip
from oracle import backward as obwd
from oracle import fp8

pytestmark = pytest.mark.gpu

HEADS = (0, 39)


def _setup():
    import tile_sparse_attention_amd as T
    w = W.get("wan480_fine")
    say("large-next wan480_fine: generating inputs")
    q, k, v = W.make_qkv(w)
    mask = T.maskgen_hash(w.B, w.H, w.L, w.M, w.N, **W.hash_params(w))
    mnp = mask_to_np(mask)
    bits = {}
    for h in HEADS:
        bits[h] = W.pack_bits(W.mask_rows_bool(w, [(0, h, i) for i in range(w.T_q)]))
        assert np.array_equal(mnp[0, h], bits[h])
    return T, w, q, k, v, mask, bits


def _rel_check(case, got, ref):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    bmax = 2e-2 * max(1.0, float(np.abs(ref).max()))
    bmean = 1e-2 * float(np.abs(ref).mean()) + 1e-5
    print(f"[parity] {case}: max_abs={mx:.3e} (<= {bmax:.3e}) mean_abs={mean:.3e} (<= {bmean:.3e})", flush=True)
    assert mx <= bmax and mean <= bmean


def test_backward_full_shape_sampled():
    torch = torch_or_skip()
    T, w, q, k, v, mask, bits = _setup()
    do = W.make_do(w)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say("large-next: forward + backward on GPU")
    o, lse = T.attention_fwd(qd, kd, vd, mask, w.M, w.N, w.scale, return_lse=True)
    dq, dk, dv = T.attention_bwd(qd, kd, vd, o, dod, lse, mask, w.M, w.N, w.scale)
    torch.cuda.synchronize()
    dq, dk, dv = (x.float().cpu().numpy() for x in (dq, dk, dv))
    tiles = W.sample_tiles(w)
    rng = np.random.default_rng(5)
    for h in HEADS:
        k_rows = np.unique(np.concatenate([[0, 127, 128, w.L - 1], rng.choice(w.L, 60, replace=False)]))
        say(f"large-next: oracle backward head {h} ({len(k_rows)} keys, 16 query tiles)")
        qr, rdq, kr, rdk, rdv = obwd.attention_bwd_rows(q[0, h], k[0, h], v[0, h], do[0, h], bits[h], w.M, w.N,
                                                        w.scale, q_tiles=tiles[0, h, :16], k_rows=k_rows)
        _rel_check(f"bwd full h{h} dQ", dq[0, h][qr], rdq)
        _rel_check(f"bwd full h{h} dK", dk[0, h][kr], rdk)
        _rel_check(f"bwd full h{h} dV", dv[0, h][kr], rdv)


def test_fp8_full_shape_sampled():
    torch = torch_or_skip()
    T, w, q, k, v, mask, bits = _setup()
    say("large-next: FP8 quantisation and attention on GPU")
    q8, qs, k8, ks = T.quantize_qk_fp8(q.cuda(), k.cuda())
    o = T.attention_fwd_fp8(q8, k8, qs, ks, v.cuda(), mask, w.M, w.N, w.scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    tiles = W.sample_tiles(w)
    got, ref = [], []
    for h in HEADS:
        rq, rqs, rk, rks = fp8.quantize_qk(q[:, h:h + 1], k[:, h:h + 1])
        gq = q8[:, h:h + 1].cpu().view(torch.float8_e4m3fn).float().numpy()
        gk = k8[:, h:h + 1].cpu().view(torch.float8_e4m3fn).float().numpy()
        assert np.array_equal(gq, rq) and np.array_equal(gk, rk)
        assert np.array_equal(qs[:, h:h + 1].cpu().numpy(), rqs) and np.array_equal(ks[:, h:h + 1].cpu().numpy(), rks)
        qdq = fp8.dequantize(rq, rqs, 16)[0, 0]
        kdq = fp8.dequantize(rk, rks[..., None], w.L)[0, 0]
        say(f"large-next: oracle FP8 attention head {h}")
        rows, ro, _ = oracle.attention_rows(qdq, kdq, v[0, h], bits[h], w.M, w.N, w.scale, tiles[0, h])
        got.append(o[0, h][rows])
        ref.append(ro)
    compare("fp8 wan480_fine sampled", np.concatenate(got), np.concatenate(ref), "bf16")


@pytest.mark.timeout(900)
def test_fp8_wan720_n1_sampled():
    """The FP8-score path of the key kernel at the full 16x1 shape
    (1 x 40 x 75600 x 128, 80% i.i.d. per-key sparsity): the FP8 bytes and
    scales of heads 0 and 39 in full, and their 256 sampled query tiles
    against the oracle on the dequantised inputs."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    w = W.get("wan720_n1")
    say("large-next wan720_n1 FP8: generating inputs")
    q, k, v = W.make_qkv(w)
    mask = T.maskgen_hash(w.B, w.H, w.L, w.M, w.N, **W.hash_params(w))
    say("large-next wan720_n1 FP8: quantisation and attention on GPU")
    q8, qs, k8, ks = T.quantize_qk_fp8(q.cuda(), k.cuda())
    o = T.attention_fwd_fp8(q8, k8, qs, ks, v.cuda(), mask, w.M, w.N, w.scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    tiles = W.sample_tiles(w)
    mnp = mask_to_np(mask)
    got, ref = [], []
    for h in (0, w.H - 1):
        bits = np.zeros((w.T_q, w.words), dtype=np.uint32)
        bits[tiles[0, h]] = W.pack_bits(W.mask_rows_bool(w, [(0, h, int(i)) for i in tiles[0, h]]))
        assert np.array_equal(mnp[0, h, tiles[0, h]], bits[tiles[0, h]])
        rq, rqs, rk, rks = fp8.quantize_qk(q[:, h:h + 1], k[:, h:h + 1])
        gq = q8[:, h:h + 1].cpu().view(torch.float8_e4m3fn).float().numpy()
        gk = k8[:, h:h + 1].cpu().view(torch.float8_e4m3fn).float().numpy()
        assert np.array_equal(gq, rq) and np.array_equal(gk, rk)
        assert np.array_equal(qs[:, h:h + 1].cpu().numpy(), rqs) and np.array_equal(ks[:, h:h + 1].cpu().numpy(), rks)
        qdq = fp8.dequantize(rq, rqs, 16)[0, 0]
        kdq = fp8.dequantize(rk, rks[..., None], w.L)[0, 0]
        say(f"large-next wan720_n1 FP8: oracle head {h}")
        rows, ro, _ = oracle.attention_rows(qdq, kdq, v[0, h], bits, w.M, w.N, w.scale, tiles[0, h])
        got.append(o[0, h][rows])
        ref.append(ro)
    compare("fp8 wan720_n1 sampled", np.concatenate(got), np.concatenate(ref), "bf16")
