"""GPU parity at the limits of the supported problem set: the longest
sequence (L = 2^22) and the most (batch, head) pairs (B*H = 2^20).

Inputs are seeded and synthetic.  At L = 2^22 the bitmap of 16x8 tiles holds
2^32 words (17 GB) and is made on the GPU by the counter-based generator;
the sampled query tiles' rows come from the host generator (checked equal to
the GPU's first) and the oracle evaluates those tiles one at a time.  At
B*H = 2^20 every head takes its Q, K, V from one of 4096 seeded heads (head h
of batch b uses head h mod 4096 of a [1, 4096, L, d] draw), while its mask
rows are its own; sampled heads are compared in full (forward, and dQ, dK,
dV of the backward), and the FP8 quantisation of sampled heads byte for
byte.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import compare, say, torch_or_skip
from oracle import fp8
from oracle.sparse_attention import tile_rows

pytestmark = pytest.mark.gpu

L_MAX = 1 << 22
BH_MAX = 1 << 20


@pytest.mark.timeout(900)
def test_maximum_sequence_length():
    """L = 2^22 (the plain octet kernel: more chunks than chunk skipping
    handles), one head, 16x8 tiles, i.i.d. 2% keep with the diagonal kept:
    16 sampled query tiles, the first and the last among them."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    w = W.Workload("maxlen", 1, 1, L_MAX, 128, 16, 8, "bf16",
                   W.MaskRecipe("hash", p_near=0.02, p_far=0.02, force_diag=True), 4321)
    say(f"limits L={w.L} 16x8: generating inputs")
    q, k, v = W.make_qkv(w)
    mask = T.maskgen_hash(w.B, w.H, w.L, w.M, w.N, **W.hash_params(w))
    say(f"limits L={w.L} 16x8: attention on GPU (bitmap {mask.numel() * 4 / 2**30:.1f} GiB)")
    o, lse = T.attention_fwd(q.cuda(), k.cuda(), v.cuda(), mask, w.M, w.N, w.scale, return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(17)
    tiles = np.unique(np.concatenate([[0, w.T_q - 1], rng.choice(w.T_q, 14, replace=False)]))
    # host rows of the sampled tiles only (the rest of this zero array is never touched)
    bits = np.zeros((w.T_q, w.words), dtype=np.uint32)
    bits[tiles] = W.pack_bits(W.mask_rows_bool(w, [(0, 0, int(i)) for i in tiles]))
    dev_rows = mask[0, 0, torch.from_numpy(tiles).cuda()].cpu().numpy().view(np.uint32)
    assert np.array_equal(dev_rows, bits[tiles])
    del mask
    say(f"limits L={w.L} 16x8: oracle on {len(tiles)} tiles")
    rows, ro, rl = oracle.attention_rows(q[0, 0], k[0, 0], v[0, 0], bits, w.M, w.N, w.scale, tiles, group=1)
    compare(f"limits L={w.L}", o[0, 0, torch.from_numpy(rows).cuda()].float().cpu().numpy(), ro, w.dtype,
            lse[0, 0, torch.from_numpy(rows).cuda()].cpu().numpy(), rl)


def _max_heads_inputs(w_src, B, H):
    """Q, K, V of B*H heads on the GPU, head (b, h) equal to head h mod the
    source heads of the seeded draw w_src."""
    torch_or_skip()
    src = W.make_qkv(w_src)
    reps = B * H // w_src.H
    L, d = w_src.L, w_src.d
    return [x.cuda().reshape(w_src.H, L, d).repeat(reps, 1, 1).reshape(B, H, L, d) for x in src], src


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,N", [(16, 8), (16, 1)])
def test_maximum_heads(M, N):
    """B*H = 2^20 (B = 16, H = 65536) at L = 40 (three query tiles, the last
    partial), d = 64, bf16: the octet kernel (16x8) and the key kernel (16x1)
    over a grid of 2^20 work-groups; eight sampled heads compared in full."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    B, H, L, d = 16, BH_MAX // 16, 40, 64
    src = W.Workload("maxheads_src", 1, 4096, L, d, M, N, "bf16", W.MaskRecipe("hash", p_near=0.3, p_far=0.3), 97)
    w = W.Workload("maxheads", B, H, L, d, M, N, "bf16",
                   W.MaskRecipe("hash", p_near=0.3, p_far=0.3, force_diag=True), 98 + N)
    say(f"limits B*H={B * H} L={L} d={d} {M}x{N}: inputs")
    (qd, kd, vd), (q, k, v) = _max_heads_inputs(src, B, H)
    mask = T.maskgen_hash(B, H, L, M, N, **W.hash_params(w))
    say(f"limits B*H={B * H} {M}x{N}: attention on GPU")
    o, lse = T.attention_fwd(qd, kd, vd, mask, M, N, w.scale, return_lse=True)
    torch.cuda.synchronize()
    del qd, kd, vd
    rng = np.random.default_rng(5 + N)
    heads = [(0, 0), (0, 1), (B - 1, H - 1), (B // 2, 4095), (7, 4096)] + \
            [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 3), rng.integers(0, H, 3))]
    got, ref, gl, rl = [], [], [], []
    for b, h in heads:
        bits = W.pack_bits(W.mask_rows_bool(w, [(b, h, i) for i in range(w.T_q)]))
        assert np.array_equal(mask[b, h].cpu().numpy().view(np.uint32), bits)
        s = h % src.H
        ro, rlse = oracle.attention(q[:, s:s + 1], k[:, s:s + 1], v[:, s:s + 1], bits[None, None], M, N, w.scale)
        got.append(o[b, h].float().cpu().numpy())
        ref.append(ro[0, 0])
        gl.append(lse[b, h].cpu().numpy())
        rl.append(rlse[0, 0])
    compare(f"limits B*H={B * H} {M}x{N}", np.concatenate(got), np.concatenate(ref), "bf16",
            np.concatenate(gl), np.concatenate(rl))


@pytest.mark.timeout(600)
def test_fp8_at_maximum_heads():
    """The e4m3 quantisation of Q and K over B*H = 2^20 heads (L = 40, d = 128;
    the per-head K maxima run over a one-dimensional grid of 64 slices per
    head): sampled heads byte for byte against the oracle; then the FP8-score
    attention over all heads (16x8 through the octet kernel, 16x1 through the
    key kernel), sampled heads against the oracle on the dequantised Q and K."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    B, H, L = 16, BH_MAX // 16, 40
    src = W.Workload("maxheads_f8", 1, 4096, L, 128, 16, 8, "bf16", W.MaskRecipe("hash", p_near=0.3, p_far=0.3), 99)
    w = W.Workload("maxheads_f8", B, H, L, 128, 16, 8, "bf16",
                   W.MaskRecipe("hash", p_near=0.3, p_far=0.3, force_diag=True), 100)
    say(f"limits B*H={B * H} L={L}: fp8 quantisation")
    (qd, kd, vd), (q, k, v) = _max_heads_inputs(src, B, H)
    q8, qs, k8, ks = T.quantize_qk_fp8(qd, kd)
    torch.cuda.synchronize()
    del qd, kd
    for b, h in [(0, 0), (B - 1, H - 1), (3, 4097), (11, 60000)]:
        s = h % src.H
        rq, rqs, rk, rks = fp8.quantize_qk(q[:, s:s + 1], k[:, s:s + 1])
        assert np.array_equal(qs[b, h].cpu().numpy(), rqs[0, 0]) and np.array_equal(ks[b, h].cpu().numpy(), rks[0, 0])
        got_q = q8[b, h].cpu().view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
        got_k = k8[b, h].cpu().view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
        assert np.array_equal(got_q, rq[0, 0]) and np.array_equal(got_k, rk[0, 0])
    say(f"limits B*H={B * H} L={L}: fp8 attention")
    mask = T.maskgen_hash(B, H, L, w.M, w.N, **W.hash_params(w))
    o = T.attention_fwd_fp8(q8, k8, qs, ks, vd, mask, w.M, w.N, w.scale)
    torch.cuda.synchronize()
    got, ref = [], []
    for b, h in [(0, 0), (B - 1, H - 1), (3, 4097), (11, 60000)]:
        s = h % src.H
        bits = W.pack_bits(W.mask_rows_bool(w, [(b, h, i) for i in range(w.T_q)]))
        assert np.array_equal(mask[b, h].cpu().numpy().view(np.uint32), bits)
        rq, rqs, rk, rks = fp8.quantize_qk(q[:, s:s + 1], k[:, s:s + 1])
        ro, _ = oracle.attention(fp8.dequantize(rq, rqs, 16), fp8.dequantize(rk, rks[..., None], L),
                                 v[:, s:s + 1], bits[None, None], w.M, w.N, w.scale)
        got.append(o[b, h].float().cpu().numpy())
        ref.append(ro[0, 0])
    compare(f"limits B*H={B * H} fp8 16x8", np.concatenate(got), np.concatenate(ref), "bf16")
    # the key kernel's FP8 mode (16x1) over all heads, on the same e4m3 inputs
    del mask, o
    w1 = W.Workload("maxheads_f8_n1", B, H, L, 128, 16, 1, "bf16",
                    W.MaskRecipe("hash", p_near=0.3, p_far=0.3, force_diag=True), 101)
    say(f"limits B*H={B * H} L={L}: fp8 attention 16x1")
    mask = T.maskgen_hash(B, H, L, w1.M, w1.N, **W.hash_params(w1))
    o = T.attention_fwd_fp8(q8, k8, qs, ks, vd, mask, w1.M, w1.N, w1.scale)
    torch.cuda.synchronize()
    got, ref = [], []
    for b, h in [(0, 0), (B - 1, H - 1), (3, 4097), (11, 60000)]:
        s = h % src.H
        bits = W.pack_bits(W.mask_rows_bool(w1, [(b, h, i) for i in range(w1.T_q)]))
        assert np.array_equal(mask[b, h].cpu().numpy().view(np.uint32), bits)
        rq, rqs, rk, rks = fp8.quantize_qk(q[:, s:s + 1], k[:, s:s + 1])
        ro, _ = oracle.attention(fp8.dequantize(rq, rqs, 16), fp8.dequantize(rk, rks[..., None], L),
                                 v[:, s:s + 1], bits[None, None], w1.M, w1.N, w1.scale)
        got.append(o[b, h].float().cpu().numpy())
        ref.append(ro[0, 0])
    compare(f"limits B*H={B * H} fp8 16x1", np.concatenate(got), np.concatenate(ref), "bf16")


@pytest.mark.timeout(900)
def test_fp8_attention_at_maximum_sequence_length():
    """FP8-score attention at L = 2^22 (one head, 16x8, 2% i.i.d. keep with
    the diagonal kept): 16 sampled query tiles against the oracle on the
    dequantised Q and K (the oracle's own e4m3 rounding, bit-exact with the
    GPU's by the quantisation tests)."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    w = W.Workload("maxlen_f8", 1, 1, L_MAX, 128, 16, 8, "bf16",
                   W.MaskRecipe("hash", p_near=0.02, p_far=0.02, force_diag=True), 4600)
    say(f"limits L={w.L} fp8 16x8: generating inputs")
    q, k, v = W.make_qkv(w)
    mask = T.maskgen_hash(w.B, w.H, w.L, w.M, w.N, **W.hash_params(w))
    q8, qs, k8, ks = T.quantize_qk_fp8(q.cuda(), k.cuda())
    say(f"limits L={w.L} fp8 16x8: attention on GPU")
    o = T.attention_fwd_fp8(q8, k8, qs, ks, v.cuda(), mask, w.M, w.N, w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(29)
    tiles = np.unique(np.concatenate([[0, w.T_q - 1], rng.choice(w.T_q, 14, replace=False)]))
    bits = np.zeros((w.T_q, w.words), dtype=np.uint32)
    bits[tiles] = W.pack_bits(W.mask_rows_bool(w, [(0, 0, int(i)) for i in tiles]))
    dev_rows = mask[0, 0, torch.from_numpy(tiles).cuda()].cpu().numpy().view(np.uint32)
    assert np.array_equal(dev_rows, bits[tiles])
    del mask, q8, k8
    say(f"limits L={w.L} fp8 16x8: oracle on {len(tiles)} tiles")
    # Q scales are per 16-row tile, so the sampled tiles' rows quantise on
    # their own; K has one scale per head
    rows = tile_rows(w.L, w.M, tiles)
    qv, qsc = fp8.quantize(q[0, 0].float().numpy()[rows], 16)
    kv, ksc = fp8.quantize(k[0, 0].float().numpy(), w.L)
    assert np.array_equal(qs[0, 0, torch.from_numpy(tiles).cuda()].cpu().numpy(), qsc)
    assert np.array_equal(ks[0, 0].cpu().numpy().reshape(1), ksc)
    qdq = np.zeros((w.L, w.d))          # only the sampled rows are read
    qdq[rows] = fp8.dequantize(qv, qsc, 16)
    kdq = fp8.dequantize(kv, ksc, w.L)
    del kv
    rows, ro, _ = oracle.attention_rows(qdq, kdq, v[0, 0], bits, w.M, w.N, w.scale, tiles, group=1)
    compare(f"limits L={w.L} fp8 16x8", o[0, 0, torch.from_numpy(rows).cuda()].float().cpu().numpy(), ro, "bf16")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("N", [8, 1])
def test_backward_at_maximum_heads(N):
    """The backward over B*H = 2^20 heads (L = 40, d = 64, 16xN): eight
    sampled heads' dQ, dK, dV against the oracle, within the backward's
    tolerance (max-abs 2% of max(1, max|ref|), mean-abs 1% of mean|ref| +
    1e-5)."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    B, H, L, d, M = 16, BH_MAX // 16, 40, 64, 16
    src = W.Workload("maxheads_bwd", 1, 4096, L, d, M, N, "bf16", W.MaskRecipe("hash", p_near=0.3, p_far=0.3), 91)
    w = W.Workload("maxheads_bwd", B, H, L, d, M, N, "bf16",
                   W.MaskRecipe("hash", p_near=0.3, p_far=0.3, force_diag=True), 92 + N)
    say(f"limits B*H={B * H} L={L} d={d} {M}x{N}: backward inputs")
    (qd, kd, vd), (q, k, v) = _max_heads_inputs(src, B, H)
    do_src = W.make_do(src)
    dod = do_src.cuda().reshape(src.H, L, d).repeat(B * H // src.H, 1, 1).reshape(B, H, L, d)
    mask = T.maskgen_hash(B, H, L, M, N, **W.hash_params(w))
    say(f"limits B*H={B * H} {M}x{N}: forward and backward on GPU")
    o, lse = T.attention_fwd(qd, kd, vd, mask, M, N, w.scale, return_lse=True)
    dq, dk, dv = T.attention_bwd(qd, kd, vd, o, dod, lse, mask, M, N, w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(60 + N)
    heads = [(0, 0), (B - 1, H - 1), (5, 4096), (9, 12345)] + \
            [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 4), rng.integers(0, H, 4))]
    for b, h in heads:
        bits = W.pack_bits(W.mask_rows_bool(w, [(b, h, i) for i in range(w.T_q)]))
        assert np.array_equal(mask[b, h].cpu().numpy().view(np.uint32), bits)
        s = h % src.H
        sl = slice(s, s + 1)
        ref = oracle.attention_bwd(q[:, sl], k[:, sl], v[:, sl], do_src[:, sl], bits[None, None], M, N, w.scale)
        for name, got, r in (("dQ", dq, ref[0]), ("dK", dk, ref[1]), ("dV", dv, ref[2])):
            g = got[b, h].float().cpu().numpy()
            err = np.abs(g - r[0, 0])
            assert np.all(np.isfinite(g))
            assert err.max() <= 2e-2 * max(1.0, float(np.abs(r).max())), (b, h, name, float(err.max()))
            assert err.mean() <= 1e-2 * float(np.abs(r).mean()) + 1e-5, (b, h, name, float(err.mean()))
    print(f"[parity] limits B*H={B * H} {M}x{N} backward: {len(heads)} heads within tolerance", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype,d,M,N,p", [("f32", 128, 16, 16, 0.02), ("bf16", 128, 16, 1, 0.002)])
def test_maximum_sequence_length_other_kernels(dtype, d, M, N, p):
    """L = 2^22 through the fp32 kernel (16x16; its V^T spans more than 2^31
    bytes per head) and the bf16 key kernel (16x1; a 2^35-word, 137 GB
    bitmap): one head, i.i.d. keep with the diagonal kept, 16 sampled query
    tiles."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    w = W.Workload(f"maxlen_{dtype}_{N}", 1, 1, L_MAX, d, M, N, dtype,
                   W.MaskRecipe("hash", p_near=p, p_far=p, force_diag=True), 4400 + N)
    say(f"limits L={w.L} {dtype} {M}x{N}: generating inputs")
    q, k, v = W.make_qkv(w)
    mask = T.maskgen_hash(w.B, w.H, w.L, w.M, w.N, **W.hash_params(w))
    say(f"limits L={w.L} {dtype} {M}x{N}: attention on GPU (bitmap {mask.numel() * 4 / 2**30:.1f} GiB)")
    o, lse = T.attention_fwd(q.cuda(), k.cuda(), v.cuda(), mask, w.M, w.N, w.scale, return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(19 + N)
    tiles = np.unique(np.concatenate([[0, w.T_q - 1], rng.choice(w.T_q, 14, replace=False)]))
    bits = np.zeros((w.T_q, w.words), dtype=np.uint32)
    bits[tiles] = W.pack_bits(W.mask_rows_bool(w, [(0, 0, int(i)) for i in tiles]))
    dev_rows = mask[0, 0, torch.from_numpy(tiles).cuda()].cpu().numpy().view(np.uint32)
    assert np.array_equal(dev_rows, bits[tiles])
    del mask
    say(f"limits L={w.L} {dtype} {M}x{N}: oracle on {len(tiles)} tiles")
    rows, ro, rl = oracle.attention_rows(q[0, 0], k[0, 0], v[0, 0], bits, w.M, w.N, w.scale, tiles, group=1)
    idx = torch.from_numpy(rows).cuda()
    compare(f"limits L={w.L} {dtype} {M}x{N}", o[0, 0, idx].float().cpu().numpy(), ro, w.dtype,
            lse[0, 0, idx].cpu().numpy(), rl)


@pytest.mark.timeout(900)
def test_backward_at_maximum_sequence_length():
    """The backward at L = 2^22 (one head, 16x8, 2% i.i.d. keep with the
    diagonal kept).  dQ of 16 sampled query tiles against the oracle (each dQ
    row needs only its own row of P); dK and dV need every query row, so they
    are checked by identities that hold at any size when every row keeps a
    key: sum_k dV[k] = sum_q dO[q] (the probabilities of a row sum to 1) and
    sum_k dK[k] = 0 (sum_k dS[q, k] = D_q - D_q sum_k P[q, k] = 0).  Bound for
    both: 1e-3 x sqrt(sum_q dO[q]^2) per d, against an expected rounding
    residue of about 0.03 from the bf16 probabilities and outputs; a dropped
    1% of rows would leave about 200."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    from oracle import backward as obwd
    w = W.Workload("maxlen_bwd", 1, 1, L_MAX, 128, 16, 8, "bf16",
                   W.MaskRecipe("hash", p_near=0.02, p_far=0.02, force_diag=True), 4500)
    say(f"limits L={w.L} 16x8 backward: generating inputs")
    q, k, v = W.make_qkv(w)
    do = W.make_do(w)
    mask = T.maskgen_hash(w.B, w.H, w.L, w.M, w.N, **W.hash_params(w))
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    say(f"limits L={w.L} 16x8 backward: forward and backward on GPU")
    o, lse = T.attention_fwd(qd, kd, vd, mask, w.M, w.N, w.scale, return_lse=True)
    dq, dk, dv = T.attention_bwd(qd, kd, vd, o, dod, lse, mask, w.M, w.N, w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(23)
    tiles = np.unique(np.concatenate([[0, w.T_q - 1], rng.choice(w.T_q, 14, replace=False)]))
    bits = np.zeros((w.T_q, w.words), dtype=np.uint32)
    bits[tiles] = W.pack_bits(W.mask_rows_bool(w, [(0, 0, int(i)) for i in tiles]))
    dev_rows = mask[0, 0, torch.from_numpy(tiles).cuda()].cpu().numpy().view(np.uint32)
    assert np.array_equal(dev_rows, bits[tiles])
    del mask, o, lse, qd, kd, vd, dod
    say(f"limits L={w.L} 16x8 backward: oracle dQ on {len(tiles)} tiles")
    qr, rdq, _, _, _ = obwd.attention_bwd_rows(q[0, 0], k[0, 0], v[0, 0], do[0, 0], bits, w.M, w.N, w.scale,
                                               q_tiles=tiles, k_rows=None, group=16)
    g = dq[0, 0, torch.from_numpy(qr).cuda()].float().cpu().numpy()
    err = np.abs(g - rdq)
    print(f"[parity] limits L={w.L} bwd dQ: max_abs={err.max():.3e} mean_abs={err.mean():.3e}", flush=True)
    assert np.all(np.isfinite(g))
    assert err.max() <= 2e-2 * max(1.0, float(np.abs(rdq).max()))
    assert err.mean() <= 1e-2 * float(np.abs(rdq).mean()) + 1e-5
    dof = do[0, 0].double().numpy()
    bound = 1e-3 * np.sqrt((dof ** 2).sum(axis=0))
    sdv = dv[0, 0].double().sum(dim=0).cpu().numpy()
    sdk = dk[0, 0].double().sum(dim=0).cpu().numpy()
    rv = np.abs(sdv - dof.sum(axis=0))
    print(f"[parity] limits L={w.L} bwd: |sum dV - sum dO| max {rv.max():.3e}, |sum dK| max "
          f"{np.abs(sdk).max():.3e} (bound {bound.min():.3e})", flush=True)
    assert np.all(rv <= bound) and np.all(np.abs(sdk) <= bound)


@pytest.mark.timeout(600)
def test_mask_calls_at_maximum_heads():
    """Compaction and mask diff over B*H = 2^20 heads at L = 272 (17 query
    tiles of 34 key tiles, 16x8): 17.8 million bitmap rows, so the count,
    fill and diff kernels all step through more work than their capped grids
    hold.  Sampled rows bit for bit against the host generator's rows: each
    row's list between its row_ptr entries, its diff count, and whole heads'
    diff sums; row_ptr starts at 0, never decreases and ends at the list
    length."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    B, H, L, M, N = 16, BH_MAX // 16, 272, 16, 8
    wa = W.Workload("maxheads_ma", B, H, L, 64, M, N, "bf16", W.MaskRecipe("hash", p_near=0.3, p_far=0.3), 201)
    wb = W.Workload("maxheads_mb", B, H, L, 64, M, N, "bf16", W.MaskRecipe("hash", p_near=0.3, p_far=0.3), 202)
    say(f"limits B*H={B * H} L={L}: masks, compaction, diff")
    a = T.maskgen_hash(B, H, L, M, N, **W.hash_params(wa))
    b = T.maskgen_hash(B, H, L, M, N, **W.hash_params(wb))
    row_ptr, col_idx = T.mask_compact(a, L, M, N)
    rows_changed, heads_changed = T.mask_diff(a, b, L, M, N)
    torch.cuda.synchronize()
    n_rows = B * H * wa.T_q
    assert int(row_ptr[0]) == 0 and int(row_ptr[-1]) == col_idx.numel()
    assert bool((row_ptr[1:] >= row_ptr[:-1]).all())
    rng = np.random.default_rng(31)
    heads = [(0, 0), (B - 1, H - 1), (7, 4096)] + [(int(x), int(y)) for x, y in
                                                   zip(rng.integers(0, B, 5), rng.integers(0, H, 5))]
    rc = rows_changed.cpu().numpy()
    hc = heads_changed.cpu().numpy()
    for bb, hh in heads:
        keys = [(bb, hh, i) for i in range(wa.T_q)]
        ka, kb = W.mask_rows_bool(wa, keys), W.mask_rows_bool(wb, keys)
        assert np.array_equal(a[bb, hh].cpu().numpy().view(np.uint32), W.pack_bits(ka))
        assert np.array_equal(b[bb, hh].cpu().numpy().view(np.uint32), W.pack_bits(kb))
        diff = (ka != kb).sum(axis=1)
        assert np.array_equal(rc[bb, hh], diff) and hc[bb, hh] == diff.sum()
        for i in range(wa.T_q):
            r = (bb * H + hh) * wa.T_q + i
            lo, hi = int(row_ptr[r]), int(row_ptr[r + 1])
            assert np.array_equal(col_idx[lo:hi].cpu().numpy(), np.flatnonzero(ka[i]))
    print(f"[parity] limits B*H={B * H} L={L}: {n_rows} rows, {col_idx.numel()} kept tiles; "
          f"{len(heads)} heads' lists and diff counts exact", flush=True)


@pytest.mark.timeout(600)
def test_predictor_at_maximum_heads():
    """The mask predictor over B*H = 2^20 heads (L = 48, d = 64, 16x16 tiles:
    3 x 3 pooled scores per head, the top one of three kept at 50%): 2^20
    work-groups of the fused score-and-select kernel in one launch.  Sampled heads
    against the oracle predictor: exactly k kept per row, and every tile
    clearly above (below) the oracle's k-th score kept (dropped)."""
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    from oracle import predictor as opred
    B, H, L, d, M, N, sp = 16, BH_MAX // 16, 48, 64, 16, 16, 50
    src = W.Workload("maxheads_pred", 1, 4096, L, d, M, N, "bf16",
                     W.MaskRecipe("predicted", sparsity_percent=sp), 301)
    say(f"limits B*H={B * H} L={L}: predictor")
    (qd, kd, _), (q, k, _) = _max_heads_inputs(src, B, H)
    bits = T.predict_mask(qd, kd, M, N, sp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(37)
    heads = [(0, 0), (B - 1, H - 1), (0, 65534), (0, 65535), (1, 0)] + \
            [(int(x), int(y)) for x, y in zip(rng.integers(0, B, 5), rng.integers(0, H, 5))]
    T_k = -(-L // N)
    kk = opred.topk_count(T_k, sp)
    for bb, hh in heads:
        s = opred.pooled_scores(q[0, hh % src.H], k[0, hh % src.H], M, N)
        keep = oracle.unpack_mask(bits[bb, hh].cpu().numpy().view(np.uint32), T_k)
        assert np.all(keep.sum(axis=1) == kk)
        thr = -np.sort(-s, axis=1)[:, kk - 1]
        delta = 1e-4 * np.abs(s).max(axis=1) + 1e-6
        assert np.all(keep[s > (thr + delta)[:, None]]) and not np.any(keep[s < (thr - delta)[:, None]])
