"""GPU parity of the tile-sparse attention forward kernel against the fp64
CPU oracle, through the C ABI, on seeded synthetic inputs."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (compare, full_compare, gpu_attention, say, small_workload, to_dev_mask,
                      torch_or_skip)

pytestmark = pytest.mark.gpu


def _hash_bits(w):
    return W.mask_bits(w)


def test_tiny_config_full():
    torch_or_skip()
    w = W.get("tiny")
    full_compare(w, W.mask_bits(w), "tiny fp32 16x16 (full)")


@pytest.mark.parametrize("M", [16, 32, 64])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 32, 64])
def test_bf16_tile_grid_ragged(M, N):
    torch_or_skip()
    # L = 1000 leaves a partial last query tile for every M and a partial last
    # key tile for N in {16, 32, 64}; 1000 is not a multiple of the key chunk.
    w = small_workload(f"grid_{M}x{N}", 1000, 128, M, N, p=0.3, seed=100 + M + N)
    full_compare(w, _hash_bits(w), f"bf16 d128 {M}x{N} L=1000")


@pytest.mark.parametrize("N,L", [(8, 1001), (16, 1003), (32, 997), (64, 1029), (8, 13)])
def test_bf16_sequence_ends_inside_an_octet(N, L):
    torch_or_skip()
    # L is not a multiple of 8: the last kept key tile has keys past L in its
    # last 8-key run, which must take no part in the softmax (numerator or
    # denominator).
    w = small_workload(f"oct_tail_{N}_{L}", L, 128, 16, N, p=0.3, seed=7 * N + L)
    full_compare(w, _hash_bits(w), f"bf16 d128 16x{N} L={L}")


@pytest.mark.parametrize("M,N", [(16, 8), (16, 16), (64, 64), (32, 8)])
def test_bf16_banded_mask_skips_chunks(M, N):
    torch_or_skip()
    # Each query tile keeps key tiles within a band around the diagonal, and
    # the rows of the second 256-row group keep nothing: most 128-key chunks
    # are needed by no row of a 256-row group (the chunk-skipping kernel).
    L = 3000
    w = small_workload(f"band_{M}x{N}", L, 128, M, N, seed=31 + M + N)
    rng = np.random.default_rng(M * 100 + N)
    keep = np.zeros((1, 2, w.T_q, w.T_k), dtype=bool)
    for h in range(2):
        for i in range(w.T_q):
            r0 = i * M
            if 256 <= r0 < 512:
                continue
            lo = max(0, (r0 - 200) // N)
            hi = min(w.T_k, (r0 + M + 200) // N + 1)
            keep[0, h, i, lo:hi] = rng.random(hi - lo) < 0.5
            keep[0, h, i, min(w.T_k - 1, r0 // N)] = True
    full_compare(w, W.pack_bits(keep), f"bf16 banded {M}x{N} L={L}")


@pytest.mark.parametrize("M,N", [(16, 8), (16, 16), (64, 64), (16, 1)])
def test_bf16_structured_masks_and_skipped_heads(M, N):
    torch_or_skip()
    # one head per pattern of the structured generator, two of them empty
    # (skipped heads: output zero, LSE -inf)
    pats = (0, 1, 2, 3, 4, 0)
    L = 2100
    w = W.Workload(f"struct_{M}x{N}", 1, len(pats), L, 128, M, N, "bf16",
                   W.MaskRecipe("structured", frame_tokens=330, patterns=pats, diag_width=300,
                                band_width=20, reach=3, stripe_period=260, stripe_width=40,
                                force_diag=False), 41 + M + N)
    full_compare(w, W.mask_bits(w), f"bf16 structured {M}x{N} L={L}")


def test_bf16_one_skipped_head_among_dense_heads():
    torch_or_skip()
    # One head with an all-zero mask among heads whose work-groups need every
    # chunk: only that head's work-groups take the chunk-skipping kernel.
    w = small_workload("one_empty", 3000, 128, 16, 8, H=8, p=0.5, seed=9)
    bits = W.mask_bits(w)
    bits[0, 3] = 0
    full_compare(w, bits, "bf16 16x8 L=3000, head 3 skipped")


@pytest.mark.parametrize("dtype,d,N", [("f32", 128, 8), ("f32", 64, 1), ("f32", 64, 4),
                                       ("bf16", 64, 8), ("bf16", 64, 1), ("f32", 128, 64)])
def test_dtype_and_head_dim(dtype, d, N):
    torch_or_skip()
    w = small_workload(f"dt_{dtype}_{d}_{N}", 777, d, 16, N, dtype=dtype, p=0.4, seed=5 + d + N)
    full_compare(w, _hash_bits(w), f"{dtype} d{d} 16x{N} L=777")


@pytest.mark.parametrize("L", [1, 15, 17, 130, 257])
def test_short_sequences(L):
    torch_or_skip()
    w = small_workload(f"short_{L}", L, 128, 16, 4, p=0.5, seed=L)
    full_compare(w, _hash_bits(w), f"bf16 16x4 L={L}")


# kept key tiles per (query tile, 128-key chunk), cycled over tiles and
# chunks: every count a pass boundary of the kernels can fall on (the key
# kernel packs 32 keys per pass and runs a last pass with <= 16 real keys on
# one score block; the octet kernel packs 4 octets and runs a last pass with
# <= 2 real octets on one block)
_PASS_COUNTS = {1: (0, 1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 100, 127, 128),
                2: (0, 1, 7, 8, 9, 15, 16, 17, 24, 31, 32, 33, 48, 63, 64),
                4: (0, 1, 3, 4, 5, 7, 8, 9, 15, 16, 17, 24, 31, 32),
                8: (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 15, 16),
                16: (0, 1, 2, 3, 4, 5, 6, 7, 8)}


@pytest.mark.parametrize("N,d", [(1, 128), (2, 128), (4, 128), (8, 128), (16, 128), (1, 64), (8, 64)])
def test_kept_counts_at_pass_boundaries(N, d):
    torch_or_skip()
    L = 2048 + 77   # 16 whole chunks and a partial one
    w = small_workload(f"passes_{N}_{d}", L, d, 16, N, seed=200 + N + d)
    tpc = 128 // N
    counts = _PASS_COUNTS[N]
    rng = np.random.default_rng(N)
    keep = np.zeros((1, w.H, w.T_q, w.T_k), dtype=bool)
    for h in range(w.H):
        for i in range(w.T_q):
            for c in range(-(-w.T_k // tpc)):
                j0, j1 = c * tpc, min(c * tpc + tpc, w.T_k)
                n = min(counts[(i + 3 * c + h) % len(counts)], j1 - j0)
                keep[0, h, i, j0 + rng.choice(j1 - j0, n, replace=False)] = True
    full_compare(w, W.pack_bits(keep), f"bf16 d={d} 16x{N} kept counts at pass boundaries")


def test_empty_mask_gives_zero_and_minus_inf():
    torch = torch_or_skip()
    w = small_workload("empty", 300, 128, 16, 8)
    say("empty mask bf16 16x8 L=300")
    q, k, v = W.make_qkv(w)
    bits = np.zeros((1, 2, w.T_q, w.words), dtype=np.uint32)
    o, lse = gpu_attention(q.cuda(), k.cuda(), v.cuda(), to_dev_mask(bits), 16, 8, w.scale)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_padding_bits_are_ignored():
    torch_or_skip()
    w = small_workload("pad", 1000, 128, 16, 8, p=0.3, seed=3)     # T_k = 125: 3 padding bits
    bits = W.mask_bits(w)
    bits[..., -1] |= np.uint32(0xE0000000)
    full_compare(w, bits, "bf16 16x8 padding bits set")


def test_all_ones_and_diagonal_only():
    torch_or_skip()
    w = small_workload("ones", 700, 128, 16, 8, seed=11)
    full_compare(w, W.pack_bits(np.ones((1, 2, w.T_q, w.T_k), dtype=bool)), "bf16 all-ones")
    wd = w.replace(mask=W.MaskRecipe("diag_only"))
    full_compare(wd, W.mask_bits(wd), "bf16 diagonal-only")


def test_single_tile_rows_and_last_partial_tile():
    torch_or_skip()
    w = small_workload("single", 1000, 128, 16, 16, seed=13)
    rng = np.random.default_rng(0)
    keep = np.zeros((1, 2, w.T_q, w.T_k), dtype=bool)
    for h in range(2):
        for i in range(w.T_q):
            keep[0, h, i, rng.integers(w.T_k)] = True
        keep[0, h, ::3, w.T_k - 1] = True       # partial last key tile (8 keys)
    full_compare(w, W.pack_bits(keep), "bf16 one tile per row + last partial key tile")


def test_large_logits_are_stable():
    torch = torch_or_skip()
    w = small_workload("big", 600, 128, 16, 8, p=0.5, seed=17)
    say("bf16 16x8 L=600 with Q scaled x8 (large logits)")
    q, k, v = W.make_qkv(w)
    q = (q.float() * 8).to(torch.bfloat16)
    bits = W.mask_bits(w)
    o, lse = gpu_attention(q.cuda(), k.cuda(), v.cuda(), to_dev_mask(bits), 16, 8, w.scale)
    ro, rl = oracle.attention(q, k, v, bits, 16, 8, w.scale)
    compare("large logits", o.float().cpu().numpy(), ro, "bf16", lse.cpu().numpy(), rl)


def test_determinism():
    torch = torch_or_skip()
    w = small_workload("det", 2000, 128, 16, 8, p=0.3, seed=19)
    say("determinism bf16 16x8 L=2000")
    q, k, v = (x.cuda() for x in W.make_qkv(w))
    m = to_dev_mask(W.mask_bits(w))
    o1, l1 = gpu_attention(q, k, v, m, 16, 8, w.scale)
    o2, l2 = gpu_attention(q, k, v, m, 16, 8, w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_multi_batch_heads():
    torch_or_skip()
    w = W.Workload("bh", 2, 3, 500, 128, 16, 8, "bf16",
                   W.MaskRecipe("hash", p_near=0.35, p_far=0.35), 23)
    full_compare(w, W.mask_bits(w), "bf16 B=2 H=3 16x8 L=500")


@pytest.mark.parametrize("dtype,d,N", [("bf16", 128, 8), ("bf16", 128, 16), ("bf16", 128, 1),
                                       ("bf16", 64, 1), ("f32", 64, 16), ("f32", 128, 8)])
def test_negative_scale(dtype, d, N):
    torch_or_skip()
    # A negative scale flips the sign of every logit; the bf16 kernels take it
    # by negating Q (exact), the f32 kernel by the signed scale.  Both the
    # octet kernel (N >= 8) and the key kernel (N < 8) are reached.
    w = small_workload(f"neg_{dtype}_{d}_{N}", 1000, d, 16, N, dtype=dtype, p=0.4, seed=61 + d + N)
    full_compare(w, _hash_bits(w), f"{dtype} d{d} 16x{N} L=1000 scale<0", scale=-w.scale)


def test_timing_events_bracket_the_attention_kernels():
    torch = torch_or_skip()
    import tile_sparse_attention_amd as T
    # events recorded around the attention kernels proper: same results, and
    # their span lies inside the whole call's
    w = small_workload("tev", 3000, 128, 16, 8, H=4, p=0.3, seed=91)
    say("timing events bf16 16x8 L=3000")
    q, k, v = (x.cuda() for x in W.make_qkv(w))
    m = to_dev_mask(W.mask_bits(w))
    o1 = T.attention_fwd(q, k, v, m, 16, 8, w.scale)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    T.set_timing_events(a, b)
    try:
        c0.record()
        o2 = T.attention_fwd(q, k, v, m, 16, 8, w.scale)
        c1.record()
    finally:
        T.set_timing_events(None, None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    kern, call = a.elapsed_time(b), c0.elapsed_time(c1)
    assert 0 < kern <= call
