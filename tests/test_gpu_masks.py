"""GPU mask generator and mask compaction against the host generator and the
CPU oracle (bit-exact), through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import mask_to_np, say, to_dev_mask, torch_or_skip

pytestmark = pytest.mark.gpu


def _gpu_mask(w):
    import tile_sparse_attention_amd as T
    return T.maskgen_hash(w.B, w.H, w.L, w.M, w.N, **W.hash_params(w))


def _rows_of(bits_np, rows):
    return np.stack([bits_np[b, h, i] for b, h, i in rows])


@pytest.mark.parametrize("name", ["tiny", "wan480_fine", "wan720_n1"])
def test_maskgen_matches_host_generator(name):
    torch = torch_or_skip()
    w = W.get(name)
    say(f"maskgen {name}")
    m = mask_to_np(_gpu_mask(w))
    rng = np.random.default_rng(1)
    rows = [(0, h, i) for h in range(w.H) for i in {0, w.T_q - 1, int(rng.integers(w.T_q))}]
    host = W.pack_bits(W.mask_rows_bool(w, rows))
    assert np.array_equal(_rows_of(m, rows), host)
    # padding bits are zero
    if w.T_k % 32:
        assert np.all(m[..., -1] >> np.uint32(w.T_k % 32) == 0)
    torch.cuda.synchronize()


def test_maskgen_small_shapes_full():
    torch_or_skip()
    for L, M, N in [(1, 16, 1), (100, 16, 8), (1000, 32, 2), (777, 64, 64)]:
        w = W.Workload("g", 2, 3, L, 64, M, N, "bf16",
                       W.MaskRecipe("hash", p_near=0.37, p_far=0.11, frame_tokens=50,
                                    frame_radius=1), 77)
        say(f"maskgen full L={L} {M}x{N}")
        assert np.array_equal(mask_to_np(_gpu_mask(w)), W.mask_bits(w))


def _compact(bits_dev, w, cap=None):
    import tile_sparse_attention_amd as T
    rp, ci = T.mask_compact(bits_dev, w.L, w.M, w.N, col_capacity=cap)
    return rp.cpu().numpy(), ci.cpu().numpy()


@pytest.mark.parametrize("L,M,N", [(512, 16, 16), (1000, 16, 1), (1000, 16, 8), (3000, 64, 64),
                                   (77, 16, 2), (1, 16, 4)])
def test_compaction_bit_exact_small(L, M, N):
    torch_or_skip()
    w = W.Workload("c", 2, 3, L, 64, M, N, "bf16", W.MaskRecipe("hash", p_near=0.3, p_far=0.3), 5)
    say(f"compaction L={L} {M}x{N}")
    bits = W.mask_bits(w)
    if w.T_k % 32:                                   # set the padding bits: they must be ignored
        bits[..., -1] |= np.uint32(0xFFFFFFFF) << np.uint32(w.T_k % 32)
    rp, ci = _compact(to_dev_mask(bits), w)
    orp, oci = oracle.compact(bits, w.T_k)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)


def test_compaction_capacity_clipping():
    torch_or_skip()
    w = W.Workload("c", 1, 2, 640, 64, 16, 8, "bf16", W.MaskRecipe("hash", p_near=0.4, p_far=0.4), 9)
    say("compaction capacity clip")
    bits = W.mask_bits(w)
    orp, oci = oracle.compact(bits, w.T_k)
    cap = int(orp[-1]) // 2
    rp, ci = _compact(to_dev_mask(bits), w, cap=cap)
    assert np.array_equal(rp, orp)
    assert np.array_equal(ci[:cap], oci[:cap])


def test_compaction_empty_and_full_rows():
    torch_or_skip()
    w = W.Workload("c", 1, 1, 300, 64, 16, 4, "bf16", W.MaskRecipe("ones"), 1)
    bits = W.mask_bits(w)
    bits[0, 0, ::2] = 0
    say("compaction empty/full rows")
    rp, ci = _compact(to_dev_mask(bits), w)
    orp, oci = oracle.compact(bits, w.T_k)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)


def test_compaction_wan480_fine_full():
    """Every row of the 40-head 16x8 bitmap (host-generated), bit-exact."""
    torch_or_skip()
    w = W.get("wan480_fine")
    say("compaction wan480_fine full (host mask)")
    bits = W.mask_bits(w)
    rp, ci = _compact(to_dev_mask(bits), w)
    orp, oci = oracle.compact(bits, w.T_k)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)


def test_compaction_wan720_n1_sampled_rows():
    """16x1 on the 75600-token shape: the full lists (2.9e9 entries) are built
    on the GPU; counts and lists of sampled rows are compared with the oracle
    applied to the host generator's rows (equal to the GPU mask's rows, which
    is asserted first)."""
    torch = torch_or_skip()
    w = W.get("wan720_n1")
    say("compaction wan720_n1 sampled rows")
    m = _gpu_mask(w)
    rp_d, ci_d = __import__("tile_sparse_attention_amd").mask_compact(m, w.L, w.M, w.N)
    tiles = W.sample_tiles(w, per_head=16)
    rows = [(0, h, int(i)) for h in (0, 17, 39) for i in tiles[0, h]]
    host = W.pack_bits(W.mask_rows_bool(w, rows))
    assert np.array_equal(_rows_of(mask_to_np(m), rows), host)
    rp = rp_d.cpu().numpy()
    for (b, h, i), hr in zip(rows, host):
        r = (b * w.H + h) * w.T_q + i
        lst = ci_d[rp[r]:rp[r + 1]].cpu().numpy()
        _, oci = oracle.compact(hr[None, None, None], w.T_k)
        assert np.array_equal(lst, oci)
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0)
    del ci_d
    torch.cuda.empty_cache()


def test_structured_maskgen_matches_host():
    torch_or_skip()
    import tile_sparse_attention_amd as T
    for L, M, N in [(1000, 16, 8), (777, 64, 64), (1000, 16, 1), (513, 32, 4)]:
        pats = (0, 1, 2, 3, 4, 2)
        w = W.Workload("s", 2, len(pats), L, 64, M, N, "bf16",
                       W.MaskRecipe("structured", frame_tokens=97, patterns=pats, diag_width=60,
                                    band_width=7, reach=4, stripe_period=50, stripe_width=9,
                                    force_diag=False), 1)
        say(f"structured maskgen L={L} {M}x{N}")
        m = mask_to_np(T.maskgen_structured(w.B, w.H, w.L, w.M, w.N, **W.structured_params(w)))
        assert np.array_equal(m, W.mask_bits(w)), (L, M, N)


def test_structured_maskgen_full_config_sampled():
    torch_or_skip()
    import tile_sparse_attention_amd as T
    w = W.get("wan480_struct")
    say("structured maskgen wan480_struct")
    m = mask_to_np(T.maskgen_structured(w.B, w.H, w.L, w.M, w.N, **W.structured_params(w)))
    rng = np.random.default_rng(3)
    rows = [(0, h, i) for h in range(w.H) for i in {0, w.T_q - 1, int(rng.integers(w.T_q))}]
    assert np.array_equal(_rows_of(m, rows), W.pack_bits(W.mask_rows_bool(w, rows)))


@pytest.mark.parametrize("L,M,N", [(1000, 16, 8), (777, 32, 1), (4000, 64, 64), (50, 16, 16), (129, 16, 2)])
def test_mask_diff_bit_exact(L, M, N):
    import tile_sparse_attention_amd as T
    torch = torch_or_skip()
    rng = np.random.default_rng(L + M + N)
    T_q, T_k = -(-L // M), -(-L // N)
    words = -(-T_k // 32)
    # random words, padding bits included: they must not count
    a = rng.integers(0, 2**32, size=(2, 3, T_q, words), dtype=np.uint64).astype(np.uint32)
    flip = rng.random(a.shape) < 0.3
    b = np.where(flip, a ^ rng.integers(0, 2**32, size=a.shape, dtype=np.uint64).astype(np.uint32), a)
    say(f"mask diff L={L} M={M} N={N} words={words}")
    rows, heads = T.mask_diff(to_dev_mask(a), to_dev_mask(b), L, M, N)
    torch.cuda.synchronize()
    r_ref, h_ref = oracle.mask_diff(a, b, T_k)
    assert np.array_equal(rows.cpu().numpy(), r_ref)
    assert np.array_equal(heads.cpu().numpy(), h_ref)
    same, _ = T.mask_diff(to_dev_mask(a), to_dev_mask(a), L, M, N)
    assert int(same.abs().max()) == 0


def test_mask_diff_wan480_fine_consecutive_masks():
    """Two masks of the 16x8 workload drawn with different seeds (a stand-in
    for masks predicted at two denoising steps): every row and head count
    equals the oracle's."""
    import tile_sparse_attention_amd as T
    torch = torch_or_skip()
    w = W.get("wan480_fine")
    w2 = W.Workload(w.name + "_next", w.B, w.H, w.L, w.d, w.M, w.N, w.dtype, w.mask, w.seed + 1000)
    a, b = W.mask_bits(w), W.mask_bits(w2)
    say("mask diff wan480_fine vs reseeded")
    rows, heads = T.mask_diff(to_dev_mask(a), to_dev_mask(b), w.L, w.M, w.N)
    torch.cuda.synchronize()
    r_ref, h_ref = oracle.mask_diff(a, b, w.T_k)
    assert np.array_equal(rows.cpu().numpy(), r_ref)
    assert np.array_equal(heads.cpu().numpy(), h_ref)


@pytest.mark.parametrize("shift", [1, 2, 3])
def test_compaction_into_a_list_not_16_byte_aligned(shift):
    """col_idx at 4-byte but not 16-byte alignment (the fill stores aligned
    16-byte runs, so its alignment follows the list's address), with a
    capacity that clips inside a run; the slots around the list stay intact."""
    torch = torch_or_skip()
    import ctypes

    import tile_sparse_attention_amd as T
    w = W.Workload("c", 2, 3, 1000, 64, 16, 1, "bf16", W.MaskRecipe("hash", p_near=0.3, p_far=0.3), 15)
    say(f"compaction col_idx offset {shift} ints")
    bits = W.mask_bits(w)
    orp, oci = oracle.compact(bits, w.T_k)
    nnz = int(orp[-1])
    cap = nnz - 5
    buf = torch.full((nnz + 8,), -7, dtype=torch.int32, device="cuda")
    rp = torch.empty(orp.size, dtype=torch.int64, device="cuda")
    m = to_dev_mask(bits)
    pr = T.problem(w.B, w.H, w.L, 0, w.M, w.N)
    ws, nws = T._workspace(T.OP_MASK_COMPACT, pr, m.device)
    T._check(T.lib().tsa_mask_compact(ctypes.byref(pr), T._ptr(m), T._ptr(rp),
                                      ctypes.c_void_p(buf.data_ptr() + 4 * shift), cap, T._ptr(ws), nws,
                                      T._stream()))
    got = buf.cpu().numpy()
    assert np.array_equal(rp.cpu().numpy(), orp)
    assert np.array_equal(got[shift:shift + cap], oci[:cap])
    assert np.all(got[:shift] == -7) and np.all(got[shift + cap:] == -7)
