"""Seeded input generators: published test vectors, format round trips and
statistical bands of the mask recipes (CPU only)."""
import numpy as np
import pytest

import oracle
import workloads as W


def test_splitmix64_published_vectors():
    # SplitMix64 (Steele, Lea & Flood 2014; Vigna's reference splitmix64.c):
    # state 0 yields 0xe220a8397b1dcdaf, 0x6e789e6aa1b965f4, 0x06c45d188009454f.
    z = W.splitmix64(0, np.arange(3))
    assert [int(x) for x in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_pack_bits_roundtrip_with_oracle_unpack():
    rng = np.random.default_rng(0)
    for T_k in (1, 31, 32, 33, 70, 4095):
        keep = rng.random((3, T_k)) < 0.3
        bits = W.pack_bits(keep)
        assert bits.shape == (3, -(-T_k // 32)) and bits.dtype == np.uint32
        assert np.array_equal(oracle.unpack_mask(bits, T_k), keep)
        # padding bits are zero
        if T_k % 32:
            assert np.all(bits[:, -1] >> np.uint32(T_k % 32) == 0)


def _binom_ok(k, n, p, sig=4.0):
    return abs(k - n * p) <= sig * np.sqrt(n * p * (1 - p)) + 1


def test_tiny_mask_diag_and_rate():
    w = W.get("tiny")
    bits = W.mask_bits(w)
    keep = oracle.unpack_mask(bits, w.T_k)
    for h in range(w.H):
        assert np.all(np.diag(keep[0, h]))
        off = ~np.eye(w.T_q, dtype=bool)
        assert _binom_ok(int(keep[0, h][off].sum()), int(off.sum()), 0.5)


def test_frame_structured_rates():
    w = W.get("wan480_fine")
    assert abs(w.mask.p_near - 0.717099) < 1e-6 and abs(w.mask.p_far - 0.179275) < 1e-6
    rows = [(0, h, i) for h in (0, 39) for i in (0, 700, 1400, 2047)]
    keep = W.mask_rows_bool(w, rows)
    fk = np.arange(w.T_k) * w.N // 1560
    for (b, h, i), kr in zip(rows, keep):
        fq = i * w.M // 1560
        near = np.abs(fk - fq) <= 2
        d = W.diag_tiles(w, i)
        assert np.all(kr[d])
        nd = np.ones(w.T_k, dtype=bool)
        nd[d] = False
        assert _binom_ok(int(kr[near & nd].sum()), int((near & nd).sum()), w.mask.p_near)
        assert _binom_ok(int(kr[~near & nd].sum()), int((~near & nd).sum()), w.mask.p_far)


def test_frame_structured_expected_fraction():
    w = W.get("wan480_fine")
    fq = np.arange(w.T_q) * w.M // 1560
    fk = np.arange(w.T_k) * w.N // 1560
    near = np.abs(fq[:, None] - fk[None, :]) <= 2
    expected = (near * w.mask.p_near + ~near * w.mask.p_far).mean()
    assert abs(expected - 0.30) < 1e-9


def test_diag_tiles_reading():
    w = W.get("wan480_fine")
    assert W.diag_tiles(w, 5).tolist() == [10, 11]
    assert W.diag_tiles(w, w.T_q - 1).tolist() == [w.T_k - 1]      # last tile: 8 rows
    w4 = W.get("wan720_n1")
    assert W.diag_tiles(w4, 3).tolist() == list(range(48, 64))


def test_n1_rows_rate():
    w = W.get("wan720_n1")
    keep = W.mask_rows_bool(w, [(0, 7, 100), (0, 39, w.T_q - 1)])
    for i, kr in zip((100, w.T_q - 1), keep):
        d = W.diag_tiles(w, i)
        assert np.all(kr[d])
        nd = np.ones(w.T_k, dtype=bool)
        nd[d] = False
        assert _binom_ok(int(kr[nd].sum()), int(nd.sum()), 0.2)


def test_exact_drop_counts():
    w = W.get("wan480_coarse").replace(H=2)
    bits = W.mask_bits(w)
    keep = oracle.unpack_mask(bits, w.T_k)
    for h in range(2):
        assert int(keep[0, h].sum()) == 512 * 512 - 183501
        assert np.all(np.diag(keep[0, h]))
    assert not np.array_equal(keep[0, 0], keep[0, 1])


def test_sample_tiles():
    w = W.get("wan480_fine")
    s = W.sample_tiles(w)
    assert s.shape == (1, 40, 256)
    for h in range(40):
        t = s[0, h]
        assert t[0] == 0 and t[-1] == w.T_q - 1 and len(set(t.tolist())) == 256
        assert np.all(np.diff(t) > 0)
    small = W.get("tiny")
    assert W.sample_tiles(small).shape == (1, 2, 32)


def test_qkv_shapes_and_offsets():
    import torch
    w = W.get("hunyuan720").replace(H=2, L=7300, offset_frame_tokens=3600)
    q, k, v = W.make_qkv(w)
    assert q.shape == (1, 2, 7300, 128) and q.dtype == torch.bfloat16
    # the shared per-frame offset shows up as correlated frame means in Q and K, not in V
    qm = q[0, 0, :3600].float().mean(0)
    km = k[0, 0, :3600].float().mean(0)
    vm = v[0, 0, :3600].float().mean(0)
    assert torch.corrcoef(torch.stack([qm, km]))[0, 1] > 0.9
    assert vm.abs().max() < 0.1
    q1, _, _ = W.make_qkv(w, heads=1)
    assert torch.equal(q1[0, 0], q[0, 0])


@pytest.mark.parametrize("name", ["tiny", "wan480_fine"])
def test_generation_is_deterministic(name):
    w = W.get(name)
    if w.L > 4096:
        w = w.replace(H=1)
        a = W.mask_rows_bool(w, [(0, 0, 3)])
        b = W.mask_rows_bool(w, [(0, 0, 3)])
    else:
        a, b = W.mask_bits(w), W.mask_bits(w)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# Structured patterns: the tile-level closed forms of the host generator
# against the token-level rules by brute force (a tile is kept iff its rule
# holds for some query/key token pair inside it).
# --------------------------------------------------------------------------
def _brute_structured(L, M, N, pat, dw, bw, F, reach, P, sw):
    q = np.arange(L)[:, None]
    k = np.arange(L)[None, :]
    if pat == W.gen.PATTERN_EMPTY:
        tok = np.zeros((L, L), dtype=bool)
    elif pat == W.gen.PATTERN_DENSE:
        tok = np.ones((L, L), dtype=bool)
    elif pat == W.gen.PATTERN_DIAGONAL:
        tok = np.abs(q - k) <= dw
    elif pat == W.gen.PATTERN_MULTI_DIAGONAL:
        tok = np.zeros((L, L), dtype=bool)
        for t in range(-reach, reach + 1):
            tok |= np.abs(q - k - t * F) <= bw
    else:
        tok = np.broadcast_to((k % P) < sw, (L, L))
    T_q, T_k = -(-L // M), -(-L // N)
    out = np.zeros((T_q, T_k), dtype=bool)
    for i in range(T_q):
        for j in range(T_k):
            out[i, j] = tok[i * M:(i + 1) * M, j * N:(j + 1) * N].any()
    return out


@pytest.mark.parametrize("L,M,N", [(97, 16, 1), (200, 16, 8), (257, 32, 4), (300, 64, 64), (130, 16, 16)])
def test_structured_masks_match_token_rules(L, M, N):
    dw, bw, F, reach, P, sw = 13, 3, 40, 3, 24, 5
    pats = (0, 1, 2, 3, 4)
    w = W.Workload("s", 1, len(pats), L, 64, M, N, "bf16",
                   W.MaskRecipe("structured", frame_tokens=F, patterns=pats, diag_width=dw,
                                band_width=bw, reach=reach, stripe_period=P, stripe_width=sw,
                                force_diag=False), 1)
    for h, pat in enumerate(pats):
        rows = np.stack([np.zeros(w.T_q, int), np.full(w.T_q, h), np.arange(w.T_q)], 1)
        got = W.mask_rows_bool(w, rows)
        ref = _brute_structured(L, M, N, pat, dw, bw, F, reach, P, sw)
        assert np.array_equal(got, ref), (L, M, N, pat)


def test_struct_workload_densities():
    w = W.get("wan480_struct")
    assert w.mask.patterns.count(W.gen.PATTERN_EMPTY) == 2
    dens = {}
    for h in (0, 5, 20, 35):
        rows = np.stack([np.zeros(w.T_q, int), np.full(w.T_q, h), np.arange(w.T_q)], 1)
        dens[h] = W.mask_rows_bool(w, rows).mean()
    assert dens[0] == 0.0
    assert 0.25 < dens[5] < 0.31 and 0.15 < dens[20] < 0.20 and 0.24 < dens[35] < 0.27
