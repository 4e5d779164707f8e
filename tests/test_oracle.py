"""Pins of the CPU oracle against things other than itself.

Each check ties the oracle to hand-worked fixtures (tests/golden/), brute
force written independently (pure-Python loops), a library routine for the
dense special case (torch's scaled_dot_product_attention in float64), closed
forms and invariants of the definition.  The mutation tests at the end plant
plausible mistakes in a copy of the oracle and confirm a pin catches each.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import sparse_attention as oatt
from oracle import predictor as opred

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _frac(s):
    return float(Fraction(s))


def _pack(keep):
    """Independent bit packer for test inputs (explicit loop, LSB first)."""
    keep = np.asarray(keep, dtype=bool)
    T_k = keep.shape[-1]
    nw = -(-T_k // 32)
    out = np.zeros(keep.shape[:-1] + (nw,), dtype=np.uint32)
    it = np.ndindex(keep.shape[:-1])
    for idx in it:
        for j in range(T_k):
            if keep[idx + (j,)]:
                out[idx + (j // 32,)] |= np.uint32(1 << (j % 32))
    return out


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, scale, keep=None):
    """torch float64 scaled_dot_product_attention on [L, d] operands."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x))[None, None] for x in (q, k, v))
    mask = None if keep is None else torch.from_numpy(keep)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=scale)[0, 0].numpy()


# --------------------------------------------------------------------------
# hand-worked fixtures
# --------------------------------------------------------------------------
def test_golden_ragged_tiles_and_empty_row():
    g = _load("attention_handworked_ragged.json")
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    bits = np.array(g["mask_words"], dtype=np.uint32)[None, None]
    o, lse = oracle.attention(q, k, v, bits, g["M"], g["N"], g["scale"])
    exp_o = np.array([[_frac(x) for x in row] for row in g["expected_o"]])
    exp_lse = np.array([-np.inf if s == "-inf" else math.log(int(s[2:])) for s in g["expected_lse"]])
    np.testing.assert_allclose(o[0, 0], exp_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], exp_lse, rtol=0, atol=1e-12)


def test_golden_multiword_n1_bit_order():
    g = _load("attention_handworked_multiword_n1.json")
    q = np.array(g["q"])
    k = np.array(g["k"])
    v = np.array(g["v"])
    bits = np.array(g["mask_words"], dtype=np.uint32)
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], bits[None, None],
                              g["M"], g["N"], g["scale"])
    o, lse = o[0, 0], lse[0, 0]
    for span, val in g["expected_o_rows"].items():
        a, b = (int(x) for x in span.split("-"))
        np.testing.assert_allclose(o[a:b + 1], np.tile(val, (b - a + 1, 1)), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse[0:16], 0.5 * q[0:16] @ k[33], atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse[16:32], math.log(2), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse[32:40], 0.5 * q[32:40] @ k[5], atol=1e-12, rtol=0)


def test_golden_compaction():
    g = _load("compaction_handworked.json")
    bits = np.array(g["mask_words"], dtype=np.uint32)[None, None]
    rp, ci = oracle.compact(bits, g["T_k"])
    assert rp.tolist() == g["expected_row_ptr"]
    assert ci.tolist() == g["expected_col_idx"]
    assert rp.dtype == np.int64 and ci.dtype == np.int32


def test_golden_predictor():
    g = _load("predictor_handworked.json")
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    for case in g["cases"]:
        got = oracle.predict_mask(q, k, g["M"], g["N"], case["sparsity_percent"])
        assert got[0, 0].tolist() == case["expected_words"]


# --------------------------------------------------------------------------
# dense special case: a library routine
# --------------------------------------------------------------------------
@pytest.mark.parametrize("L,d,M,N", [(50, 8, 16, 4), (33, 16, 16, 1), (64, 4, 64, 64)])
def test_all_ones_equals_library_dense_attention(L, d, M, N):
    q, k, v = _rand((3, L, d), 1 + L)
    scale = 0.37
    T_q, T_k = -(-L // M), -(-L // N)
    bits = _pack(np.ones((1, 2, T_q, T_k), dtype=bool))
    qq = np.stack([q, -q])[None]
    kk = np.stack([k, k[::-1]])[None]
    vv = np.stack([v, v * 2])[None]
    o, lse = oracle.attention(qq, kk, vv, bits, M, N, scale)
    sc = float(np.float32(scale))
    for h in range(2):
        ref = _sdpa(qq[0, h], kk[0, h], vv[0, h], sc)
        np.testing.assert_allclose(o[0, h], ref, atol=1e-12, rtol=0)
        s = torch.from_numpy(sc * qq[0, h] @ kk[0, h].T)
        np.testing.assert_allclose(lse[0, h], torch.logsumexp(s, dim=1).numpy(), atol=1e-12)


def test_arbitrary_mask_equals_library_with_boolean_mask():
    """The library's boolean attn_mask at score granularity, built by loops."""
    L, d, M, N = 45, 6, 16, 3
    q, k, v = _rand((3, L, d), 7)
    T_q, T_k = -(-L // M), -(-L // N)
    keep_t = np.random.default_rng(3).random((T_q, T_k)) < 0.4
    keep_t[:, 0] = True
    keep = np.zeros((L, L), dtype=bool)
    for r in range(L):
        for c in range(L):
            keep[r, c] = keep_t[r // M, c // N]
    o, _ = oracle.attention(q[None, None], k[None, None], v[None, None], _pack(keep_t)[None, None],
                            M, N, 0.25)
    np.testing.assert_allclose(o[0, 0], _sdpa(q, k, v, 0.25, keep), atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# brute force in pure Python
# --------------------------------------------------------------------------
def _brute(q, k, v, keep_t, M, N, scale):
    L, d = len(q), len(q[0])
    o = [[0.0] * d for _ in range(L)]
    lse = [-math.inf] * L
    for r in range(L):
        cols = [c for c in range(L) if keep_t[r // M][c // N]]
        if not cols:
            continue
        s = {c: scale * sum(q[r][t] * k[c][t] for t in range(d)) for c in cols}
        mx = max(s.values())
        w = {c: math.exp(s[c] - mx) for c in cols}
        tot = sum(w.values())
        for t in range(d):
            o[r][t] = sum(w[c] * v[c][t] for c in cols) / tot
        lse[r] = mx + math.log(tot)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("L,d,M,N,p", [(19, 3, 16, 3, 0.5), (40, 5, 16, 1, 0.3), (37, 4, 32, 8, 0.6)])
def test_brute_force_loops(L, d, M, N, p):
    q, k, v = _rand((3, L, d), 11 * L + d)
    T_q, T_k = -(-L // M), -(-L // N)
    keep_t = np.random.default_rng(L).random((T_q, T_k)) < p
    keep_t[-1, :] = False                      # one empty query tile
    scale = 0.31
    sc = float(np.float32(scale))
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None],
                              _pack(keep_t)[None, None], M, N, scale)
    bo, blse = _brute(q.tolist(), k.tolist(), v.tolist(), keep_t.tolist(), M, N, sc)
    np.testing.assert_allclose(o[0, 0], bo, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse[0, 0], blse, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# special cases and closed forms
# --------------------------------------------------------------------------
def _diag_keep(L, M, N):
    T_q, T_k = -(-L // M), -(-L // N)
    keep = np.zeros((T_q, T_k), dtype=bool)
    for i in range(T_q):
        r0, r1 = i * M, min(i * M + M, L)
        for j in range(T_k):
            c0, c1 = j * N, min(j * N + N, L)
            keep[i, j] = c0 < r1 and r0 < c1
    return keep


@pytest.mark.parametrize("L,M,N", [(37, 8, 8), (61, 16, 8), (50, 16, 1), (70, 64, 64)])
def test_diagonal_only_equals_local_block_attention(L, M, N):
    d = 8
    q, k, v = _rand((3, L, d), L * 3 + N)
    keep = _diag_keep(L, M, N)
    o, _ = oracle.attention(q[None, None], k[None, None], v[None, None], _pack(keep)[None, None],
                            M, N, 0.5)
    for i in range(keep.shape[0]):
        r0, r1 = i * M, min(i * M + M, L)
        js = np.flatnonzero(keep[i])
        c0, c1 = js[0] * N, min(js[-1] * N + N, L)
        ref = _sdpa(q[r0:r1], k[c0:c1], v[c0:c1], 0.5)
        np.testing.assert_allclose(o[0, 0, r0:r1], ref, atol=1e-12, rtol=0)


def test_zero_queries_give_mean_of_kept_values():
    L, d, M, N = 53, 5, 16, 4
    _, k, v = _rand((3, L, d), 5)
    q = np.zeros((L, d))
    T_q, T_k = -(-L // M), -(-L // N)
    keep_t = np.random.default_rng(9).random((T_q, T_k)) < 0.5
    keep_t[:, 1] = True
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], _pack(keep_t)[None, None],
                              M, N, 1.0)
    for r in range(L):
        cols = [c for c in range(L) if keep_t[r // M, c // N]]
        np.testing.assert_allclose(o[0, 0, r], v[cols].mean(axis=0), atol=1e-13, rtol=0)
        assert abs(lse[0, 0, r] - math.log(len(cols))) < 1e-13


def test_single_kept_tile_is_local_softmax():
    L, d, M, N = 48, 6, 16, 8
    q, k, v = _rand((3, L, d), 21)
    T_q, T_k = 3, 6
    keep = np.zeros((T_q, T_k), dtype=bool)
    choice = [4, 0, 5]
    for i, j in enumerate(choice):
        keep[i, j] = True
    o, _ = oracle.attention(q[None, None], k[None, None], v[None, None], _pack(keep)[None, None],
                            M, N, 0.7)
    sc = float(np.float32(0.7))
    for i, j in enumerate(choice):
        ref = _sdpa(q[i * M:(i + 1) * M], k[j * N:(j + 1) * N], v[j * N:(j + 1) * N], sc)
        np.testing.assert_allclose(o[0, 0, i * M:(i + 1) * M], ref, atol=1e-12, rtol=0)


def test_empty_rows_are_zero_and_lse_minus_inf():
    L, d, M, N = 40, 4, 16, 8
    q, k, v = _rand((3, L, d), 2)
    bits = np.zeros((1, 1, 3, 1), dtype=np.uint32)
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], bits, M, N, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def _case(seed=0, L=64, d=8, M=16, N=8, p=0.4):
    q, k, v = _rand((3, L, d), seed)
    T_q, T_k = L // M, L // N
    keep = np.random.default_rng(seed + 1).random((T_q, T_k)) < p
    keep[:, 0] = True
    return q, k, v, keep


def _att(q, k, v, keep, M=16, N=8, scale=0.5):
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], _pack(keep)[None, None],
                              M, N, scale)
    return o[0, 0], lse[0, 0]


def test_convex_combination_of_kept_values():
    q, k, v, keep = _case(4)
    o, _ = _att(q, k, v, keep)
    for r in range(64):
        cols = [c for c in range(64) if keep[r // 16, c // 8]]
        lo, hi = v[cols].min(axis=0), v[cols].max(axis=0)
        assert np.all(o[r] >= lo - 1e-12) and np.all(o[r] <= hi + 1e-12)


def test_key_shift_invariance():
    q, k, v, keep = _case(5)
    u = _rand(8, 99)
    o1, _ = _att(q, k, v, keep)
    o2, _ = _att(q, k + u[None, :], v, keep)
    np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)


def test_value_affine_equivariance():
    q, k, v, keep = _case(6)
    o1, _ = _att(q, k, v, keep)
    o2, _ = _att(q, k, -2.5 * v + 0.75, keep)
    np.testing.assert_allclose(o2, -2.5 * o1 + 0.75, atol=1e-12, rtol=0)


def test_key_tile_permutation_invariance():
    q, k, v, keep = _case(7)
    perm = np.random.default_rng(1).permutation(8)         # key tiles of 8 keys
    key_perm = (perm[:, None] * 8 + np.arange(8)[None, :]).ravel()
    o1, _ = _att(q, k, v, keep)
    o2, _ = _att(q, k[key_perm], v[key_perm], keep[:, perm])
    np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)


def test_query_tile_permutation_equivariance():
    q, k, v, keep = _case(8)
    perm = np.random.default_rng(2).permutation(4)         # query tiles of 16 rows
    row_perm = (perm[:, None] * 16 + np.arange(16)[None, :]).ravel()
    o1, _ = _att(q, k, v, keep)
    o2, _ = _att(q[row_perm], k, v, keep[perm])
    np.testing.assert_allclose(o2, o1[row_perm], atol=1e-12, rtol=0)


def test_rows_variant_matches_full():
    L, d, M, N = 70, 6, 16, 4
    q, k, v = _rand((3, L, d), 31)
    T_q, T_k = -(-L // M), -(-L // N)
    keep = np.random.default_rng(4).random((T_q, T_k)) < 0.5
    bits = _pack(keep)
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], bits[None, None], M, N, 0.3)
    rows, o_r, lse_r = oatt.attention_rows(q, k, v, bits, M, N, 0.3, [4, 0, 2], group=2)
    assert rows.tolist() == list(range(64, 70)) + list(range(0, 16)) + list(range(32, 48))
    np.testing.assert_allclose(o_r, o[0, 0, rows], atol=0, rtol=0)
    np.testing.assert_allclose(lse_r, lse[0, 0, rows], atol=0, rtol=0)


# --------------------------------------------------------------------------
# compaction, kept FLOPs
# --------------------------------------------------------------------------
def test_compaction_brute_force_and_invariants():
    rng = np.random.default_rng(12)
    T_k = 77
    bits = rng.integers(0, 2**32, size=(2, 3, 5, 3), dtype=np.uint64).astype(np.uint32)
    rp, ci = oracle.compact(bits, T_k)
    r = 0
    for b in range(2):
        for h in range(3):
            for i in range(5):
                lst = [j for j in range(T_k) if (int(bits[b, h, i, j // 32]) >> (j % 32)) & 1]
                assert ci[rp[r]:rp[r + 1]].tolist() == lst
                pc = sum(bin(int(w)).count("1") for w in bits[b, h, i, :2]) + \
                    bin(int(bits[b, h, i, 2]) & ((1 << 13) - 1)).count("1")
                assert rp[r + 1] - rp[r] == pc
                r += 1
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and rp[-1] == len(ci)


def test_kept_flops_brute_force():
    L, M, N, d = 45, 16, 8, 32
    T_q, T_k = 3, 6
    keep = np.random.default_rng(5).random((2, T_q, T_k)) < 0.5
    bits = _pack(keep)[None]
    exp = 0
    for h in range(2):
        for r in range(L):
            for c in range(L):
                if keep[h, r // M, c // N]:
                    exp += 4 * d
    assert oracle.kept_flops(bits, L, M, N, d) == exp
    ones = _pack(np.ones((1, 1, T_q, T_k), dtype=bool))
    assert oracle.kept_flops(ones, L, M, N, d) == 4 * L * L * d


# --------------------------------------------------------------------------
# predictor
# --------------------------------------------------------------------------
def test_predictor_brute_force_loops():
    L, d, M, N = 37, 4, 16, 4
    q, k, _ = _rand((3, L, d), 17)
    sp = 70
    got = oracle.predict_mask(q[None, None], k[None, None], M, N, sp)[0, 0]
    T_q, T_k = -(-L // M), -(-L // N)
    kk = T_k - 1 - (sp * (T_k - 1)) // 100
    for i in range(T_q):
        rows = list(range(i * M, min(i * M + M, L)))
        qb = [sum(q[r][t] for r in rows) / len(rows) for t in range(d)]
        scores = []
        for j in range(T_k):
            cols = list(range(j * N, min(j * N + N, L)))
            kb = [sum(k[c][t] for c in cols) / len(cols) for t in range(d)]
            scores.append((-sum(a * b for a, b in zip(qb, kb)), j))
        chosen = sorted(j for _, j in sorted(scores)[:kk])
        bits = [j for j in range(T_k) if (int(got[i, j // 32]) >> (j % 32)) & 1]
        assert bits == chosen


def test_predictor_count_matches_numpy_percentile():
    rng = np.random.default_rng(8)
    for T_k in (7, 100, 7425):
        s = rng.standard_normal((3, T_k))
        for sp in (0, 50, 85, 99):
            keep = opred.predict_keep(s, sp)
            thr = np.percentile(s, sp, axis=1)
            assert np.array_equal(keep, s > thr[:, None])
            assert keep.sum(axis=1).tolist() == [opred.topk_count(T_k, sp)] * 3


def test_predictor_exact_k_with_many_ties():
    s = np.array([[1.0, 2.0, 2.0, 2.0, 0.0, 2.0]])
    keep = opred.predict_keep(s, 50)            # k = 5 - 2 = 3
    assert keep[0].tolist() == [False, True, True, True, False, False]


def test_mask_diff_brute_force_and_invariants():
    """Per-row count of differing keep bits j < T_k, by explicit bit loops."""
    rng = np.random.default_rng(77)
    for T_k in (1, 31, 32, 33, 70):
        nw = -(-T_k // 32)
        a = rng.integers(0, 2**32, size=(2, 3, 5, nw), dtype=np.uint64).astype(np.uint32)
        b = rng.integers(0, 2**32, size=(2, 3, 5, nw), dtype=np.uint64).astype(np.uint32)
        rows, heads = oracle.mask_diff(a, b, T_k)
        for idx in np.ndindex(2, 3, 5):
            n = 0
            for j in range(T_k):
                wa, wb = int(a[idx + (j // 32,)]), int(b[idx + (j // 32,)])
                n += ((wa >> (j % 32)) & 1) != ((wb >> (j % 32)) & 1)
            assert rows[idx] == n
        assert np.array_equal(heads, rows.sum(axis=-1))
        # identity, full flip (padding bits are not decisions), symmetry, triangle inequality
        assert not oracle.mask_diff(a, a, T_k)[0].any()
        assert np.all(oracle.mask_diff(a, ~a, T_k)[0] == T_k)
        assert np.array_equal(oracle.mask_diff(b, a, T_k)[0], rows)
        c = rng.integers(0, 2**32, size=a.shape, dtype=np.uint64).astype(np.uint32)
        assert np.all(rows <= oracle.mask_diff(a, c, T_k)[0] + oracle.mask_diff(c, b, T_k)[0])


# --------------------------------------------------------------------------
# mutation tests: planted mistakes must be caught by the pins above
# --------------------------------------------------------------------------
def _pins_pass():
    checks = [test_golden_ragged_tiles_and_empty_row, test_golden_multiword_n1_bit_order,
              lambda: test_all_ones_equals_library_dense_attention(50, 8, 16, 4),
              test_arbitrary_mask_equals_library_with_boolean_mask,
              lambda: test_brute_force_loops(37, 4, 32, 8, 0.6),
              lambda: test_diagonal_only_equals_local_block_attention(61, 16, 8)]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def test_pins_pass_unmutated():
    assert _pins_pass()


@pytest.mark.parametrize("mutation", ["transposed_tile_index", "msb_first_bits", "no_scale",
                                      "mask_as_zero_not_minus_inf", "qk_transposed",
                                      "m_for_n"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    orig_keep, orig_unpack, orig_sm = oatt.keep_matrix, oatt.unpack_mask, oatt._softmax_pv
    if mutation == "transposed_tile_index":
        def keep_matrix(bits, L, M, N, rows=None):
            full = orig_keep(bits, L, M, N)       # [L, L]; the mistake reads it transposed
            return full.T if rows is None else full.T[np.asarray(rows)]
        monkeypatch.setattr(oatt, "keep_matrix", keep_matrix)
    elif mutation == "msb_first_bits":
        def unpack(bits, T_k):
            bits = np.asarray(bits, dtype=np.uint64)
            j = np.arange(T_k)
            return ((bits[..., j // 32] >> (31 - j % 32).astype(np.uint64)) & np.uint64(1)).astype(bool)
        monkeypatch.setattr(oatt, "unpack_mask", unpack)
    elif mutation == "no_scale":
        real = oatt.attention

        def attention(q, k, v, bits, M, N, scale):
            return real(q, k, v, bits, M, N, 1.0)
        monkeypatch.setattr(oracle, "attention", attention)
    elif mutation == "mask_as_zero_not_minus_inf":
        def sm(s, keep, v):
            return orig_sm(np.where(keep, s, 0.0), np.ones_like(keep), v)
        monkeypatch.setattr(oatt, "_softmax_pv", sm)
    elif mutation == "qk_transposed":
        real = oatt.attention

        def attention(q, k, v, bits, M, N, scale):
            return real(k, q, v, bits, M, N, scale)
        monkeypatch.setattr(oracle, "attention", attention)
    elif mutation == "m_for_n":
        def keep_matrix(bits, L, M, N, rows=None):
            return orig_keep(bits, L, M, M, rows)
        monkeypatch.setattr(oatt, "keep_matrix", keep_matrix)
    assert not _pins_pass(), f"planted mistake {mutation!r} went unnoticed"


def test_mask_diff_planted_mistake_is_caught(monkeypatch):
    """Counting the padding bits past T_k (a plausible slip) fails the pins."""
    real = oracle.mask_diff

    def counts_padding(a_bits, b_bits, T_k):
        return real(a_bits, b_bits, np.asarray(a_bits).shape[-1] * 32)

    monkeypatch.setattr(oracle, "mask_diff", counts_padding)
    with pytest.raises(AssertionError):
        test_mask_diff_brute_force_and_invariants()
