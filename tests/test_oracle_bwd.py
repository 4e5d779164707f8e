"""Pins of the backward oracle against things other than itself.

The backward oracle (oracle/backward.py) is the derivative of the
forward oracle, which tests/test_oracle.py pins.  Here it is tied to:
  * central finite differences of the forward oracle's output (the
    derivative by its definition, with no chain-rule algebra);
  * torch autograd in float64 through the library's softmax and through
    scaled_dot_product_attention with the boolean keep mask;
  * closed forms (one kept key per row) and invariants (the rows of dS sum
    to zero, so the dK rows of a head sum to zero; the dV rows sum to the dO
    rows that have a kept key; D equals the row sum of dO * O);
  * planted mistakes, each of which a pin must catch.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as obwd

from test_oracle import _pack, _rand


def _tile_keep(T_q, T_k, p, seed, diag=True, empty_rows=()):
    rng = np.random.default_rng(seed)
    keep = rng.random((T_q, T_k)) < p
    if diag:
        for i in range(T_q):
            keep[i, min(i * T_k // T_q, T_k - 1)] = True
    for i in empty_rows:
        keep[i] = False
    return keep


def _problem(L, d, M, N, p, seed, H=1, empty_rows=()):
    T_q, T_k = -(-L // M), -(-L // N)
    q = _rand((1, H, L, d), seed)
    k = _rand((1, H, L, d), seed + 1)
    v = _rand((1, H, L, d), seed + 2)
    do = _rand((1, H, L, d), seed + 3)
    keep = np.stack([_tile_keep(T_q, T_k, p, seed + 10 + h, empty_rows=empty_rows) for h in range(H)])
    bits = _pack(keep[None])
    return q, k, v, do, bits


def _finite_difference(q, k, v, do, bits, M, N, scale, h=1e-5):
    """d(sum(O * dO)) / d(q, k, v) by central differences of the forward oracle."""
    grads = []
    for which in range(3):
        x = [q, k, v]
        g = np.zeros_like(x[which])
        for idx in np.ndindex(x[which].shape):
            vals = []
            for sgn in (1.0, -1.0):
                xs = [a.copy() for a in x]
                xs[which][idx] += sgn * h
                o, _ = oracle.attention(xs[0], xs[1], xs[2], bits, M, N, scale)
                vals.append(float((o * do).sum()))
            g[idx] = (vals[0] - vals[1]) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("L,d,M,N,p,empty", [(37, 4, 16, 8, 0.5, ()), (29, 3, 32, 1, 0.3, ()),
                                             (41, 4, 16, 4, 0.4, (1,))])
def test_matches_finite_differences_of_forward(L, d, M, N, p, empty):
    scale = 0.45
    q, k, v, do, bits = _problem(L, d, M, N, p, seed=L + N, empty_rows=empty)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, bits, M, N, scale)
    fq, fk, fv = _finite_difference(q, k, v, do, bits, M, N, scale)
    for got, ref in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.abs(got - ref).max() <= 1e-7 * (1.0 + np.abs(ref).max())


def _torch_grads(q, k, v, do, scale, keep=None, use_sdpa=False):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)).requires_grad_(True) for x in (q, k, v))
    if use_sdpa:
        mask = torch.from_numpy(keep)[None, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qt[None, None], kt[None, None], vt[None, None], attn_mask=mask, scale=scale)[0, 0]
    else:
        o = torch.softmax(scale * (qt @ kt.T), dim=-1) @ vt
    o.backward(torch.from_numpy(np.ascontiguousarray(do)))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("L,d,M,N", [(50, 8, 16, 4), (64, 16, 64, 64), (33, 5, 16, 1)])
def test_all_ones_equals_torch_autograd(L, d, M, N):
    scale = float(np.float32(d ** -0.5))
    q, k, v, do, _ = _problem(L, d, M, N, 1.0, seed=7 + L)
    bits = _pack(np.ones((1, 1, -(-L // M), -(-L // N)), dtype=bool))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, bits, M, N, scale)
    tq, tk, tv = _torch_grads(q[0, 0], k[0, 0], v[0, 0], do[0, 0], scale)
    for got, ref in ((dq[0, 0], tq), (dk[0, 0], tk), (dv[0, 0], tv)):
        assert np.abs(got - ref).max() <= 1e-12 * (1.0 + np.abs(ref).max())


def test_tile_mask_equals_torch_sdpa_autograd_with_boolean_mask():
    L, d, M, N, scale = 70, 6, 16, 8, float(np.float32(0.3))   # the float32 scale the oracle uses
    q, k, v, do, bits = _problem(L, d, M, N, 0.4, seed=99)
    keep = oracle.keep_matrix(bits[0, 0], L, M, N)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, bits, M, N, scale)
    tq, tk, tv = _torch_grads(q[0, 0], k[0, 0], v[0, 0], do[0, 0], scale, keep, use_sdpa=True)
    for got, ref in ((dq[0, 0], tq), (dk[0, 0], tk), (dv[0, 0], tv)):
        assert np.abs(got - ref).max() <= 1e-12 * (1.0 + np.abs(ref).max())


def test_one_kept_key_per_row_closed_form():
    """P is one-hot, so dS = 0: dQ = dK = 0 and dV[r] = dO[r] (mask = identity at M = N = 1)."""
    L, d = 23, 4
    q, k, v, do, _ = _problem(L, d, 1, 1, 0.0, seed=5)
    bits = _pack(np.eye(L, dtype=bool)[None, None])
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, bits, 1, 1, 0.7)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0
    assert np.array_equal(dv, do)


def test_gradient_row_sums_and_d_identity():
    L, d, M, N, scale = 61, 5, 16, 2, 0.5
    q, k, v, do, bits = _problem(L, d, M, N, 0.35, seed=21, empty_rows=(2,))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, bits, M, N, scale)
    keep = oracle.keep_matrix(bits[0, 0], L, M, N)
    has_key = keep.any(axis=1)
    # rows of dS sum to zero -> the dK rows of a head sum to zero
    assert np.abs(dk[0, 0].sum(axis=0)).max() <= 1e-12 * (1 + np.abs(dk).max())
    # rows of P sum to one (or zero for an empty row) -> dV rows sum to those dO rows
    assert np.allclose(dv[0, 0].sum(axis=0), do[0, 0][has_key].sum(axis=0), atol=1e-12, rtol=0)
    # D = rowsum(P * dP) equals rowsum(dO * O)
    o, _ = oracle.attention(q, k, v, bits, M, N, scale)
    p = obwd._probs(np.float32(scale) * (q[0, 0] @ k[0, 0].T), keep)
    dp = do[0, 0] @ v[0, 0].T
    assert np.allclose((p * dp).sum(axis=1), (do[0, 0] * o[0, 0]).sum(axis=1), atol=1e-12, rtol=0)


def test_empty_rows_contribute_nothing():
    L, d, M, N, scale = 48, 4, 16, 8, 0.5
    q, k, v, do, bits = _problem(L, d, M, N, 0.5, seed=33, empty_rows=(1,))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, bits, M, N, scale)
    assert np.abs(dq[0, 0, 16:32]).max() == 0.0
    do2 = do.copy()
    do2[0, 0, 16:32] = 1e3
    _, dk2, dv2 = oracle.attention_bwd(q, k, v, do2, bits, M, N, scale)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def test_rows_variant_matches_full():
    L, d, M, N, scale = 90, 6, 16, 8, 0.4
    q, k, v, do, bits = _problem(L, d, M, N, 0.4, seed=44, H=2)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, bits, M, N, scale)
    for h in range(2):
        k_rows = np.array([0, 7, 8, 50, 89])
        qr, dqr, kr, dkr, dvr = obwd.attention_bwd_rows(q[0, h], k[0, h], v[0, h], do[0, h], bits[0, h],
                                                        M, N, scale, q_tiles=[0, 5], k_rows=k_rows, group=7)
        assert np.allclose(dqr, dq[0, h][qr], atol=1e-12, rtol=0)
        assert np.allclose(dkr, dk[0, h][k_rows], atol=1e-12, rtol=0)
        assert np.allclose(dvr, dv[0, h][k_rows], atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# mutation tests: planted mistakes must be caught by the pins above
# --------------------------------------------------------------------------
def _pins_pass():
    checks = [lambda: test_matches_finite_differences_of_forward(37, 4, 16, 8, 0.5, ()),
              lambda: test_all_ones_equals_torch_autograd(50, 8, 16, 4),
              test_tile_mask_equals_torch_sdpa_autograd_with_boolean_mask]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def test_pins_pass_unmutated():
    assert _pins_pass()


@pytest.mark.parametrize("mutation", ["no_d_term", "dv_untransposed", "dk_unscaled", "dq_uses_v",
                                      "softmax_over_all_keys"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    real_probs = obwd._probs

    def head(q, k, v, do, keep, sc):
        p = obwd._probs(sc * (q @ k.T), keep)
        dp = do @ v.T
        dsum = (p * dp).sum(axis=1)
        if mutation == "no_d_term":
            dsum = 0.0 * dsum
        ds = p * (dp - dsum[:, None])
        dv = (p @ do) if mutation == "dv_untransposed" else p.T @ do
        dq = sc * (ds @ (v if mutation == "dq_uses_v" else k))
        dk = (ds.T @ q) if mutation == "dk_unscaled" else sc * (ds.T @ q)
        return dq, dk, dv

    monkeypatch.setattr(obwd, "_head_bwd", head)
    if mutation == "softmax_over_all_keys":
        monkeypatch.setattr(obwd, "_probs", lambda s, keep: real_probs(s, np.ones_like(keep)))
    assert not _pins_pass(), f"planted mistake {mutation!r} went unnoticed"
