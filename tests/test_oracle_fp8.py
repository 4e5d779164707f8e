"""Pins of the FP8 quantisation oracle (oracle/fp8.py) against things other
than itself: torch's float8_e4m3fn conversion (a library routine), brute-force
tile maxima, the format's error bound, and idempotence on the e4m3 grid."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).float().numpy()


def _codes():
    """All finite e4m3 values, ascending (from torch's decoding of the 256 codes)."""
    v = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    return np.unique(v[np.isfinite(v)])


def test_round_matches_torch_on_every_code_and_tie():
    c = _codes()
    assert len(c) == 253 and c.max() == 448.0          # +-0 share a value; the NaN codes are dropped
    mids = (c[:-1].astype(np.float64) + c[1:]) / 2        # exact ties between neighbours
    x = np.concatenate([c, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                        np.nextafter(mids.astype(np.float32), np.float32(-np.inf))]).astype(np.float32)
    assert np.array_equal(fp8.round_e4m3(x), _torch_e4m3(x).astype(np.float64))


def test_round_matches_torch_on_random_magnitudes():
    rng = np.random.default_rng(11)
    x = (rng.choice([-1.0, 1.0], 200000) * np.exp2(rng.uniform(-12, np.log2(463.9), 200000))).astype(np.float32)
    assert np.array_equal(fp8.round_e4m3(x), _torch_e4m3(x).astype(np.float64))
    assert np.all(np.isnan(fp8.round_e4m3(np.float32([464.0, 1000.0]))))


def test_tile_scales_brute_force():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 3, 37, 8)).astype(np.float32)
    x[0, 1, 16:32] = 0.0                                  # an all-zero tile
    s = fp8.tile_scales(x, 16)
    for b in range(2):
        for h in range(3):
            for t in range(3):
                m = 0.0
                for r in range(16 * t, min(37, 16 * t + 16)):
                    for c in range(8):
                        m = max(m, abs(float(x[b, h, r, c])))
                want = np.float32(m) / np.float32(448.0) if m > 0 else np.float32(1.0)
                assert s[b, h, t] == want


def test_quantize_error_bound_max_and_idempotence():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((1, 2, 100, 16)) * np.exp2(rng.uniform(-8, 4, (1, 2, 100, 1)))).astype(np.float32)
    v, s = fp8.quantize(x, 16)
    deq = fp8.dequantize(v, s, 16)
    s_rows = np.repeat(s.astype(np.float64), 16, axis=-1)[..., :100, None]
    assert np.all(np.abs(x - deq) <= np.abs(x) * 2.0 ** -4 + s_rows * 2.0 ** -10 * (1 + 1e-6))
    tile_max = np.array([np.abs(v[..., t * 16:t * 16 + 16, :]).max(axis=(-2, -1)) for t in range(7)])
    assert np.all(tile_max == 448.0)
    v2, s2 = fp8.quantize(deq.astype(np.float32), 16)
    assert np.array_equal(s2, s) and np.array_equal(v2, v)


def test_quantize_qk_shapes_and_reuse_of_attention_oracle():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((1, 2, 40, 8)).astype(np.float32)
    k = rng.standard_normal((1, 2, 40, 8)).astype(np.float32)
    q8, qs, k8, ks = fp8.quantize_qk(q, k)
    assert qs.shape == (1, 2, 3) and ks.shape == (1, 2)
    assert np.all(np.abs(k8).max(axis=(-2, -1)) == 448.0)
    assert np.allclose(fp8.dequantize(k8, ks[..., None], 40), k, rtol=2.0 ** -4, atol=1e-6)


@pytest.mark.parametrize("mutation", ["truncate", "bias8", "flush_subnormals"])
def test_planted_rounding_mistakes_are_caught(monkeypatch, mutation):
    real = fp8.round_e4m3

    def bad(x):
        x = np.asarray(x, dtype=np.float32).astype(np.float64)
        a = np.abs(x)
        e = np.clip(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6 if mutation != "bias8" else -7, 8)
        quantum = np.exp2(e - 3)
        r = (np.floor(a / quantum) if mutation == "truncate" else np.round(a / quantum)) * quantum
        if mutation == "flush_subnormals":
            r = np.where(a < 2.0 ** -6, 0.0, r)
        return np.copysign(np.where(a >= 464.0, np.nan, np.minimum(r, 448.0)), x)

    monkeypatch.setattr(fp8, "round_e4m3", bad)
    with pytest.raises(AssertionError):
        test_round_matches_torch_on_every_code_and_tie()
        test_round_matches_torch_on_random_magnitudes()
    monkeypatch.setattr(fp8, "round_e4m3", real)
