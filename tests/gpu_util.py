"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and compare it with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import workloads as W

# Tolerances: fp32 inputs max-abs 1e-4; bf16 inputs max-abs 2e-2 and mean-abs 2e-3.
TOL = {"f32": dict(max_abs=1e-4, mean_abs=1e-4), "bf16": dict(max_abs=2e-2, mean_abs=2e-3)}


def torch_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg: str):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev_mask(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int32)).cuda()


def mask_to_np(m) -> np.ndarray:
    return m.cpu().numpy().view(np.uint32)


def gpu_attention(q, k, v, bits_dev, M, N, scale):
    import torch
    import tile_sparse_attention_amd as T
    o, lse = T.attention_fwd(q, k, v, bits_dev, M, N, scale, return_lse=True)
    torch.cuda.synchronize()
    return o, lse


def compare(name, got_o, ref_o, dtype, got_lse=None, ref_lse=None):
    err = np.abs(got_o.astype(np.float64) - ref_o)
    mx, mean = float(err.max()), float(err.mean())
    tol = TOL[dtype]
    print(f"[parity] {name}: max_abs={mx:.3e} mean_abs={mean:.3e} n={err.size}", flush=True)
    assert np.all(np.isfinite(got_o)), f"{name}: non-finite output"
    assert mx <= tol["max_abs"], f"{name}: max-abs {mx} > {tol['max_abs']}"
    assert mean <= tol["mean_abs"], f"{name}: mean-abs {mean} > {tol['mean_abs']}"
    if got_lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(got_lse), fin), f"{name}: LSE finiteness differs"
        assert np.all(np.isneginf(got_lse[~fin]))
        if fin.any():
            lerr = float(np.abs(got_lse[fin] - ref_lse[fin]).max())
            print(f"[parity] {name}: lse max_abs={lerr:.3e}", flush=True)
            assert lerr <= (1e-4 if dtype == "f32" else 2e-2)
    return mx, mean


def small_workload(name, L, d, M, N, dtype="bf16", H=2, p=0.3, diag=True, seed=7):
    return W.Workload(name, 1, H, L, d, M, N, dtype,
                      W.MaskRecipe("hash", p_near=p, p_far=p, force_diag=diag), seed)


def full_compare(w: W.Workload, bits: np.ndarray, case: str, scale: float | None = None):
    """GPU vs oracle on every row of a small workload (scale: the workload's
    1/sqrt(d) unless given)."""
    import torch
    scale = w.scale if scale is None else scale
    say(f"{case}: B={w.B} H={w.H} L={w.L} d={w.d} M={w.M} N={w.N} {w.dtype} seed={w.seed} "
        f"scale={scale}")
    q, k, v = W.make_qkv(w)
    o, lse = gpu_attention(q.cuda(), k.cuda(), v.cuda(), to_dev_mask(bits), w.M, w.N, scale)
    ro, rl = oracle.attention(q, k, v, bits, w.M, w.N, scale)
    return compare(case, o.float().cpu().numpy(), ro, w.dtype, lse.cpu().numpy(), rl)


def sampled_compare(w: W.Workload, q, k, v, o_dev, lse_dev, bits_rows, tiles, heads, case: str):
    """Oracle on sampled query tiles of the given heads.

    bits_rows(b, h) -> uint32 [T_q, words] bitmap of that head (host, from the
    workload generators or the oracle predictor).
    """
    errs = []
    o_host = o_dev.float().cpu().numpy()
    l_host = lse_dev.cpu().numpy()
    for h in heads:
        if len(heads) > 4 and h % 8 == 0:
            say(f"{case}: oracle head {h} of {len(heads)}")
        rows, ro, rl = oracle.attention_rows(q[0, h], k[0, h], v[0, h], bits_rows(0, h), w.M, w.N,
                                             w.scale, tiles[0, h])
        errs.append((o_host[0, h, rows], ro, l_host[0, h, rows], rl))
    got = np.concatenate([e[0] for e in errs])
    ref = np.concatenate([e[1] for e in errs])
    gl = np.concatenate([e[2] for e in errs])
    rl = np.concatenate([e[3] for e in errs])
    return compare(case, got, ref, w.dtype, gl, rl)
