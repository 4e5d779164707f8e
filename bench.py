"""Benchmark of the tile-sparse attention forward pass on one MI355X.

One step = one tsa_attention_fwd call (bitmap in -> O out: on-the-fly mask
compaction, kept-K/V staging, QK^T, online softmax, PV, normalisation) on
the Wan 2.1 480p shape with 16x8 tiles at 70% frame-structured sparsity,
inputs resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

With --backward it times the backward pass (tsa_attention_bwd) of the same
workload instead and prints that line; --fp8, --mask-diff, --compact and
--predict time the FP8 forward, the mask diff, the mask compaction and the
mask predictor likewise.  Each line carries the fp64 CPU oracle timed on a
bounded sample of the same workload (cpu_baseline) unless --no-cpu.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "kept-tile effective TFLOPS (% bf16 MFMA peak) + ms/call at 70% sparsity"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}     # MI355X dense matrix-core peaks
KERNEL_SOURCES = ("tile_sparse_attention_amd/csrc/attention_fwd_impl.h",
                  "tile_sparse_attention_amd/csrc/attention_fwd_octet.h",
                  "tile_sparse_attention_amd/csrc/attention_fwd_keys.h",
                  "tile_sparse_attention_amd/csrc/attention_fwd_inst.h",
                  "tile_sparse_attention_amd/csrc/launch.h",
                  "tile_sparse_attention_amd/csrc/tsa_device.h",
                  "tile_sparse_attention_amd/build.py")


def kernel_name(w) -> str:
    """The attention kernel the library launches for this workload."""
    if w.dtype != "bf16":
        return "attn_fwd_kernel"
    return "attn_oct_kernel" if w.N >= 8 else "attn_key_kernel"


def sig(x: float, digits: int = 5) -> float:
    """x rounded to `digits` significant digits: a small but measured rate never
    prints as 0."""
    return float(f"{x:.{digits}g}")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def make_mask(w, q, k):
    """Device keep-bitmap of the workload (int32 storage of uint32 words)."""
    import numpy as np
    import torch

    import tile_sparse_attention_amd as T
    import workloads as W
    kind = w.mask.kind
    if kind == "hash":
        return T.maskgen_hash(w.B, w.H, w.L, w.M, w.N, **W.hash_params(w))
    if kind == "structured":
        return T.maskgen_structured(w.B, w.H, w.L, w.M, w.N, **W.structured_params(w))
    if kind == "predicted":
        return T.predict_mask(q, k, w.M, w.N, w.mask.sparsity_percent)
    bits = W.mask_bits(w)
    return torch.from_numpy(bits.view(np.int32)).cuda()


def kept_flops_device(w, mask) -> int:
    """4*d*sum over kept tiles of m_i*n_j, counted on the GPU from the bitmap
    (row counts from the library's compaction call, last partial key tile
    corrected with its bit)."""
    import torch

    import tile_sparse_attention_amd as T
    row_ptr, _ = T.mask_compact(mask, w.L, w.M, w.N, col_capacity=0)
    counts = (row_ptr[1:] - row_ptr[:-1]).view(w.B, w.H, w.T_q)
    m = torch.clamp(w.L - torch.arange(w.T_q, device=mask.device) * w.M, max=w.M).to(torch.int64)
    n_last = w.L - (w.T_k - 1) * w.N
    last = w.T_k - 1
    last_bit = ((mask[..., last // 32] >> (last % 32)) & 1).to(torch.int64)
    keys = counts * w.N - last_bit * (w.N - n_last)
    return int(4 * w.d * (keys * m).sum().item())


def time_calls(fn, steps, warmup, kernel_events=False, stats=None):
    """(ms per step over the bracketed region, mean per-call ms from events,
    min per-call ms); with kernel_events also the mean ms of the attention
    kernels proper, from events the library records around them on the same
    stream (tsa_set_timing_events).  A `stats` dict receives the median
    per-call ms."""
    import torch

    import tile_sparse_attention_amd as T
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)] if kernel_events else None
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        if kev is not None:
            T.set_timing_events(*kev[i])
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    if kev is not None:
        T.set_timing_events(None, None)
    per = [a.elapsed_time(b) for a, b in ev]
    if stats is not None:
        stats["median_ms"] = sorted(per)[len(per) // 2] if len(per) % 2 else \
            0.5 * (sorted(per)[len(per) // 2 - 1] + sorted(per)[len(per) // 2])
    out = (wall / steps, sum(per) / len(per), min(per))
    if kev is not None:
        kern = [a.elapsed_time(b) for a, b in kev]
        out = out + (sum(kern) / len(kern),)
    return out


def cpu_baseline(w, q, k, v, mask, budget_s=20.0, kept_total=None):
    """fp64 oracle on a bounded sample of the workload, in the metric's unit: the
    first `per_head` of each head's sampled query tiles (tile 0, the last tile and
    random ones), over all heads, with `per_head` sized to the time budget."""
    import numpy as np

    import oracle
    import workloads as W
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    tiles = W.sample_tiles(w)
    bits = mask.cpu().numpy().view(np.uint32)
    nj = np.minimum(w.N, w.L - np.arange(w.T_k) * w.N)

    def run(b, h, sample):
        oracle.attention_rows(q[b, h], k[b, h], v[b, h], bits[b, h], w.M, w.N, w.scale, sample,
                              group=16)
        keep = oracle.unpack_mask(bits[b, h][sample], w.T_k)
        m = np.minimum(w.M, w.L - sample * w.M)
        return 4 * w.d * int((m[:, None] * keep * nj[None, :]).sum())

    run(0, 0, tiles[0, 0, :16])                  # warm-up, then a probe that sizes the sample
    t0 = time.perf_counter()
    run(0, 0, tiles[0, 0, :16])
    per_tile = (time.perf_counter() - t0) / 16
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    per_head = int(max(4, min(tiles.shape[2], budget_s / max(per_tile, 1e-6) / len(heads))))
    kept, secs = 0, 0.0
    for b, h in heads:
        t0 = time.perf_counter()
        kept += run(b, h, tiles[b, h, :per_head])
        secs += time.perf_counter() - t0
    n = per_head * len(heads)
    rate = kept / secs
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(), "blas": blas_name(),
            # the whole call's kept FLOPs at the sampled rate (not measured)
            "extrapolated_ms_per_call": round(kept_total / rate * 1e3, 1) if kept_total else None,
            "sample": f"{per_head} sampled query tiles per head x {len(heads)} heads ({n} tiles, "
                      f"{n * w.M} query rows) against all {w.L} keys, fp64 numpy, {secs:.1f} s; "
                      f"kept FLOPs of those rows / time"}


FLOP_PER_CLK_PER_CU = {"bf16": 4096, "f32": 256}  # dense matrix cores (16x16x32 bf16, 16x16x4 f32)


def _sampled(units, run_one, budget_s):
    """Runs run_one(u) over `units` in order (every unit at least once for the
    first, then until budget_s of wall time is spent); returns (units run,
    summed work, seconds).  run_one returns the unit's work."""
    done, work, secs = 0, 0, 0.0
    for u in units:
        t0 = time.perf_counter()
        work += run_one(u)
        secs += time.perf_counter() - t0
        done += 1
        if secs >= budget_s:
            break
    return done, work, secs


def _oracle_env():
    return {"cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(), "blas": blas_name()}


def cpu_baseline_backward(w, q, k, v, do, mask, budget_s=20.0):
    """fp64 backward oracle on a bounded sample: dQ rows of each head's sampled
    query tiles (S, dP and dQ for those rows: 3 of the 5 GEMMs), credited with
    1.5x the rows' kept forward FLOPs, in TFLOP/s."""
    import numpy as np

    import oracle
    import workloads as W
    tiles = W.sample_tiles(w)
    bits = mask.cpu().numpy().view(np.uint32)
    nj = np.minimum(w.N, w.L - np.arange(w.T_k) * w.N)
    per = 8
    units = [(b, h, i0) for i0 in range(0, tiles.shape[2], per) for b in range(w.B) for h in range(w.H)]

    def run(u):
        b, h, i0 = u
        t = tiles[b, h, i0:i0 + per]
        oracle.attention_bwd_rows(q[b, h], k[b, h], v[b, h], do[b, h], bits[b, h], w.M, w.N, w.scale,
                                  q_tiles=t)
        keep = oracle.unpack_mask(bits[b, h][t], w.T_k)
        m = np.minimum(w.M, w.L - t * w.M)
        return 1.5 * 4 * w.d * int((m[:, None] * keep * nj[None, :]).sum())

    n, work, secs = _sampled(units, run, budget_s)
    return {"value": work / secs / 1e12, "unit": "TFLOP/s", **_oracle_env(),
            "sample": f"dQ rows of {n * per} sampled query tiles over {min(n, w.B * w.H)} heads (S, dP, dQ: "
                      f"3 of the 5 GEMMs, credited 1.5x their kept forward FLOPs), fp64 numpy, {secs:.1f} s"}


def cpu_baseline_rows(w, bits_list, fn, per_row_bytes, budget_s=10.0):
    """An oracle over bitmap rows (compaction, mask diff) on a bounded sample
    of the flattened rows, in GB/s of the line's algorithmic bytes.
    per_row_bytes(rows, result) gives the bytes those rows account for."""
    import numpy as np
    flat = [np.ascontiguousarray(x).reshape(-1, x.shape[-1]) for x in bits_list]
    R = flat[0].shape[0]
    chunk = max(1, min(R, 4096))
    units = list(range(0, R, chunk))

    def run(r0):
        part = [f[r0:r0 + chunk][None, None] for f in flat]
        return per_row_bytes(part[0].shape[2], fn(*part, w.T_k))

    n, work, secs = _sampled(units, run, budget_s)
    rows = min(R, n * chunk)
    return {"value": work / secs / 1e9, "unit": "GB/s", **_oracle_env(),
            "sample": f"the first {rows} of {R} bitmap rows, numpy, {secs:.2f} s"}


def cpu_baseline_predict(w, q, k, budget_s=20.0):
    """fp64 predictor oracle (pool, pooled scores, stable top-k, pack) on
    bounded samples of query-tile rows, one head at a time, in TFLOP/s of the
    rows' score products (2 T_k d per row; the pooling of the head's tiles is
    in the timed work)."""
    import numpy as np

    import oracle
    import workloads as W
    tiles = W.sample_tiles(w)
    per = tiles.shape[2]   # one call per head: the oracle pools the whole head on every call
    units = [(b, h, 0) for b in range(w.B) for h in range(w.H)]

    def run(u):
        b, h, i0 = u
        t = tiles[b, h, i0:i0 + per]
        oracle.predict_mask(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], w.M, w.N, w.mask.sparsity_percent,
                            tiles=t[None, None])
        return 2 * len(t) * w.T_k * w.d

    n, work, secs = _sampled(units, run, budget_s)
    return {"value": work / secs / 1e12, "unit": "TFLOP/s", **_oracle_env(),
            "sample": f"{n * per} sampled query-tile rows over {min(n, w.B * w.H)} heads (each head's pooling "
                      f"included), fp64 numpy, {secs:.1f} s"}


def derived_peak_tflops(dtype="bf16"):
    """The dense matrix-core peak re-derived from the device: compute units
    (torch) x the GPU agent's maximum clock (rocminfo) x the matrix cores'
    FLOP per clock per compute unit for `dtype`; None when rocminfo is not
    there."""
    import subprocess

    import torch
    try:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    mhz, in_gpu = None, False
    for line in txt.splitlines():
        t = line.strip()
        if t.startswith("Name:"):
            in_gpu = t.split(":", 1)[1].strip().startswith("gfx")
        elif in_gpu and t.startswith("Max Clock Freq. (MHz):"):
            mhz = float(t.split(":", 1)[1].strip())
            break
    if mhz is None:
        return None
    f = FLOP_PER_CLK_PER_CU[dtype]
    return {"tflops": round(cus * mhz * 1e6 * f / 1e12, 1), "cus": cus, "max_mhz": mhz,
            "flop_per_clk_per_cu": f}


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def blas_name() -> str:
    """numpy's BLAS library and version, as numpy reports them."""
    import numpy as np
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # older numpy without mode="dicts"
        return "unknown"


def traffic_for(workload: str, sha: str):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary, or None when it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != sha:
        return None
    return rec.get("bytes_per_launch")


BWD_METRIC = ("backward kept-tile effective TFLOPS (dQ, dK, dV; 5 GEMMs per kept tile = 2.5x the "
              "forward's kept FLOPs)")
BWD_SOURCES = ("tile_sparse_attention_amd/csrc/attention_bwd.h", "tile_sparse_attention_amd/csrc/attention_bwd.hip")


def bench_backward(args, w, name, qd, kd, vd, mask, flops, dense_flops, out, ws, q_cpu, k_cpu, v_cpu):
    """One step = one tsa_attention_bwd call (LSE/D preparation, the dK/dV kernel
    and the dQ kernel) on the workload, given the forward's O and LSE."""
    import torch

    import tile_sparse_attention_amd as T
    import workloads as W
    if w.dtype != "bf16":
        raise SystemExit("the backward is bf16 only")
    do = W.make_do(w).cuda()
    o, lse = T.attention_fwd(qd, kd, vd, mask, w.M, w.N, w.scale, out=out, return_lse=True, workspace=ws)
    pr = T.problem(w.B, w.H, w.L, w.d, w.M, w.N, T.DTYPE_BF16)
    wsb = torch.empty(T.workspace_size(T.OP_ATTENTION_BWD, pr), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step():
        T.attention_bwd(qd, kd, vd, o, do, lse, mask, w.M, w.N, w.scale, workspace=wsb)

    ms_step, ms_kernel, ms_min = time_calls(step, args.steps, args.warmup)
    fb = 2.5 * flops
    tflops = fb / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    log(f"backward: {ms_step:.3f} ms/step, call mean {ms_kernel:.3f} ms (min {ms_min:.3f}), "
        f"{tflops:.1f} TFLOP/s")
    cfg = {"workload": name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "M": w.M, "N": w.N,
           "mask": w.description, "kept_fraction": round(flops / dense_flops, 6),
           "backward_flops": int(fb), "pct_of_peak": round(100 * tflops / peak, 2), "peak_tflops": peak}
    if not args.no_dense:
        ones = torch.full_like(mask, -1)
        o2, l2 = T.attention_fwd(qd, kd, vd, ones, w.M, w.N, w.scale, return_lse=True, workspace=ws)

        def dense_step():
            T.attention_bwd(qd, kd, vd, o2, do, l2, ones, w.M, w.N, w.scale, workspace=wsb)
        d_step, _, _ = time_calls(dense_step, max(3, args.steps // 4), 1)
        cfg["all_ones_ms"] = round(d_step, 4)
        cfg["all_ones_tflops"] = round(2.5 * dense_flops / (d_step * 1e-3) / 1e12, 2)
        cfg["speedup_vs_all_ones"] = round(d_step / ms_step, 3)
        log(f"all-ones backward: {d_step:.3f} ms/step ({cfg['all_ones_tflops']} TFLOP/s), "
            f"sparse speedup {cfg['speedup_vs_all_ones']}x")
    h = hashlib.sha256()
    for p in BWD_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    achieved = fb / (ms_kernel * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None,
            "kernel": "bwd_prep_kernel + bwd_dkdv_kernel + bwd_dq_kernel", "kernel_sha": h.hexdigest()[:16]}
    rec = {"metric": BWD_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded normal Q/K/V/dO, generated masks)", "config": cfg, "roofline": roof}
    if not args.no_cpu:
        log("timing the CPU backward oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline_backward(w, q_cpu, k_cpu, v_cpu, do.cpu(), mask)
    print(json.dumps(rec), flush=True)


def bench_fp8(args, w, name, qd, kd, vd, mask, flops, dense_flops, out, ws, q_cpu, k_cpu, v_cpu):
    """One step = one tsa_attention_fwd_fp8 call (Q, K already quantised to e4m3
    and resident in HBM); the quantisation is timed on its own."""
    import torch

    import tile_sparse_attention_amd as T
    if w.dtype != "bf16" or w.d != 128:
        raise SystemExit("the FP8 path takes bf16, d = 128")
    q8, qs, k8, ks = T.quantize_qk_fp8(qd, kd)
    torch.cuda.synchronize()
    qms, qcall, _ = time_calls(lambda: T.quantize_qk_fp8(qd, kd), args.steps, args.warmup)

    def step():
        T.attention_fwd_fp8(q8, k8, qs, ks, vd, mask, w.M, w.N, w.scale, out=out, workspace=ws)

    ms_step, ms_call, ms_min, ms_kernel = time_calls(step, args.steps, args.warmup, kernel_events=True)
    tflops = flops / (ms_step * 1e-3) / 1e12
    # half of the kept FLOPs (QK^T) run at the FP8 peak, half (PV) at the bf16 peak
    peak = 2.0 / (1.0 / 5000.0 + 1.0 / PEAK_TFLOPS["bf16"])
    log(f"fp8 scores: {ms_step:.3f} ms/step, kernel mean {ms_kernel:.3f} ms, {tflops:.1f} TFLOP/s; "
        f"quantisation {qcall:.3f} ms")
    cfg = {"workload": name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "M": w.M, "N": w.N,
           "mask": w.description, "kept_fraction": round(flops / dense_flops, 6), "kept_flops": flops,
           "quantise_ms": round(qcall, 4), "peak_tflops": round(peak, 1)}
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    rec = {"metric": "FP8-score kept-tile effective TFLOPS (QK^T on e4m3 with per-tile scales, PV bf16)",
           "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3 scores, bf16 PV",
           "data": "synthetic (seeded normal Q/K/V, generated masks)", "config": cfg,
           "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                        "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                        "kernel": "attn_oct_kernel (FP8 scores)"}}
    if not args.no_cpu:
        import oracle.fp8 as F
        log("timing the CPU oracle (on the dequantised Q and K) on a bounded sample ...")
        q8c, qsc, k8c, ksc = F.quantize_qk(q_cpu, k_cpu)
        qdq = F.dequantize(q8c, qsc, F.Q_TILE_ROWS)
        kdq = F.dequantize(k8c, ksc[..., None], w.L)
        del q8c, k8c
        rec["cpu_baseline"] = cpu_baseline(w, qdq, kdq, v_cpu, mask, kept_total=flops)
        rec["cpu_baseline"]["sample"] += " (Q, K dequantised from e4m3)"
    print(json.dumps(rec), flush=True)


PREDICT_METRIC = ("pooled-score predictor throughput: fp32-accurate score products (2 T_q T_k d per head) "
                  "per whole prediction (pool, products, top-k select, pack), TFLOP/s")


def bench_predict(args, w, name, qd, kd, q_cpu, k_cpu):
    """One step = one tsa_predict_mask call (Q, K in, keep-bitmap out), inputs
    resident in HBM, with the workload's sparsity (85% unless it names one)."""
    import torch

    import tile_sparse_attention_amd as T
    sp = w.mask.sparsity_percent if w.mask.kind == "predicted" else 85
    out = torch.empty((w.B, w.H, w.T_q, T.mask_row_words(w.L, w.N)), dtype=torch.int32, device="cuda")
    T.predict_mask(qd, kd, w.M, w.N, sp, out=out)
    first = out.clone()
    torch.cuda.synchronize()

    def step():
        T.predict_mask(qd, kd, w.M, w.N, sp, out=out)

    st = {}
    ms_step, ms_call, ms_min = time_calls(step, args.steps, args.warmup, stats=st)
    if not torch.equal(first, out):
        raise SystemExit("predictor: repeated calls gave different masks")
    fl = 2 * w.B * w.H * w.T_q * w.T_k * w.d
    tflops = fl / (ms_step * 1e-3) / 1e12
    achieved = fl / (ms_call * 1e-3) / 1e12
    peak = PEAK_TFLOPS["f32"]
    log(f"predictor: {ms_step:.3f} ms/step, call mean {ms_call:.3f} ms, {tflops:.1f} TFLOP/s of "
        f"fp32-accurate score products")
    rec = {"metric": PREDICT_METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32 (products as three bf16 matrix-core products of hi/lo parts)",
           "data": "synthetic (seeded normal Q/K with per-frame offsets)",
           "config": {"workload": name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "M": w.M, "N": w.N,
                      "T_q": w.T_q, "T_k": w.T_k, "sparsity_percent": sp, "score_flops": fl},
           "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(achieved / peak, 4), "traffic": None,
                        "kernel": "pool_tiles_kernel + predict_fused_kernel + predict_rows_fallback_kernel",
                        "call_ms": round(ms_call, 4), "call_median_ms": round(st["median_ms"], 4),
                        "note": "the fp32 matrix-core peak: the products are fp32-accurate"}}
    if not args.no_cpu:
        log("timing the CPU predictor oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline_predict(w, q_cpu, k_cpu)
    print(json.dumps(rec), flush=True)


def bench_mask_diff(args, w, name):
    """One step = one tsa_mask_diff call between two masks of the workload
    (the workload's own and one drawn with another seed), both resident in HBM:
    per-row and per-head counts of differing keep decisions."""
    import numpy as np
    import torch

    import tile_sparse_attention_amd as T
    import workloads as W
    w2 = W.Workload(w.name + "_next", w.B, w.H, w.L, w.d, w.M, w.N, w.dtype, w.mask, w.seed + 1000)
    a = torch.from_numpy(np.ascontiguousarray(W.mask_bits(w)).view(np.int32)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(W.mask_bits(w2)).view(np.int32)).cuda()
    rows = torch.empty(a.shape[:3], dtype=torch.int64, device="cuda")
    heads = torch.empty(a.shape[:2], dtype=torch.int64, device="cuda")
    pr = T.problem(w.B, w.H, w.L, 0, w.M, w.N)
    lib = T.lib()

    def step():
        T._check(lib.tsa_mask_diff(T.ctypes.byref(pr), T._ptr(a), T._ptr(b), T._ptr(rows), T._ptr(heads),
                                   T._stream()))

    ms_step, ms_call, ms_min = time_calls(step, args.steps, args.warmup)
    nbytes = 2 * a.numel() * 4 + rows.numel() * 8 * 2 + heads.numel() * 8
    gbs = nbytes / (ms_call * 1e-3) / 1e9
    changed = int(heads.sum())
    log(f"mask diff: {ms_step:.4f} ms/step, call mean {ms_call:.4f} ms, {gbs:.0f} GB/s, "
        f"{changed} of {a.shape[0] * a.shape[1] * a.shape[2] * w.T_k} decisions differ")
    rec = {"metric": "mask diff HBM throughput (two keep-bitmaps in, per-row and per-head counts out)",
           "value": sig(nbytes / (ms_step * 1e-3) / 1e9), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": sig(ms_step),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
           "data": "synthetic (two seeded masks of the workload)",
           "config": {"workload": name, "B": w.B, "H": w.H, "L": w.L, "M": w.M, "N": w.N,
                      "bitmap_bytes": a.numel() * 4, "changed_decisions": changed},
           "roofline": {"bound": "hbm", "achieved": sig(gbs), "peak": 8000.0, "unit": "GB/s",
                        "frac": sig(gbs / 8000.0), "traffic": None,
                        "kernel": "diff_rows_kernel + diff_heads_kernel"}}
    if not args.no_cpu:
        import oracle
        words = a.shape[-1]
        rec["cpu_baseline"] = cpu_baseline_rows(
            w, [a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32)], oracle.mask_diff,
            lambda rows, res: rows * (2 * words * 4 + 8))
    print(json.dumps(rec), flush=True)


def bench_compact(args, w, name):
    """One step = one tsa_mask_compact call (the workload's bitmap in, CSR
    row_ptr and col_idx out, capacity exact), all resident in HBM."""
    import torch

    import tile_sparse_attention_amd as T
    import workloads as W
    qd = kd = None
    if w.mask.kind == "predicted":
        q, k, _ = W.make_qkv(w)
        qd, kd = q.cuda(), k.cuda()
    mask = make_mask(w, qd, kd)
    del qd, kd
    pr = T.problem(w.B, w.H, w.L, 0, w.M, w.N)
    rows = w.B * w.H * w.T_q
    nnz = int(T.mask_compact(mask, w.L, w.M, w.N, col_capacity=0)[0][-1])
    row_ptr = torch.empty(rows + 1, dtype=torch.int64, device="cuda")
    col_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device="cuda")
    ws, nws = T._workspace(T.OP_MASK_COMPACT, pr, mask.device)
    lib = T.lib()

    def step():
        T._check(lib.tsa_mask_compact(T.ctypes.byref(pr), T._ptr(mask), T._ptr(row_ptr), T._ptr(col_idx),
                                      nnz, T._ptr(ws), nws, T._stream()))

    ms_step, ms_call, ms_min = time_calls(step, args.steps, args.warmup)
    if int(row_ptr[-1]) != nnz:
        raise SystemExit("compaction: list length differs from the count-only call")
    # algorithmic bytes: the bitmap read once, row_ptr and col_idx written once
    nbytes = mask.numel() * 4 + (rows + 1) * 8 + nnz * 4
    gbs = nbytes / (ms_call * 1e-3) / 1e9
    log(f"compaction: {ms_step:.4f} ms/step, call mean {ms_call:.4f} ms, {gbs:.0f} GB/s, "
        f"{nnz} kept tiles in {rows} rows")
    rec = {"metric": "mask compaction HBM throughput (keep-bitmap in, CSR row_ptr / col_idx out)",
           "value": sig(nbytes / (ms_step * 1e-3) / 1e9), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": sig(ms_step),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
           "data": "synthetic (the workload's seeded mask)",
           "config": {"workload": name, "B": w.B, "H": w.H, "L": w.L, "M": w.M, "N": w.N,
                      "bitmap_bytes": mask.numel() * 4, "kept_tiles": nnz, "algorithmic_bytes": nbytes},
           "roofline": {"bound": "hbm", "achieved": sig(gbs), "peak": 8000.0, "unit": "GB/s",
                        "frac": sig(gbs / 8000.0), "traffic": None,
                        "kernel": "compact_count_kernel + scan_groups_kernel + compact_fill_kernel"}}
    if not args.no_cpu:
        import numpy as np

        import oracle
        words = mask.shape[-1]
        rec["cpu_baseline"] = cpu_baseline_rows(
            w, [mask.cpu().numpy().view(np.uint32)], oracle.compact,
            lambda rows, res: rows * (words * 4 + 8) + int(res[0][-1]) * 4)
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dQ, dK, dV) of the workload instead and print "
                         "its own JSON line")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8-score forward (tsa_attention_fwd_fp8) of the workload, and the "
                         "quantisation of Q and K separately, and print its own JSON line")
    ap.add_argument("--compact", action="store_true",
                    help="time tsa_mask_compact (bitmap -> CSR lists) on the workload's mask instead")
    ap.add_argument("--mask-diff", action="store_true",
                    help="time tsa_mask_diff between the workload's mask and a reseeded one (mask reuse "
                         "across denoising steps) and print its own JSON line")
    ap.add_argument("--predict", action="store_true",
                    help="time tsa_predict_mask (pool, pooled scores, top-k select, pack) on the workload "
                         "(default hunyuan720) and print its own JSON line")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run one plain device copy of BYTES bytes (calibrates the HBM "
                         "byte counters of a profiler run) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(every (batch, head) is independent, so a caller shards by heads)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tile_sparse_attention_amd as T
    import workloads as W
    if args.copy_probe:
        src = torch.ones(args.copy_probe, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe}), flush=True)
        return
    name = args.workload or ("hunyuan720" if args.predict else W.HEADLINE)
    w = W.get(name)
    if args.mask_diff:
        bench_mask_diff(args, w, name)
        return
    if args.compact:
        bench_compact(args, w, name)
        return
    log(f"workload {name}: B={w.B} H={w.H} L={w.L} d={w.d} M={w.M} N={w.N} {w.dtype}")
    t0 = time.perf_counter()
    q, k, v = W.make_qkv(w)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mask = make_mask(w, qd, kd)
    torch.cuda.synchronize()
    out = torch.empty_like(qd)
    ws = torch.empty(T.workspace_size(T.OP_ATTENTION_FWD, T.problem(w.B, w.H, w.L, w.d, w.M, w.N,
                                                                    T.DTYPE_BF16 if w.dtype == "bf16"
                                                                    else T.DTYPE_F32)),
                     dtype=torch.uint8, device="cuda")
    flops = kept_flops_device(w, mask)
    dense_flops = 4 * w.B * w.H * w.L * w.L * w.d
    log(f"kept FLOPs {flops:.4e} ({flops / dense_flops:.4f} of dense)")

    if args.backward:
        bench_backward(args, w, name, qd, kd, vd, mask, flops, dense_flops, out, ws, q, k, v)
        return
    if args.fp8:
        bench_fp8(args, w, name, qd, kd, vd, mask, flops, dense_flops, out, ws, q, k, v)
        return
    if args.predict:
        bench_predict(args, w, name, qd, kd, q, k)
        return

    def step():
        T.attention_fwd(qd, kd, vd, mask, w.M, w.N, w.scale, out=out, workspace=ws)

    st = {}
    ms_step, ms_call, ms_min, ms_kernel = time_calls(step, args.steps, args.warmup, kernel_events=True,
                                                     stats=st)
    tflops = flops / (ms_step * 1e-3) / 1e12
    log(f"sparse: {ms_step:.3f} ms/step, call mean {ms_call:.3f} ms (min {ms_min:.3f}), attention "
        f"kernels {ms_kernel:.3f} ms, {tflops:.1f} TFLOP/s")
    peak = PEAK_TFLOPS[w.dtype]
    cfg = {"workload": name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "M": w.M, "N": w.N,
           "mask": w.description, "kept_fraction": round(flops / dense_flops, 6),
           "kept_flops": flops, "pct_of_peak": round(100 * tflops / peak, 2),
           "peak_tflops": peak}
    if w.mask.kind == "predicted":
        # the predictor is timed on its own and reported beside the attention call
        mask2 = torch.empty_like(mask)

        def predict_step():
            T.predict_mask(qd, kd, w.M, w.N, w.mask.sparsity_percent, out=mask2)
        p_step, p_call, _ = time_calls(predict_step, max(3, args.steps // 4), 1)
        if not torch.equal(mask2, mask):
            raise SystemExit("predictor: repeated calls gave different masks")
        cfg["predictor_ms"] = round(p_step, 4)
        cfg["attention_plus_predictor_ms"] = round(ms_step + p_step, 4)
        log(f"predictor: {p_step:.3f} ms/step; attention + predictor {ms_step + p_step:.3f} ms")
        del mask2
    if not args.no_dense:
        ones = torch.full_like(mask, -1)
        out2 = torch.empty_like(qd)

        def dense_step():
            T.attention_fwd(qd, kd, vd, ones, w.M, w.N, w.scale, out=out2, workspace=ws)
        d_step, d_kernel, _ = time_calls(dense_step, max(3, args.steps // 4), 1)
        cfg["all_ones_ms"] = round(d_step, 4)
        cfg["all_ones_tflops"] = round(dense_flops / (d_step * 1e-3) / 1e12, 2)
        cfg["speedup_vs_all_ones"] = round(d_step / ms_step, 3)
        log(f"all-ones: {d_step:.3f} ms/step ({cfg['all_ones_tflops']} TFLOP/s), "
            f"sparse speedup {cfg['speedup_vs_all_ones']}x")
        del ones, out2
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    sha = kernel_sha()
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic_for(name, sha),
            "kernel": kernel_name(w), "kernel_ms": round(ms_kernel, 4), "call_ms": round(ms_call, 4),
            "call_median_ms": round(st["median_ms"], 4), "kernel_sha": sha,
            "peak_derived": derived_peak_tflops(w.dtype)}
    rec = {"metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": w.dtype, "data": "synthetic (seeded normal Q/K/V, generated masks)",
           "config": cfg, "roofline": roof}
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, mask, kept_total=flops)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
