"""The benchmark's output contract on the GPU, on small workloads (1x2x512x64
fp32 16x16 tiles; 1x2x2048x128 bf16 16x8 and 16x16): one JSON line on stdout
with the fields the measurement relies on, for the forward, backward, FP8,
predictor, compaction and mask-diff lines, each with its CPU oracle timing.  The
kept-tile counts it reports are checked against the host generator's mask.
The file name sorts after every parity file, so a failure here never hides a
parity test in a run that stops at the first failure."""
import json
import math
import os
import subprocess
import sys

import pytest

import oracle
import workloads as W
from gpu_util import say, torch_or_skip

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
        "scaling", "vs_baseline", "dtype", "data", "config", "roofline"}


def _kept_tiles():
    w = W.get("tiny")
    return int(oracle.unpack_mask(W.mask_bits(w), w.T_k).sum()), w.B * w.H * w.T_q * w.T_k


def _bench(*argv):
    torch_or_skip()
    say(f"bench {' '.join(argv)}")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    rec = json.loads(lines[0])
    assert KEYS <= rec.keys()
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    # what the bench guarantees: a measured time, and a rate that is finite and
    # not negative (a tiny workload's rate may be small)
    assert rec["ms_per_step"] > 0
    assert math.isfinite(rec["value"]) and rec["value"] >= 0
    roof = rec["roofline"]
    assert {"bound", "achieved", "peak", "unit", "frac", "traffic"} <= roof.keys()
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-3, abs=1e-4)
    return rec


def test_forward_line():
    rec = _bench("--workload", "tiny", "--steps", "3", "--warmup", "1", "--no-cpu")
    assert rec["config"]["workload"] == "tiny" and rec["dtype"] == "f32"
    assert rec["roofline"]["bound"] == "mfma" and rec["roofline"]["peak"] == 157.3
    kept, total = _kept_tiles()   # L = 512 is a whole number of 16x16 tiles
    assert rec["config"]["kept_fraction"] == pytest.approx(kept / total, abs=1e-6)
    assert rec["config"]["speedup_vs_all_ones"] > 0
    roof = rec["roofline"]
    assert roof["call_median_ms"] > 0
    pd = roof["peak_derived"]   # 256 CUs x 2400 MHz x 256 FLOP/clk for f32 matrix cores
    assert pd is None or pd["tflops"] == pytest.approx(roof["peak"], rel=0.05)


def test_forward_line_with_cpu_baseline():
    rec = _bench("--workload", "tiny", "--steps", "3", "--warmup", "1", "--no-dense")
    cb = rec["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["cpu_model"] and cb["blas"] and cb["nproc"] >= 1
    assert cb["extrapolated_ms_per_call"] > 0


def _check_cpu(rec, unit):
    cb = rec["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == unit and cb["value"] > 0 and cb["sample"]
    assert cb["cores"] >= 1 and cb["cpu_model"] and cb["blas"]


def test_compaction_line():
    rec = _bench("--compact", "--workload", "tiny", "--steps", "3", "--warmup", "1")
    assert rec["unit"] == "GB/s" and rec["roofline"]["bound"] == "hbm"
    assert rec["config"]["kept_tiles"] == _kept_tiles()[0]
    _check_cpu(rec, "GB/s")


def test_backward_line():
    rec = _bench("--backward", "--workload", "small_fine", "--steps", "3", "--warmup", "1")
    assert rec["unit"] == "TFLOP/s" and rec["dtype"] == "bf16"
    assert rec["roofline"]["bound"] == "mfma" and rec["config"]["speedup_vs_all_ones"] > 0
    _check_cpu(rec, "TFLOP/s")


def test_fp8_line():
    rec = _bench("--fp8", "--workload", "small_fine", "--steps", "3", "--warmup", "1", "--no-dense")
    assert rec["unit"] == "TFLOP/s" and rec["roofline"]["bound"] == "mfma"
    assert rec["config"]["quantise_ms"] > 0
    _check_cpu(rec, "TFLOP/s")


def test_predict_line():
    rec = _bench("--predict", "--workload", "small_pred", "--steps", "3", "--warmup", "1")
    w = W.get("small_pred")
    assert rec["unit"] == "TFLOP/s" and rec["roofline"]["peak"] == 157.3
    assert rec["config"]["score_flops"] == 2 * w.B * w.H * w.T_q * w.T_k * w.d
    _check_cpu(rec, "TFLOP/s")


def test_mask_diff_line():
    rec = _bench("--mask-diff", "--workload", "tiny", "--steps", "3", "--warmup", "1")
    assert rec["unit"] == "GB/s" and rec["roofline"]["bound"] == "hbm"
    _check_cpu(rec, "GB/s")
