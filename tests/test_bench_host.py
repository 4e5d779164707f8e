"""Host-side logic of bench.py (no GPU): the one-GPU guard, the kernel-source
gate on the committed HBM traffic figure, and the consistency of that figure
with the raw counter values and copy calibration it was computed from."""
import json
import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"]])
def test_more_than_one_gpu_is_refused(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")],
                       capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 2 and r.stdout == ""


def test_kernel_name_follows_dtype_and_n():
    assert bench.kernel_name(W.get("tiny")) == "attn_fwd_kernel"          # f32
    assert bench.kernel_name(W.get("wan480_fine")) == "attn_oct_kernel"   # N = 8
    assert bench.kernel_name(W.get("wan480_coarse")) == "attn_oct_kernel"
    assert bench.kernel_name(W.get("wan720_n1")) == "attn_key_kernel"     # N = 1


def test_traffic_is_gated_on_kernel_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    rec = {"workload": "x", "kernel_sha": "abc", "bytes_per_launch": 123}
    (tmp_path / "profiles" / "attn_fwd_x_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_for("x", "abc") == 123
    assert bench.traffic_for("x", "abd") is None      # kernel changed since the counters
    assert bench.traffic_for("y", "abc") is None      # never profiled


def test_kernel_sha_changes_with_any_source(tmp_path, monkeypatch):
    for p in bench.KERNEL_SOURCES:
        dst = tmp_path / p
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, p), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_sha()
    for p in bench.KERNEL_SOURCES:
        f = tmp_path / p
        orig = f.read_bytes()
        f.write_bytes(orig + b"\n")
        assert bench.kernel_sha() != base, p
        f.write_bytes(orig)
    assert bench.kernel_sha() == base


def test_committed_traffic_is_consistent():
    path = os.path.join(ROOT, "profiles", "attn_fwd_wan480_fine_traffic.json")
    rec = json.load(open(path))
    cal = rec["copy_calibration"]
    # a plain copy of `bytes` reads and writes `bytes`: the factors are that
    # size over what the counters read for it
    assert cal["fetch_factor"] == pytest.approx(cal["bytes"] / (cal["fetch_kib"] * 1024))
    assert cal["write_factor"] == pytest.approx(cal["bytes"] / (cal["write_kib"] * 1024))
    total = (rec["fetch_kib_raw"] * cal["fetch_factor"] + rec["write_kib_raw"] * cal["write_factor"]) * 1024
    assert rec["bytes_per_launch"] == pytest.approx(total, rel=1e-6)
    # at least the algorithmic bytes: Q, K, V read and O written once
    w = W.get(rec["workload"])
    assert rec["bytes_per_launch"] >= 4 * w.B * w.H * w.L * w.d * 2
    # the bench reports the figure only while the kernel sources are the ones
    # the counters were taken on, and null after any change
    expect = rec["bytes_per_launch"] if rec["kernel_sha"] == bench.kernel_sha() else None
    assert bench.traffic_for(rec["workload"], bench.kernel_sha()) == expect
