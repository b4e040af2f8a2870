"""bench.py's host-side contract, without a GPU: one GPU only, and the HBM
traffic figure reported only while the product kernels' sources are the ones
the committed counter profile was taken on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_follows_the_kernel_sources(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    key = "gemm_w8a8[dit_gateup]"
    assert key in rec["kernels"]
    monkeypatch.setattr(bench, "_src_hash", lambda: rec["source_hash"])
    assert bench._traffic_for(key) == rec["kernels"][key]["bytes_per_launch"]
    assert bench._traffic_for("no such launch") is None
    monkeypatch.setattr(bench, "_src_hash", lambda: "0" * 16)  # the kernels changed since the counters
    assert bench._traffic_for(key) is None


def test_source_hash_covers_the_product_sources(tmp_path, monkeypatch):
    """Editing any product source changes the hash (so stale counts are not reported)."""
    src = os.path.join(ROOT, "int4_quantized_gemm_amd", "csrc")
    copy = tmp_path / "int4_quantized_gemm_amd" / "csrc"
    copy.mkdir(parents=True)
    for f in bench.GEMM_SOURCES:
        (copy / f).write_bytes(open(os.path.join(src, f), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench._src_hash()
    assert h0 == bench._src_hash()
    for f in bench.GEMM_SOURCES:
        p = copy / f
        orig = p.read_bytes()
        p.write_bytes(orig + b"\n")
        assert bench._src_hash() != h0, f"{f} is not covered"
        p.write_bytes(orig)
    assert bench._src_hash() == h0
