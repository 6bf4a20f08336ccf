"""Host-side checks of bench.py's reporting logic (no GPU): the one-GPU
guard, and the calibrated-traffic record that feeds roofline.traffic, which
must be dropped as soon as the decode source or its build flags change."""

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
    assert "one GPU" in r.stderr


def test_traffic_record_is_keyed_on_source_and_build_flags(monkeypatch):
    path = os.path.join(ROOT, "profiles", "decode_split_b32_ctx8192_k3v4_traffic.json")
    with open(path) as f:
        rec = json.load(f)
    monkeypatch.setattr(bench, "_kernel_source_sha", lambda: rec["kernel_source_sha"])
    assert bench._traffic_record(None) == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "_kernel_source_sha", lambda: "0" * 16)
    assert bench._traffic_record(None) is None


def test_sha_covers_the_build_script(monkeypatch, tmp_path):
    src = os.path.join(ROOT, "kv_cache_vector_03_amd")
    fake = tmp_path / "kv_cache_vector_03_amd"
    (fake / "csrc").mkdir(parents=True)
    for name in ("csrc/tq_decode.hip", "csrc/tq_common.hip.h", "build.py"):
        with open(os.path.join(src, name), "rb") as f:
            (fake / name).write_bytes(f.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    before = bench._kernel_source_sha()
    (fake / "build.py").write_bytes((fake / "build.py").read_bytes() + b"\n# flags changed\n")
    assert bench._kernel_source_sha() != before


def test_traffic_record_arithmetic():
    """hbm_bytes_per_launch = FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by what the counter reads for a copy of known size."""
    with open(os.path.join(ROOT, "profiles", "decode_split_b32_ctx8192_k3v4_traffic.json")) as f:
        rec = json.load(f)
    cal = rec["copy_calibration"]
    n = cal["bytes_read_and_written"]
    assert abs(cal["fetch_scale"] - n / (cal["fetch_size_kib"] * 1024)) < 1e-4
    assert abs(cal["write_scale"] - n / (cal["write_size_kib"] * 1024)) < 1e-4
    hbm = (rec["fetch_size_kib_per_dispatch"] * 1024 * n / (cal["fetch_size_kib"] * 1024)
           + rec["write_size_kib_per_dispatch"] * 1024 * n / (cal["write_size_kib"] * 1024))
    assert abs(rec["hbm_bytes_per_launch"] - hbm) <= 1e-6 * hbm  # the KiB figures are stored rounded
    # 32 sequences x 8 KV heads x 8192 tokens x 148 B per K3V4 token-head
    assert rec["algorithmic_bytes_per_launch"] == 32 * 8 * 8192 * 148 == 32 * 8 * 8192 * bench.REC_BYTES_K3V4
