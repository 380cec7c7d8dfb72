"""Host logic of bench.py (CPU): the roofline arithmetic against figures worked by hand,
the committed HBM-traffic records and their source check, and the one-GPU contract."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from beam_inputs import WORKLOADS  # noqa: E402


def test_gate_up_roofline_decode_is_hbm_bound_with_hand_counted_bytes():
    """16 tokens, 100 routed experts: gate and up weights 100 x 2 x 2560 x 5120 BF16 bytes,
    plus x (16 x 5120 BF16) and the SwiGLU output (128 x 2560 BF16)."""
    w = WORKLOADS["beam_decode_t16"]
    r = bench.gate_up_roofline(w, 16, 100, 1.0)
    weights = 100 * 2 * 2560 * 5120 * 2
    assert r["algorithmic_bytes"] == weights + 16 * 5120 * 2 + 16 * 8 * 2560 * 2 == 5_243_699_200
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(5_243_699_200 / 1e-3 / 1e9, rel=1e-6)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, abs=1e-4)


def test_gate_up_roofline_skewed_layer_is_mfma_bound():
    """32768 tokens x top-8: 2 x 262144 x 5120 x 5120 flops = 13.74 TFLOP; at 10 ms that is
    1374 TFLOP/s, 0.55 of the 2.5 PFLOP/s BF16 peak."""
    w = WORKLOADS["beam_skewed_t32768"]
    r = bench.gate_up_roofline(w, 32768, 241, 10.0)
    assert r["algorithmic_flops"] == 2.0 * 262144 * 5120 * 5120
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(1374.4, abs=0.1)
    assert r["frac"] == pytest.approx(0.5498, abs=1e-4)


def test_gate_up_roofline_fp8_counts_block_scales_and_one_byte_weights():
    w = WORKLOADS["beam_sublayer_fp8_t8192"]
    r = bench.gate_up_roofline(w, 8192, 256, 2.0)
    weights = 256 * 2 * 2560 * 5120 + 256 * (2 * 2560 // 128) * (5120 // 128) * 4
    assert r["algorithmic_bytes"] == weights + 8192 * 5120 + 8192 * 8 * 2560 * 2
    assert r["bound"] == "hbm"


def test_traffic_records_are_current_for_the_committed_sources():
    recs = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert {"beam_decode_t16", "beam_skewed_t32768", "beam_sublayer_fp8_t8192"} <= set(recs)
    for name, rec in recs.items():
        cal = rec["copy_calibration"]
        # the copy reads and writes `bytes`; the factors turn the counters into bytes
        assert cal["fetch_factor"] == pytest.approx(cal["bytes"] / 1024 / cal["fetch_size_kib"], rel=1e-3)
        assert cal["write_factor"] == pytest.approx(cal["bytes"] / 1024 / cal["write_size_kib"], rel=1e-3)
        expect = (rec["fetch_size_kib_per_dispatch"] * cal["fetch_factor"]
                  + rec["write_size_kib_per_dispatch"] * cal["write_factor"]) * 1024
        assert rec["traffic_bytes_per_launch"] == pytest.approx(expect, rel=1e-3)
        assert bench.measured_traffic(name) == rec["traffic_bytes_per_launch"], name


def test_traffic_record_is_dropped_once_a_kernel_source_changes(tmp_path, monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["beam_skewed_t32768"]
    os.makedirs(tmp_path / "profiles")
    shutil.copy(os.path.join(ROOT, "profiles", "traffic.json"), tmp_path / "profiles")
    for src in rec["sources"]:
        os.makedirs(os.path.dirname(tmp_path / src), exist_ok=True)
        shutil.copy(os.path.join(ROOT, src), tmp_path / src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("beam_skewed_t32768") == rec["traffic_bytes_per_launch"]
    with open(tmp_path / rec["sources"][0], "a") as f:
        f.write("\n// edited\n")
    assert bench.measured_traffic("beam_skewed_t32768") is None
    assert bench.measured_traffic("no_such_workload") is None


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
