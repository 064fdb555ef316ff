"""Host-side logic of bench.py (no GPU): the algorithmic byte counts the
reported rates divide by, the HBM traffic record and its source check, and
the one-GPU guard."""
import csv
import json
import os
import shutil
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from decode_attention_dq_amd import workloads  # noqa: E402


def test_headline_algorithmic_bytes():
    """128 sequences x 8192 tokens x 8 KV heads x (37-byte K + fp16 norm + 37-byte V + fp16 norm)."""
    w = workloads.WORKLOADS["decode_qwen3_8b"]
    lens = workloads.context_lengths(w)
    assert bench.algorithmic_bytes(w, lens) == 128 * 8192 * 8 * 2 * 39 == 654_311_424


def test_long_context_algorithmic_bytes():
    w4, w1 = workloads.WORKLOADS["long_llama_b4"], workloads.WORKLOADS["long_llama_b1"]
    assert bench.algorithmic_bytes(w4, workloads.context_lengths(w4)) == 4 * 65536 * 8 * 2 * 39
    assert bench.algorithmic_bytes(w1, workloads.context_lengths(w1)) == 131072 * 8 * 2 * 39


def test_window_and_means_bytes():
    """A bf16 window token adds K and V rows of 256 bytes per KV head; a key block
    of up to 128 tokens adds 128 INT8 means and an fp16 scale per KV head."""
    w = workloads.WORKLOADS["decode_qwen3_8b"]
    lens = np.array([300, 128], np.int64)
    base = bench.algorithmic_bytes(w, lens)
    assert bench.algorithmic_bytes(w, lens, window_lens=np.array([5, 0])) == base + 5 * 8 * 2 * 256

    class WithMeans:
        container, cv, num_kv_heads, means = w.container, w.cv, w.num_kv_heads, True
    assert bench.algorithmic_bytes(WithMeans, lens) == base + (3 + 1) * 8 * 130


def test_traffic_record_follows_sources(monkeypatch):
    """The record is reported only while it carries the hash of the decode
    kernel's current sources and names the workload; otherwise null."""
    rec = json.load(open(bench.TRAFFIC_JSON))["attn_kernel"]
    current = rec["source_sha256"] == bench.attn_source_hash()
    expected = int(rec["traffic_bytes_per_launch"]) if current else None
    assert bench.recorded_traffic("attn_kernel", "decode_qwen3_8b") == expected
    assert bench.recorded_traffic("attn_kernel", "long_llama_b4") is None
    monkeypatch.setattr(bench, "attn_source_hash", lambda: "0" * 64)
    assert bench.recorded_traffic("attn_kernel", "decode_qwen3_8b") is None


def test_issue_record_follows_sources(monkeypatch):
    """The measured VALU-issue and LDS-active fractions are reported only while
    their record carries the current sources' hash."""
    sq = json.load(open(bench.TRAFFIC_JSON))["attn_kernel"].get("sq")
    got = bench.recorded_issue("attn_kernel", "decode_qwen3_8b")
    if sq is not None and sq["source_sha256"] == bench.attn_source_hash():
        assert got == {"valu_issue_frac": sq["valu_issue_frac"], "lds_active_frac": sq["lds_active_frac"]}
        # the VALU figure counts 4 cycles per wave instruction and can pass 1 (simple
        # VOP2 instructions issue in fewer); the LDS figure is a true fraction
        assert 0.0 < got["valu_issue_frac"] < 1.5 and 0.0 < got["lds_active_frac"] <= 1.0
    else:
        assert got is None
    monkeypatch.setattr(bench, "attn_source_hash", lambda: "0" * 64)
    assert bench.recorded_issue("attn_kernel", "decode_qwen3_8b") is None


def test_record_traffic_scales_by_copy(tmp_path, monkeypatch):
    """Traffic = FETCH_SIZE and WRITE_SIZE (KiB, mean over the headline
    kernel's dispatches) times the copy calibration's bytes-per-KiB factors."""
    tj = tmp_path / "traffic.json"
    shutil.copy(bench.TRAFFIC_JSON, tj)
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tj))
    name = "void dq::(anonymous namespace)::attn_kernel<false, false, false>(dq::(anonymous namespace)::AttnLaunch)"

    def write(path, counter, values):
        with open(path, "w", newline="") as f:
            wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            wr.writeheader()
            for v in values:
                wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})
            wr.writerow({"Kernel_Name": "other", "Counter_Name": counter, "Counter_Value": 1e9})
    write(tmp_path / "f.csv", "FETCH_SIZE", [100.0, 300.0])
    write(tmp_path / "w.csv", "WRITE_SIZE", [10.0])
    rec = bench.record_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    fs = rec["copy_bytes"] / (rec["copy_fetch_kib"] * 1024)
    ws = rec["copy_bytes"] / (rec["copy_write_kib"] * 1024)
    assert rec["fetch_size_kib"] == 200.0 and rec["write_size_kib"] == 10.0 and rec["dispatches"] == [2, 1]
    assert abs(rec["traffic_bytes_per_launch"] - (200.0 * 1024 * fs + 10.0 * 1024 * ws)) < 1e-6
    assert json.load(open(tj))["attn_kernel"]["traffic_bytes_per_launch"] == rec["traffic_bytes_per_launch"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_units_and_host_info():
    """The CPU baseline's work units run the oracle on the workloads' shapes and
    report their own work; the host record names the core count and CPU."""
    info = bench.host_info()
    assert info["cpu_count"] == os.cpu_count() and isinstance(info["cpu_model"], str)
    t, nbytes, streams = bench._cpu_decode_unit((0, 3, 1))
    assert t > 0 and nbytes == 8192 * 2 * 39 and streams == 2 * 8192
    t, streams = bench._cpu_encode_unit((0, 0, 5))
    assert t > 0 and streams == 8192
