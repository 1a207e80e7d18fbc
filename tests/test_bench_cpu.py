"""Host logic of bench.py (no GPU): the one-GPU guard, the HBM-traffic summary
built from two rocprofv3 counter CSVs scaled by the calibration copy, and the
rule that traffic taken on other kernel sources is not reported."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


@pytest.fixture
def traffic_file(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    return path


def test_counter_summary_scales_by_the_copy(tmp_path, traffic_file):
    gib_kib = (1 << 30) / 1024
    # the copy moves 1 GiB each way; FETCH_SIZE reads half of it, WRITE_SIZE all
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _write_csv(fetch, "FETCH_SIZE", [
        ("copyBuffer(...)", gib_kib / 2),
        ("void lce::k_logits_lse<unsigned short, true, false, false>(...)", 1000.0),
        ("void lce::k_logits_lse<unsigned short, true, false, false>(...)", 1200.0),
        ("void lce::k_logits_lse<unsigned short, true, false, false>(...)", 1100.0),
        ("void lce::k_gemm_grad_w<unsigned short, 3, false, true>(...)", 50.0),
        ("void lce::k_gemm_grad_w<unsigned short, 0, false, true>(...)", 5.0),
        ("some_other_kernel", 9e9),
    ])
    _write_csv(write, "WRITE_SIZE", [
        ("copyBuffer(...)", gib_kib),
        ("void lce::k_logits_lse<unsigned short, true, false, false>(...)", 300.0),
        ("void lce::k_logits_lse<unsigned short, true, false, false>(...)", 300.0),
        ("void lce::k_gemm_grad_w<unsigned short, 3, false, true>(...)", 7.0),
        ("void lce::k_gemm_grad_w<unsigned short, 0, false, true>(...)", 1.0),
    ])
    out = bench.summarize_counters(str(fetch), str(write), "w1", "cmd")
    # grad_W's main launch (bf16 store) and its K-split tail are kept apart
    assert set(out) == {"logits", "gemm_w", "gemm_w_tail"}
    assert out["gemm_w"]["read_bytes"] == pytest.approx(50.0 * 2.0 * 1024)
    assert out["gemm_w_tail"]["write_bytes"] == pytest.approx(1.0 * 1024)
    lg = out["logits"]
    assert lg["copy_scale_fetch"] == pytest.approx(2.0)
    assert lg["copy_scale_write"] == pytest.approx(1.0)
    assert lg["read_bytes"] == pytest.approx(1100.0 * 2.0 * 1024)     # the median dispatch
    assert lg["write_bytes"] == pytest.approx(300.0 * 1024)
    assert lg["bytes_per_launch"] == pytest.approx(lg["read_bytes"] + lg["write_bytes"])
    assert json.loads(traffic_file.read_text())["w1"]["gemm_w"]["command"] == "cmd"
    assert bench.load_traffic("logits", "w1") == pytest.approx(lg["bytes_per_launch"])
    assert bench.load_traffic("gemm_x", "w1") is None
    assert bench.load_traffic("logits", "other") is None


def test_traffic_of_other_kernel_sources_is_not_reported(tmp_path, traffic_file, monkeypatch):
    traffic_file.write_text(json.dumps(
        {"w1": {"logits": {"bytes_per_launch": 5.0, "source_sha": bench.kernel_source_sha()}}}))
    assert bench.load_traffic("logits", "w1") == 5.0
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 16)
    assert bench.load_traffic("logits", "w1") is None


def test_no_copy_calibration_means_no_traffic(tmp_path, traffic_file):
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    _write_csv(fetch, "FETCH_SIZE", [("k_logits_lse", 10.0)])
    _write_csv(write, "WRITE_SIZE", [("k_logits_lse", 10.0)])
    assert bench.summarize_counters(str(fetch), str(write), "w1", "cmd") == {}


def test_host_cpu_record():
    """The CPU baseline states the host's logical CPU count and model next to
    the threads the oracle used."""
    h = bench.host_cpu()
    assert h["nproc"] == os.cpu_count() and h["nproc"] >= 1
    assert h["nproc_usable"] is None or 1 <= h["nproc_usable"] <= h["nproc"]
    assert "cpu_model" in h


def test_bench_flags_parse():
    """The default line's extra records can be switched off; --group-rows
    reaches the op."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for flag in ("--group-rows", "--no-per-chunk", "--no-ce"):
        assert flag in r.stdout


def test_traffic_only_for_the_counted_plan():
    """The committed counters were taken on the default plan; compact, a group
    cap, another chunk size or the loss-only forward launch other shapes."""
    import argparse
    cfg = type("Cfg", (), {"name": "large-vocab-bf16"})()
    base = dict(acc_policy="accurate", group_rows=0, chunk_rows=None, forward_only=False)
    assert bench.counted_plan(argparse.Namespace(**base), "large-vocab-bf16", cfg)
    for k, v in (("acc_policy", "compact"), ("group_rows", 2048), ("chunk_rows", 1024),
                 ("forward_only", True)):
        assert not bench.counted_plan(argparse.Namespace(**{**base, k: v}), "large-vocab-bf16", cfg)
    assert not bench.counted_plan(argparse.Namespace(**base), "large-vocab-f16", cfg)
