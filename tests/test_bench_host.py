"""Host logic of bench.py (no GPU): the one-GPU contract, the per-token byte
count the roofline uses, and the HBM-traffic summary (counter arithmetic and the
rule that a summary taken on other decode sources is not reported)."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_fp4_bytes_per_token_head():
    # K and V, each 16 B of codes and 1 scale byte per 32 channels
    assert bench.fp4_kv_bytes_per_token_head(128) == 2 * (64 + 4) == 136
    assert bench.fp4_kv_bytes_per_token_head(64) == 68


def _counter_csv(path, counter, decode_vals, copy_vals):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for v in decode_vals:
            w.writerow({"Kernel_Name": "void uq::decode_kernel<uq::Fp4PairPol<128>, 128, 0, 0, true, false>",
                        "Counter_Name": counter, "Counter_Value": v})
        for v in copy_vals:
            w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter, "Counter_Value": v})
        w.writerow({"Kernel_Name": "other", "Counter_Name": counter, "Counter_Value": 1e9})


def test_counter_summary_scales_traffic_by_the_copy(tmp_path, monkeypatch):
    # a 1 GiB copy that reads as 2 GiB of fetch (factor 1/2) and 1 GiB of write
    # (factor 1): decode 1000 KiB fetched -> 500 KiB, 10 KiB written -> 10 KiB
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "traffic.md"))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    (tmp_path / "profiles").mkdir()
    fetch, write, mfma = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "m.csv"
    _counter_csv(fetch, "FETCH_SIZE", [1000.0, 1000.0], [2.0 * (1 << 20), 5.0])
    _counter_csv(write, "WRITE_SIZE", [10.0, 10.0], [1.0 * (1 << 20)])
    with open(mfma, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        k = "void uq::decode_kernel<uq::Fp4PairPol<128>, 128, 0, 0, true, false>"
        w.writerow({"Kernel_Name": k, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES", "Counter_Value": 1024 * 100.0})
        w.writerow({"Kernel_Name": k, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 1000.0})
    d = bench.summarize_counters("decode", [str(fetch), str(write), str(mfma)])
    assert d["traffic"] == 522240                                     # (500 + 10) KiB
    assert abs(d["mfma_busy"] - 0.8) < 1e-12                          # 102400 / (1000 / 8 x 256 x 4)
    text = (tmp_path / "profiles" / "decode_fp4_64x8192_counters.md").read_text()
    assert "--pmc-pass decode" in text and f"source_sha256: {bench.decode_source_sha()}" in text
    assert bench.recorded_traffic() == 522240
    # the same summary is not reported once the decode sources differ
    monkeypatch.setattr(bench, "decode_source_sha", lambda: "0" * 16)
    assert bench.recorded_traffic() is None


def test_counter_summary_needs_the_kernels_dispatches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    fetch = tmp_path / "f.csv"
    _counter_csv(fetch, "FETCH_SIZE", [], [1.0 * (1 << 20)])
    with pytest.raises(SystemExit):
        bench.summarize_counters("decode", [str(fetch)])


def test_oracle_baseline_of_a_step_without_prefix():
    # the tiny configuration writes its whole sequence in the step: no prefix to
    # build, one (sequence, KV head) pair
    from bit_kv_cache_wht_amd import workloads as W
    r = bench.cpu_baseline(W.tiny(), 1.0)
    assert r["kind"] == "oracle" and r["unit"] == "us/step" and r["value"] > 0
    assert r["sample"].startswith("1 of 1 ")


def test_oracle_append_baseline_covers_every_token():
    from bit_kv_cache_wht_amd import workloads as W
    wl = W.make_workload("append_small", 1, 2, 2, 64, [300], [300], seed=5)
    r = bench.cpu_append_baseline(wl)
    assert r["kind"] == "oracle" and r["unit"] == "us/call" and r["value"] > 0
    assert r["sample"].startswith("all 300 tokens x 2 KV heads")
    assert abs(r["tokens_per_s"] - 300 / (r["value"] * 1e-6)) <= 0.01 * r["tokens_per_s"]
