"""Host logic of bench.py (CPU only): the one-GPU guard, the algorithmic work
per launch that the rooflines divide by, the roofline record, and the
counter arithmetic of --write-traffic on synthetic rocprofv3 output."""
import csv
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_forward_units_at_text64k():
    w = workloads.get("text64k")  # B=1, H=8, L=65536, d=128, nb=1024, R=4, m=64
    N, R, d = 8 * 65536, 4, 128
    u = bench.algorithmic_units(w, "bf16", 2, None, 2, None)
    # attention: two rows read and one fp16 row plus lse written per (round, slot)
    assert u["attend"]["bytes"] == N * R * (2 * d * 2 + 4 + d * 2 + 4) == 1_627_389_952
    assert u["attend"]["flops"] == N * R * 4 * d * 128
    # hash: nb/2 MACs of length d per token-head and round, two flops each
    assert u["hash"]["flops"] == N * R * d * 1024
    # combine: R fp16 rows and lse read, one bf16 row written
    assert u["combine"]["bytes"] == N * R * (d * 2 + 4) + N * d * 2
    # the look-ahead variant widens the window by half
    u3 = bench.algorithmic_units(w, "bf16", 2, None, 3, None)
    assert 2 * u3["attend"]["flops"] == 3 * u["attend"]["flops"]


def test_backward_units_follow_the_row_width():
    w = workloads.get("text64k")
    N, R, d = 8 * 65536, 4, 128
    h = bench.backward_units(w, "bf16", 2)
    f = bench.backward_units(w, "bf16", 4)
    assert f["products"]["bytes"] - h["products"]["bytes"] == N * R * 2 * d * 2
    assert f["reduce"]["bytes"] - h["reduce"]["bytes"] == N * R * 2 * d * 2
    assert h["products"]["flops"] == N * R * 5 * 2 * d * 2 * 64


def test_ffn_units():
    u = bench.ffn_units(16384, 1024, 4096, 2)
    assert u["ffn_up"]["flops"] == u["ffn_down"]["flops"] == 2 * 16384 * 1024 * 4096
    assert u["ffn_up"]["bytes"] == 176_168_960
    assert u["ffn_down"]["bytes"] == 209_717_248


def test_roofline_record():
    units = {"attend": {"flops": 1e12, "bytes": 8e9}, "sort": {"bytes": 4e9}}
    r = bench.roofline("attend", units, 2.0)  # 2 ms: 4 TB/s, 500 TFLOP/s
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"  # 1 ms of HBM > 0.4 ms of MFMA
    assert r["achieved"] == pytest.approx(4000.0)
    assert r["frac"] == pytest.approx(0.5)
    assert r["kernel"] == "k_attend_mfma"
    units["attend"]["flops"] = 1e14  # now 40 ms of MFMA against 1 ms of HBM
    r = bench.roofline("attend", units, 100.0)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(1000.0)
    assert r["frac"] == pytest.approx(0.4)
    r = bench.roofline("sort", units, 1.0)
    assert r["bound"] == "hbm" and r["achieved"] == pytest.approx(4000.0)


def _pmc_csv(folder, counter, rows):
    os.makedirs(folder)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_write_traffic_scales_by_the_calibration_copy(tmp_path):
    mib = 64
    copy = "__amd_rocclr_copyBuffer"
    up, down = "void lsh::k_ffn_mfma<true, 256>(int)", "void lsh::k_ffn_mfma<false, 256>(int)"
    # the copy of 64 MiB reads half of its bytes in FETCH_SIZE, all in WRITE_SIZE
    _pmc_csv(str(tmp_path / "f"), "FETCH_SIZE",
             [(copy, mib * 512), (up, 1000.0), (up, 3000.0), (down, 500.0)])
    _pmc_csv(str(tmp_path / "w"), "WRITE_SIZE",
             [(copy, mib * 1024), (up, 100.0), (up, 100.0), (down, 40.0)])
    out = tmp_path / "traffic.json"
    args = types.SimpleNamespace(write_traffic=[str(tmp_path / "f"), str(tmp_path / "w")],
                                 calib_copy_mib=mib, traffic_json=str(out), workload="text64k",
                                 backward=False, ffn=True)
    bench.write_traffic(args)
    got = json.loads(out.read_text())["text64k:ffn"]
    # mean per dispatch, each counter scaled by known bytes / what it read for the copy
    assert got["ffn_up"]["bytes_per_launch"] == round(2000.0 * 1024 * 2.0 + 100.0 * 1024 * 1.0)
    assert got["ffn_down"]["bytes_per_launch"] == round(500.0 * 1024 * 2.0 + 40.0 * 1024 * 1.0)
    assert got["ffn_up"]["source_hash"] == bench.kernel_source_hash("ffn_up")
