"""Host logic of bench.py that needs no GPU: the rocprofv3 summary
(durations, calibrated traffic, MFMA utilisation) and the multi-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _counter_rows(kernel, counter, values, dur_ns):
    return [[kernel, counter, v, 1000, 1000 + dur_ns] for v in values]


CH = ["Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def test_summarize_calibrates_traffic_and_mfma(tmp_path):
    k_gemm = "void bl::(anonymous namespace)::k_gemm<8, 4>(unsigned char const*, long)"
    k_copy = "__amd_rocclr_copyBuffer"
    _write_csv(str(tmp_path / "stats" / "s_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
               [[k_gemm, 4, 400000, 100000, 100.0, 90000, 110000, 1.0]])
    # FETCH_SIZE reads half the bytes for the copy (factor 2), WRITE_SIZE all of them
    _write_csv(str(tmp_path / "calf" / "c_counter_collection.csv"), CH,
               _counter_rows(k_copy, "FETCH_SIZE", [524288.0], 1000))
    _write_csv(str(tmp_path / "calw" / "c_counter_collection.csv"), CH,
               _counter_rows(k_copy, "WRITE_SIZE", [1048576.0], 1000))
    _write_csv(str(tmp_path / "fetch" / "f_counter_collection.csv"), CH,
               _counter_rows(k_gemm, "FETCH_SIZE", [1000.0, 3000.0], 100000))
    _write_csv(str(tmp_path / "write" / "w_counter_collection.csv"), CH,
               _counter_rows(k_gemm, "WRITE_SIZE", [512.0], 100000))
    # MFMA busy for half the SIMD-cycles of a 100 us dispatch; 1e6 MFMA instructions
    busy = 0.5 * 100e3 * 2.4 * 1024
    _write_csv(str(tmp_path / "mfma" / "m_counter_collection.csv"), CH,
               _counter_rows(k_gemm, "SQ_VALU_MFMA_BUSY_CYCLES", [busy], 100000) +
               _counter_rows(k_gemm, "SQ_INSTS_MFMA", [1e6], 100000))
    out = tmp_path / "out"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize", "t", "--workload", "w",
                        "--stats", str(tmp_path / "stats"), "--pmc", str(tmp_path / "fetch"),
                        "--pmc", str(tmp_path / "write"), "--pmc", str(tmp_path / "mfma"),
                        "--calib", str(tmp_path / "calf"), str(tmp_path / "calw"), "--command", "cmd",
                        "--out-dir", str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    md = (out / "t.md").read_text()
    assert "| k_gemm | 4 | 100.000 |" in md
    assert "| k_gemm | 50.0% | 1000000 |" in md
    traffic = json.loads((out / "traffic.json").read_text())["w"]["k_gemm"]
    # (2000 KiB * 2 + 512 KiB * 1) per launch
    assert traffic["bytes_per_launch"] == round(2000 * 1024 * 2.0 + 512 * 1024)
    assert traffic["calibration"] == {"fetch": 2.0, "write": 1.0}


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
