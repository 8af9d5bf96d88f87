"""Host-side checks of bench.py (no GPU): the algorithmic byte counts that the
roofline divides by, the counter summaries' scaling by the calibration copy
kernel, the source-hash guard on recorded traffic, and the one-GPU contract."""
import csv
import os
import subprocess
import sys

import pytest

import bench
import quantized_gemv_quantize_amd as qk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_workloads():
    wls = bench.workloads(qk)
    # 4096 x 11008 Q4_K: 4096 rows of 43 superblocks (6192 B), one Q8_K row of 43
    # blocks (12,556 B), 4096 f32 outputs
    assert bench.algorithmic_bytes(wls["q4_K_decode_4096x11008"], qk) == 25_362_432 + 12_556 + 16_384
    # Q6_K head dequantized: 107,520,000 B of blocks read, 524,288,000 B of f32 written
    assert bench.algorithmic_bytes(wls["q6_K_dequantize_32000x4096"], qk) == 631_808_000
    # f32 weights read, Q4_0 blocks written
    assert bench.algorithmic_bytes(wls["q4_0_quantize_row_4096x11008"], qk) == 4 * 4096 * 11008 + 25_362_432
    # gate + up pair (x read once, one f32 per row) and the Q6_K down projection
    ffn = 2 * 25_362_432 + 4_672 + 4 * 11008 + 36_986_880 + 12_556 + 4 * 4096
    assert bench.algorithmic_bytes(wls["ffn_7b_swiglu"], qk) == ffn
    # Q5_K 4096 x 11008: 43 superblocks of 176 B per row
    assert bench.algorithmic_bytes(wls["q5_K_decode_4096x11008"], qk) == 4096 * 43 * 176 + 12_556 + 16_384
    # the same FFN step with Q5_K gate / up (11008 rows of 16 superblocks of 176 B each)
    ffn5 = 2 * 11008 * 16 * 176 + 4_672 + 4 * 11008 + 36_986_880 + 12_556 + 4 * 4096
    assert bench.algorithmic_bytes(wls["ffn_7b_q5_K_swiglu"], qk) == ffn5
    # 64 columns: activations 64 x 4,672 B, outputs 64 x 14336 f32
    assert bench.algorithmic_bytes(wls["q4_K_batched_14336x4096_n64"], qk) == \
        33_030_144 + 64 * 4_672 + 4 * 64 * 14336


def test_kernel_families():
    assert bench.kernel_family("q4_K_decode_4096x11008") == "gemv"
    assert bench.kernel_family("ffn_7b_swiglu") == "gemv"
    assert bench.kernel_family("ffn_7b_q5_K_swiglu") == "gemv"
    assert bench.kernel_family("q5_K_decode_4096x11008") == "gemv"
    assert bench.kernel_family("q4_K_batched_14336x4096_n16") == "gemm"
    assert bench.kernel_family("q6_K_dequantize_32000x4096") == "dequant"
    assert bench.kernel_family("q4_0_quantize_row_4096x11008") == "quantize_row"
    assert bench._is_family("void qk::(anonymous namespace)::gemv_q4_K_kernel<4, 3, false>(...)", "gemv")
    assert not bench._is_family("qk::(anonymous namespace)::quantize_q8_K_kernel(...)", "gemv")
    assert bench._is_calib("void at::native::elementwise_kernel<neg_kernel>(...)")


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_pmc_scales_by_the_copy_kernel(tmp_path, capsys):
    gemv = "void qk::(anonymous namespace)::gemv_q4_K_kernel<4, 3, false>(unsigned char const*)"
    neg = "void at::native::vectorized_elementwise_kernel<neg_kernel_cuda>(...)"
    calib_kib = bench.CALIB_BYTES / 1024
    # FETCH_SIZE: the copy kernel reads CALIB_BYTES but the counter shows half of it;
    # two GEMV steps of 12,500 KiB (split over two counter instances each)
    _counter_csv(tmp_path / "f", [
        {"Dispatch_Id": 1, "Kernel_Name": neg, "Counter_Name": "FETCH_SIZE", "Counter_Value": calib_kib / 2},
        {"Dispatch_Id": 2, "Kernel_Name": gemv, "Counter_Name": "FETCH_SIZE", "Counter_Value": 6000},
        {"Dispatch_Id": 2, "Kernel_Name": gemv, "Counter_Name": "FETCH_SIZE", "Counter_Value": 6500},
        {"Dispatch_Id": 3, "Kernel_Name": gemv, "Counter_Name": "FETCH_SIZE", "Counter_Value": 12500},
    ])
    _counter_csv(tmp_path / "w", [
        {"Dispatch_Id": 1, "Kernel_Name": neg, "Counter_Name": "WRITE_SIZE", "Counter_Value": calib_kib},
        {"Dispatch_Id": 2, "Kernel_Name": gemv, "Counter_Name": "WRITE_SIZE", "Counter_Value": 16},
        {"Dispatch_Id": 3, "Kernel_Name": gemv, "Counter_Name": "WRITE_SIZE", "Counter_Value": 16},
    ])
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "q4_K_decode_4096x11008")
    out = dict(line.split(":", 1) for line in capsys.readouterr().out.splitlines()
               if ":" in line and not line.startswith(" "))
    assert int(out["fetch_size_bytes_per_step"]) == 2 * 12500 * 1024
    assert int(out["write_size_bytes_per_step"]) == 16 * 1024
    assert int(out["traffic_bytes_per_step"]) == 2 * 12500 * 1024 + 16 * 1024
    assert out["source_sha256"].strip() == bench.source_hash("gemv")


def test_recorded_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    f = tmp_path / "t.txt"
    monkeypatch.setattr(bench, "traffic_file", lambda workload: str(f))
    f.write_text(f"source_sha256: {bench.source_hash('gemv')}\ntraffic_bytes_per_step: 123\n")
    assert bench.recorded_traffic("q4_K_decode_4096x11008") == 123
    f.write_text("source_sha256: 0000000000000000\ntraffic_bytes_per_step: 123\n")
    assert bench.recorded_traffic("q4_K_decode_4096x11008") is None
    f.unlink()
    assert bench.recorded_traffic("q4_K_decode_4096x11008") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
