"""The measurement plumbing on the CPU: bench.py refuses more than one GPU,
the roofline's traffic and clock records are taken only while the kernel
sources match their hash, and the rocprofv3 summaries come out of small
synthetic CSV files with the figures their formulas give."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_and_clock_follow_the_kernel_hash(tmp_path, monkeypatch):
    import bench
    h = bench.kernel_source_hash()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "attn_d256_f16_paged_32k_traffic.json").write_text(
        json.dumps({"kernel_source_hash": h, "hbm_bytes_per_launch": 123.0}))
    (prof / "attn_d256_f16_paged_32k_mfma_counters.json").write_text(
        json.dumps({"kernel_source_hash": h, "clock_ghz_upper_bound": 1.5}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic(h) == 123.0
    assert bench.load_clock(h) == 1.5
    assert bench.load_traffic("0" * 16) is None
    assert bench.load_clock("0" * 16) is None


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


COUNTER_HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
                  "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
                  "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"]
KERNEL = "void ppa::(anonymous namespace)::attn_partial_kernel<256, ppa::(anonymous namespace)::F16, " \
         "(ppa::(anonymous namespace)::Addr)2, false, 1>(ppa::AttnArgs)"


def _counter_row(dispatch, kernel, name, value, t0=1000, t1=2000):
    return [dispatch, dispatch, "Agent 1", 1, 1, 1, 1024, 7, kernel, 256, 0, 0, 8, 0, 32, name, value, t0, t1]


def test_traffic_summary_scales_by_the_copy(tmp_path):
    from paged_kv_prefill_amd import profsum
    copy = 1 << 30
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the copy reads half its bytes by FETCH_SIZE's count and writes all of them
    _write_csv(fetch, COUNTER_HEADER, [_counter_row(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", copy / 1024 / 2),
                                       _counter_row(2, KERNEL, "FETCH_SIZE", 1000.0)])
    _write_csv(write, COUNTER_HEADER, [_counter_row(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", copy / 1024),
                                       _counter_row(2, KERNEL, "WRITE_SIZE", 100.0)])
    out = tmp_path / "t.json"
    profsum.traffic(str(fetch), str(write), str(out), "attn_partial_kernel<256, F16, (Addr)2", copy, "f", "w")
    rec = json.loads(out.read_text())
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_bytes_per_launch"] == pytest.approx((1000.0 * 2 + 100.0) * 1024)


def test_counter_summary_figures(tmp_path):
    from paged_kv_prefill_amd import profsum
    path = tmp_path / "c.csv"
    dur_ns = 1_000_000
    rows = []
    vals = {"SQ_INSTS_VALU_MFMA_MOPS_F16": 64.0 * 1000, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 0.0,
            "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 800_000.0, "SQ_INSTS_MFMA": 1000.0,
            "GRBM_GUI_ACTIVE": 8 * 1.6 * dur_ns}
    for name, v in vals.items():
        rows.append(_counter_row(5, KERNEL, name, v, 0, dur_ns))
    _write_csv(path, COUNTER_HEADER, rows)
    out = tmp_path / "c.txt"
    profsum.counters(str(path), str(out), "attn_partial_kernel<256, F16, (Addr)2", 64.0 * 1000 * 512, 10.0,
                     1000.0, "cmd")
    text = out.read_text()
    rec = json.loads((tmp_path / "c.json").read_text())
    assert rec["mfma_flops_counted"] == pytest.approx(64.0 * 1000 * 512)
    assert rec["clock_ghz_upper_bound"] == pytest.approx(1.6)
    assert rec["mfma_busy_cycles_per_simd"] == pytest.approx(800_000.0)
    assert "1.000 x exact" in text
    # 800,000 busy cycles per SIMD over 1 ms at 1.6 GHz: 50% of the engine cycles
    assert "50.0 %" in text
    # against the launch at 2.4 GHz: 800,000 / 2,400,000
    assert "33.3 %" in text


def test_power_summary_and_its_hash(tmp_path, monkeypatch):
    import bench
    from paged_kv_prefill_amd import profsum
    phases = {"samples": 40,
              "idle": {"power_w_median": 300.0, "gfx_clock_mhz_mean": 2400.0, "n_samples": 8},
              "matmul_f16_8192": {"power_w_median": 1400.0, "gfx_clock_mhz_mean": 1700.0, "n_samples": 10,
                                  "ms_per_call": 0.88, "tflops": 1250.0},
              "sweep_32768": {"power_w_median": 1350.0, "gfx_clock_mhz_mean": 1690.0, "n_samples": 10,
                              "ms_per_call": 1.07, "tflops": 1000.0}}
    out = tmp_path / "bench.json"
    out.write_text("# log line\n" + json.dumps({"config": {"power": phases}}) + "\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    txt = prof / "power_clock_sustained_chunks_and_f16_matmul.txt"
    profsum.power(str(out), str(txt), "python3 bench.py --power 10")
    body = txt.read_text()
    assert "python3 bench.py --power 10" in body
    row = next(l for l in body.splitlines() if l.startswith("sweep_32768"))
    assert row.split()[-2:] == ["0.400", "0.800"]   # of 2.5 PF, of the matmul
    rec = json.loads((prof / "power_clock_sustained_chunks_and_f16_matmul.json").read_text())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_power(rec["kernel_source_hash"])["matmul_f16_8192"]["tflops"] == 1250.0
    assert bench.load_power("0" * 16) is None
