"""Host logic of bench.py, on the CPU: the one-GPU contract and the profile
summaries built from rocprofv3 CSV output (synthetic CSVs, checked against
numbers worked out by hand)."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

DKDV = "void attn::(anonymous namespace)::attn_dkdv_pair_kernel<128>(attn::BwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _counters(path, values):
    """values: [(kernel, dispatch, grid, counter, value)], one row each."""
    _write_csv(path, ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"],
               [[d, g, k, c, v] for k, d, g, c, v in values])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_summaries_from_synthetic_rocprof_output(tmp_path):
    stats, fetch, write, mfma, out = (str(tmp_path / n) for n in ("stats", "fetch", "write", "mfma", "out"))
    os.makedirs(out)
    _write_csv(os.path.join(stats, "run_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
               [[DKDV, 6, 9300000, 1550000, 100, 1000000, 2100000, 0]])
    # --warmup 1 --steps 2: the headline leg is 3 dispatches (1 untimed), then the causal leg 3 (1 untimed).
    durations_us = [2100, 2000, 2000, 1200, 1000, 1000]
    t = 0
    rows = []
    for d in durations_us:
        rows.append([DKDV, t, t + d * 1000])
        t += d * 1000 + 500
    _write_csv(os.path.join(stats, "run_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               rows)
    # The copy reads 256 MiB and writes 256 MiB; FETCH_SIZE reads half of it, WRITE_SIZE all of it.
    _counters(os.path.join(fetch, "run_counter_collection.csv"),
              [(COPY, 1, 4096, "FETCH_SIZE", 65536.0), (COPY, 1, 4096, "FETCH_SIZE", 65536.0),
               (DKDV, 2, 524288, "FETCH_SIZE", 200000.0)])
    _counters(os.path.join(write, "run_counter_collection.csv"),
              [(COPY, 1, 4096, "WRITE_SIZE", 262144.0), (DKDV, 2, 524288, "WRITE_SIZE", 100000.0)])
    cyc = 4.2e6  # cycles per XCD during the launch: 2.1 GHz over the 2000 us headline median
    _counters(os.path.join(mfma, "run_counter_collection.csv"),
              [(DKDV, d, 524288, c, v) for d in range(1, 7)
               for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * 1024), ("SQ_INSTS_MFMA", 7.0e7),
                            ("GRBM_GUI_ACTIVE", 8 * cyc))])
    cmd = "rocprofv3 ... -- python3 bench.py --warmup 1 --steps 2"
    bench.summarize(stats, fetch, write, cmd, "counter command", out_dir=out)
    bench.summarize_mfma(stats, mfma, "mfma command", cmd, out_dir=out)

    traffic = json.load(open(os.path.join(out, "hbm_traffic.json")))
    # (200000 KiB x 2 + 100000 KiB x 1) per launch
    assert traffic["kernels"]["attn_dkdv_pair_kernel"]["bytes_per_launch"] == (200000 * 2 + 100000) * 1024
    assert traffic["source_digest"] == bench.source_digest()
    stats_md = open(os.path.join(out, "fwd_bwd_d128_T8192_kernel_stats.md")).read()
    assert "| `attn_dkdv_pair_kernel<128>` | 3 | 2000.00 | 1000.00 |" in stats_md
    mfma_md = open(os.path.join(out, "fwd_bwd_d128_T8192_mfma_util.md")).read()
    assert "| 2000.0 | 2.10 | 50.0% |" in mfma_md


def test_traffic_counts_the_headline_leg_and_every_decode_dispatch(tmp_path):
    """Later legs launch the tile kernels on other workloads with the same grid; they must not be averaged in."""
    stats, fetch, write, out = (str(tmp_path / n) for n in ("stats", "fetch", "write", "out"))
    os.makedirs(out)
    _write_csv(os.path.join(stats, "run_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"], [])
    _write_csv(os.path.join(stats, "run_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], [])
    split = "void attn::(anonymous namespace)::attn_decode_split_kernel<128>(attn::DecodeArgs)"
    # --warmup 1 --steps 2: dispatches 2-4 are the headline leg (300000 KiB each), 5-7 the causal leg
    # (same grid, 150000 KiB); the decode kernel runs twice later, 1000 and 3000 KiB.
    f_rows = [(COPY, 1, 4096, "FETCH_SIZE", 131072.0)]
    f_rows += [(DKDV, d, 524288, "FETCH_SIZE", 300000.0 if d < 5 else 150000.0) for d in range(2, 8)]
    f_rows += [(split, 8, 1024, "FETCH_SIZE", 1000.0), (split, 9, 1024, "FETCH_SIZE", 3000.0)]
    # A kernel that only a later leg launches (another head_dim) is not part of the headline leg.
    short = "void attn::(anonymous namespace)::attn_fwd_bf16_kernel<64>(attn::FwdArgs)"
    f_rows += [(short, 10, 32768, "FETCH_SIZE", 5.0e6)]
    _counters(os.path.join(fetch, "run_counter_collection.csv"), f_rows)
    w_rows = [(COPY, 1, 4096, "WRITE_SIZE", 262144.0)]
    w_rows += [(DKDV, d, 524288, "WRITE_SIZE", 100000.0 if d < 5 else 10.0) for d in range(2, 8)]
    w_rows += [(split, 8, 1024, "WRITE_SIZE", 10.0), (split, 9, 1024, "WRITE_SIZE", 30.0)]
    _counters(os.path.join(write, "run_counter_collection.csv"), w_rows)
    bench.summarize(stats, fetch, write, "python3 bench.py --warmup 1 --steps 2",
                    "rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --warmup 1 --steps 2", out_dir=out)
    kern = json.load(open(os.path.join(out, "hbm_traffic.json")))["kernels"]
    assert "attn_fwd_bf16_kernel" not in kern
    assert kern["attn_dkdv_pair_kernel"]["bytes_per_launch"] == (300000 * 2 + 100000) * 1024
    assert kern["attn_decode_split_kernel"]["bytes_per_launch"] == (2000 * 2 + 20) * 1024


def test_stored_traffic_needs_the_current_sources(tmp_path):
    path = str(tmp_path / "hbm_traffic.json")
    rec = {"source_digest": bench.source_digest(), "kernels": {"attn_dkdv_pair_kernel": {"bytes_per_launch": 7}}}
    json.dump(rec, open(path, "w"))
    assert bench.stored_traffic("attn_dkdv_pair_kernel", path) == 7
    assert bench.stored_traffic("attn_fwd_bf16_kernel", path) is None
    rec["source_digest"] = "0" * 16
    json.dump(rec, open(path, "w"))
    assert bench.stored_traffic("attn_dkdv_pair_kernel", path) is None


@pytest.mark.parametrize("steps", [2])
def test_fp32_summary_splits_full_and_causal_launches(tmp_path, steps):
    stats, out = str(tmp_path / "stats"), str(tmp_path / "out")
    os.makedirs(out)
    name = "void attn::(anonymous namespace)::attn_fwd_f32_kernel<128>(attn::FwdArgs)"
    grid = 256 * (4096 // 128) * 8 * 4  # B4 H8 T4096, 128 query rows per workgroup
    rows, t = [], 0
    for d in (2200, 2200, 2210, 1250, 1240, 1250):  # non-causal launches first, then causal
        rows.append([name, t, t + d * 1000, grid])
        t += d * 1000 + 500
    _write_csv(os.path.join(stats, "run_kernel_trace.csv"),
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"], rows)
    bench.summarize_fp32(stats, "cmd", out_dir=out)
    md = open(os.path.join(out, "fp32_grid_kernel_stats.md")).read()
    # 4 B H T^2 D = 2.749e11 flop in 2.2 ms; half of it in 1.25 ms when causal.
    assert "| fp32_d128_T4096_full | 3 | 2200.0 | 124.9 | 79% |" in md
    assert "| fp32_d128_T4096_causal | 3 | 1250.0 | 110.0 | 70% |" in md


def test_issue_counter_summary_from_synthetic_passes(tmp_path):
    """Ratios of the issue/wait summary, from two synthetic counter passes of
    two dispatches each (the values are averaged per dispatch)."""
    a, b, out = (str(tmp_path / n) for n in ("a", "b", "out"))
    os.makedirs(out)
    _counters(os.path.join(a, "run_counter_collection.csv"),
              [(DKDV, d, 1048576, c, v) for d in (1, 2)
               for c, v in (("SQ_WAVE_CYCLES", 1000.0), ("SQ_WAIT_ANY", 300.0), ("SQ_WAIT_INST_ANY", 250.0),
                            ("SQ_ACTIVE_INST_ANY", 450.0))])
    _counters(os.path.join(b, "run_counter_collection.csv"),
              [(DKDV, d, 1048576, c, v) for d in (1, 2)
               for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", 3200.0), ("SQ_VALU_MFMA_COEXEC_CYCLES", 800.0),
                            ("SQ_INSTS_MFMA", 100.0), ("SQ_INSTS_VALU", 460.0), ("SQ_INSTS_SALU", 230.0),
                            ("SQ_INSTS_LDS", 150.0), ("SQ_LDS_BANK_CONFLICT", 0.0))])
    bench.summarize_stalls([a, b], "pass a\npass b", out_dir=out)
    md = open(os.path.join(out, "fwd_bwd_d128_T8192_issue_counters.md")).read()
    # co-issue 800/3200, waits 300/1000 and 250/1000, active 450/1000, 4.6 / 2.3 / 1.5 per MFMA
    assert "| `attn_dkdv_pair_kernel<128>` | 1048576 | 25% | 30% | 25% | 45% | 4.60 | 2.30 | 1.50 | 0 |" in md
    assert "pass a\npass b" in md


def test_suites_summary_from_a_bench_line(tmp_path):
    """The --summarize-suites tables come from a bench JSON line alone (no GPU)."""
    import json
    import bench
    line = {"value": 900.0, "steps": 20, "ms_per_step": 4.2, "per_kernel_ms": {"attn_fwd": 1.0},
            "roofline": {"kernel": "attn_dkdv_pair_kernel", "achieved": 1200.0, "frac": 0.48, "peak": 2516.6},
            "timing_spread": {"per_step_ms": {"median": 4.2, "q1": 4.1, "q3": 4.3}},
            "decode_suite": {"rows": [{"B": 8, "keys": 65536, "Hkv": 8, "us_per_call": 300.0, "gbs": 6000.0,
                                       "workspace_bytes": 2**21, "output_bytes": 65536 + 1024,
                                       "device_peak_bytes": 3 * 2**20}]},
            "memory": {"device_peak": {"rows": [{"T": 1024, "device_peak_mb": 3.0, "inputs_mb": 32.0}]},
                       "residuals": {"rows": [{"T": 1024, "residual_mb": 2.06}]}},
            "cpu_baseline": {"value": 0.12, "cores": 16, "sample": "s", "blas": "openblas",
                             "per_workload": {"unit": "ms", "threads": 16, "rows": [
                                 {"workload": "fp32_mha_T128_d64", "sample": "whole workload", "calls": 3,
                                  "fwd_ms": 0.5, "fwd_bwd_ms": 2.0, "fwd_ms_1thread": 0.6,
                                  "fwd_bwd_ms_1thread": 2.4}]}}}
    log = tmp_path / "bench.log"
    log.write_text("progress\n" + json.dumps(line) + "\n")
    bench.summarize_suites(str(log), "python3 bench.py --suites", out_dir=str(tmp_path))
    text = (tmp_path / "suites_and_legs.md").read_text()
    assert "| 8 | 65536 | 8 | 300.0 | 6000.0 | 2.00 |" in text
    assert "python3 bench.py --suites" in text and "openblas" in text and "| 1024 | 2.06 |" in text
