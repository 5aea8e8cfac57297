"""Host-side modes of bench.py that turn rocprofv3 output into the profiles'
tables (no GPU): the per-(kernel, grid) trace summary, the counter totals
and the dominant kernel's traffic record, on small hand-written CSVs in the
layout rocprofv3 writes."""
import csv
import json
import os

import bench


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_groups_by_kernel_and_grid(tmp_path):
    p = tmp_path / "trace.csv"
    hdr = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Workgroup_Size_X",
           "Workgroup_Size_Y", "Workgroup_Size_Z", "Start_Timestamp", "End_Timestamp"]
    rows = [
        ["void dinfer::(anonymous namespace)::swiglu_kernel<8>(int const*, int)", 64, 1, 1, 256, 1, 1, 0, 5000],
        ["void dinfer::(anonymous namespace)::swiglu_kernel<8>(int const*, int)", 64, 1, 1, 256, 1, 1, 10000, 13000],
        ["void dinfer::(anonymous namespace)::swiglu_kernel<8>(int const*, int)", 4096, 1, 1, 256, 1, 1, 20000, 120000],
        ["gemm_kernel(float const*)", 512, 4, 2, 512, 1, 1, 200000, 202000],
    ]
    _write(p, hdr, rows)
    text = bench.trace_summary(str(p))
    lines = [l for l in text.splitlines() if l.startswith("| `")]
    # three groups, largest total first; the anonymous namespace and "void " are dropped
    assert len(lines) == 3
    assert lines[0].startswith("| `dinfer::swiglu_kernel<8>` | 4096x1x1 | 256x1x1 | 1 | 0.10 | 100.00 |")
    assert "| `dinfer::swiglu_kernel<8>` | 64x1x1 | 256x1x1 | 2 | 0.01 | 4.00 |" in text
    assert "| `gemm_kernel` | 512x4x2 | 512x1x1 | 1 | 0.00 | 2.00 |" in text
    assert "over 4 dispatches" in text


def test_counter_totals_and_traffic_record(tmp_path):
    def counters(path, name, counter, vals):
        _write(path, ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [[name, counter, v] for v in vals])
    kf, kw = tmp_path / "kf.csv", tmp_path / "kw.csv"
    cf, cw = tmp_path / "cf.csv", tmp_path / "cw.csv"
    counters(kf, "dinfer::gemm_skinny_kernel<...>", "FETCH_SIZE", [100.0, 300.0])
    counters(kw, "dinfer::gemm_skinny_kernel<...>", "WRITE_SIZE", [10.0, 30.0])
    # a 1 GiB copy whose FETCH_SIZE reads half its size and WRITE_SIZE all of it
    counters(cf, "__amd_rocclr_copyBuffer", "FETCH_SIZE", [(1 << 30) / 1024 / 2])
    counters(cw, "__amd_rocclr_copyBuffer", "WRITE_SIZE", [(1 << 30) / 1024])
    tot = bench.counter_totals([str(kf), str(kw)])
    assert tot == {"FETCH_SIZE": {"sum": 400.0, "dispatches": 2},
                   "WRITE_SIZE": {"sum": 40.0, "dispatches": 2}}
    rec = bench.traffic_record(str(kf), str(kw), str(cf), str(cw), ["cmd"])
    assert rec["dispatches"] == 2
    assert rec["calibration"]["fetch_factor"] == 2.0
    assert rec["calibration"]["write_factor"] == 1.0
    # mean 200 KiB fetched x 2 + mean 20 KiB written x 1
    assert rec["bytes_per_launch"] == (200 * 2 + 20) * 1024
    assert rec["source_hash"] == bench.source_hash()
    json.dumps(rec)   # serialisable as written to profiles/


def test_committed_traffic_record_matches_the_sources():
    """The record bench.py reports as `traffic` is keyed on the current kernel
    sources (a changed kernel reports null until its counters are retaken)."""
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert rec["source_hash"] == bench.source_hash()
    assert rec["bytes_per_launch"] > 0
    assert os.path.basename(bench.TRAFFIC_FILE) == "gemm_skinny_qkv_gateup_dense8b_traffic.json"


def test_committed_bench_line_keeps_the_output_contract():
    """The kept bench line carries every field of the one-line contract, its
    roofline fraction is achieved / peak, and its CPU baseline is the
    oracle's."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "..", "profiles", "dense8b_b1_bench_line.json")
    line = json.load(open(path))
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in line, k
    assert line["n_gpus"] == 1 and line["higher_is_better"] is True
    assert line["config"]["workload"] == "dense8b_b1"
    r = line["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and r["unit"] in ("GB/s", "TFLOP/s")
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    c = line["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    r = subprocess.run([sys.executable, os.path.join(here, "..", "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr + r.stdout
