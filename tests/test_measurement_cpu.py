"""Host-side checks of the measurement tooling (no GPU).

profile_summary.py: the FETCH_SIZE / WRITE_SIZE scaling by the 1 GiB copy,
the busy-interval union of a trace, and the derived counter figures, on small
synthetic CSV files in the rocprofv3 layout.  bench.py: the one-GPU guard, the
gated-figure assembly and the bytes-per-token constants.
"""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


@pytest.fixture
def ps(tmp_path, monkeypatch):
    import profile_summary
    monkeypatch.setattr(profile_summary, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    for f in profile_summary.SOURCES:  # the source hash reads these under ROOT
        os.makedirs(os.path.dirname(tmp_path / f), exist_ok=True)
        (tmp_path / f).write_text("x")
    return profile_summary


def _stats(d, rows):
    _write(str(d / "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"], rows)


def _counters(d, rows):
    _write(str(d / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)


def test_traffic_scaled_by_the_copy(ps, tmp_path):
    t, fch, wrt = tmp_path / "t", tmp_path / "f", tmp_path / "w"
    _stats(t, [["void qmv::(anonymous namespace)::k<1>(int)", 2, 1000, 900, 1100, 50.0]])
    copy = "__amd_rocclr_copyBuffer"
    # the copy moves 1 GiB each way; FETCH_SIZE counts half of it, WRITE_SIZE all of it
    _counters(fch, [[copy, "FETCH_SIZE", 524288], ["k<1>(int)", "FETCH_SIZE", 100], ["k<1>(int)", "FETCH_SIZE", 300]])
    _counters(wrt, [[copy, "WRITE_SIZE", 1048576], ["k<1>(int)", "WRITE_SIZE", 10]])
    ps.main(["traffic", "unit", str(t), str(fch), str(wrt), "cmd a ;; cmd b"])
    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))["unit"]
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    k = rec["kernels"]["k<1>"]
    assert k["fetch_kib"] == 200 and k["bytes"] == (200 * 2.0 + 10) * 1024  # median of 100, 300
    md = open(tmp_path / "profiles" / "unit.md").read()
    assert "cmd a" in md and "cmd b" in md and "x2.0000" in md


def test_busy_union_of_overlapping_dispatches(ps, tmp_path):
    d = tmp_path / "t"
    _write(str(d / "run_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [["matvec_a", 0, 1000], ["matvec_b", 500, 1500], ["matvec_c", 3000, 4000], ["other", 0, 9000]])
    lines = ps.span(str(d), "matvec", 1)
    text = " ".join(lines)
    # durations 1000 + 1000 + 1000; union [0, 1500] + [3000, 4000] = 2500 ns
    assert "sum of durations 3.0 us" in text and "busy intervals 2.5 us" in text and "16.7 %" in text


def test_pmc_derived_figures(ps, tmp_path):
    t, c = tmp_path / "t", tmp_path / "c"
    _stats(t, [["void gemm_k<1>(int)", 4, 10000, 9000, 11000, 90.0]])
    n_mfma = 1000
    _counters(c, [["gemm_k<1>(int)", "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.0e6],
                  ["gemm_k<1>(int)", "SQ_INSTS_MFMA", n_mfma],
                  ["gemm_k<1>(int)", "SQ_INSTS_VALU", 5 * n_mfma],
                  ["gemm_k<1>(int)", "SQ_VALU_MFMA_BUSY_CYCLES", 16 * n_mfma]])
    ps.main(["pmc", "g", "gemm_k", str(t), "cmd", str(c)])
    md = open(tmp_path / "profiles" / "g.md").read()
    # 2e6 MOPS x 512 flops over 10 us = 102.4 TFLOP/s; 4 other VALU per MFMA; 16 busy cycles each
    assert "1.024e+09" in md and "102.4 TFLOP/s" in md and "0.041 of the 2.5 PFLOP/s" in md
    assert "4.00 per MFMA instruction" in md and "busy cycles per MFMA instruction 16.0" in md


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bench_token_constants_and_gated_figures():
    import bench
    import workloads as wl
    cfg = wl.c5_sweep(1)
    packed = sum(int(round(wl.bytes_per_weight(f) * N * K)) for _, f, N, K, _ in cfg["mats"])
    flops = 2 * sum(N * K for _, _, N, K, _ in cfg["mats"])
    assert packed == bench.TOKEN_BYTES_1B1 and flops == bench.TOKEN_FLOPS_1B1
    out = {"value": 800.0, "extras": {
        "decode_sweep_1.1B_b1": {"gbs": 1600.0, "tok_per_s": 2400.0},
        "q4k_vocab_head_151936x1024_b1_cold": {"gbs": 4000.0, "tok_per_s_equiv": 6000.0},
        "gemm_w4a16_M512": {"error": "skipped"}}}
    g = bench.gated_figures(out)
    assert g["c2_w4a16_mlp_stream_b1"]["frac_hbm"] == 0.1
    assert g["c5_decode_token_b1"] == {"gbs": 1600.0, "frac_hbm": 0.2, "tok_per_s": 2400.0}
    assert g["c3_q4k_vocab_head"]["tok_per_s_equiv"] == 6000.0
    assert "c4_w4a16_gemm_M512" not in g  # a leg that failed is left out, not faked


def test_pages_context_names_hardware_and_source():
    import bench
    assert bench.PAGES_CONTEXT
    for e in bench.PAGES_CONTEXT:
        assert e["hardware"] and e["source"] and e["value"] and e["figure"]
        assert "MI355X" not in e["hardware"]  # the pages measured other machines

