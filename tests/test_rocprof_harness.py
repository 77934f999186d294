"""Host logic of the rocprofv3 harness: kernel-name parsing, algorithmic
bytes, CSV parsing, the copy calibration and the traffic summary that
bench.py reads back.  The CSV files are small synthetic ones in the column
layout rocprofv3 writes; no profiler or GPU runs here."""

import csv
import os

import pytest

from scaled_dot_product_03_amd import rocprof

MANGLED_NC = ("_ZN6sdpa0315attn_fwd_kernelIDF16bLi128ELi4ELi1ELi64ELi2ELi0ELb0ELb0ELb0EE"
              "EvNS_7FwdArgsE")
MANGLED_C_BIAS = ("_ZN6sdpa0315attn_fwd_kernelIDF16bLi128ELi4ELi1ELi64ELi2ELi0ELb1ELb0ELb1EE"
                  "EvNS_7FwdArgsE")
DEMANGLED_NC = ("void sdpa03::attn_fwd_kernel<__bf16, 128, 4, 1, 64, 2, 0, false, false, false>"
                "(sdpa03::FwdArgs)")
COPY = "__amd_rocclr_copyBuffer"


def test_short_names_agree_across_manglings():
    want = "attn_fwd_kernel<bf16, 128, 4, 1, 64, 2, 0, false, false, false>"
    assert rocprof.short_name(MANGLED_NC) == want
    assert rocprof.short_name(DEMANGLED_NC) == want
    assert rocprof.short_name("attn_fwd_kernel<DF16bLi128ELi4ELi1ELi64ELi2ELi0ELb0ELb0ELb0>") == want
    assert rocprof.short_name(COPY) == COPY
    assert rocprof.short_name("_ZN6sdpa0321attn_fwd_merge_kernelIDF16_Li64EEEvNS_9MergeArgsE") == \
        "attn_fwd_merge_kernel<fp16, 64>"


def test_dominant_kernel_is_dense_bf16_d128_without_mask_split_or_bias():
    assert rocprof.is_dominant(rocprof.short_name(MANGLED_NC))
    assert not rocprof.is_dominant(rocprof.short_name(MANGLED_C_BIAS))
    assert not rocprof.is_dominant("attn_fwd_kernel<fp16, 64, 4, 1, 64, 2, 0, false, false, false>")
    assert not rocprof.is_dominant("attn_fwd_kernel<bf16, 128, 4, 1, 64, 2, 1, false, false, false>")


def test_algorithmic_bytes_closed_forms():
    B, H, S, D = 4, 16, 2048, 128
    qkvo = 4 * B * H * S * D * 2 + B * H * S * 4
    assert rocprof.algorithmic_bytes(rocprof.short_name(MANGLED_NC)) == qkvo
    # Non-causal bias: every (row, key) entry once.
    nc_bias = "attn_fwd_kernel<bf16, 128, 4, 1, 64, 2, 0, false, false, true>"
    assert rocprof.algorithmic_bytes(nc_bias) == qkvo + B * H * S * S * 2
    # Causal bias with 128-row query tiles: tile m loads 128 (m + 1) keys for
    # its 128 rows, i.e. 128^2 * (1 + ... + 16) entries per (batch, head).
    c_bias = rocprof.algorithmic_bytes(rocprof.short_name(MANGLED_C_BIAS))
    assert c_bias == qkvo + B * H * 128 * 128 * (16 * 17 // 2) * 2
    # A split launch needs the split count for its workspace bytes.
    assert rocprof.algorithmic_bytes("attn_fwd_kernel<fp16, 64, 4, 1, 64, 2, 0, false, true, "
                                     "false>") is None
    # Kernels of no bench workload.
    assert rocprof.kernel_accounting("attn_fwd_kernel<fp32, 64, 4, 1, 32, 2, 0, false, false, "
                                     "false>") is None
    assert rocprof.kernel_accounting("__amd_rocclr_copyBuffer") is None


def test_accounting_of_every_bench_kernel():
    # fp16 Sq 512 Sk 8192 D 64, B 2 H 32: unsplit, split in two, merge.
    rq, rk, d = 2 * 32 * 512, 2 * 32 * 8192, 64
    plain = rocprof.kernel_accounting("attn_fwd_kernel<fp16, 64, 4, 1, 64, 2, 0, false, false, "
                                      "false>")
    assert plain["workload"] == "dense_fp16_b2h32sq512sk8192d64"
    assert plain["bytes"] == rq * (2 * d * 2 + 4) + rk * 2 * d * 2
    assert plain["flops"] == 4.0 * 512 * 8192 * 64 * 32 * 2
    split = rocprof.kernel_accounting("attn_fwd_kernel<fp16, 64, 4, 1, 64, 2, 0, false, true, "
                                      "false>", splits=2)
    assert split["bytes"] == rq * d * 2 + rk * 2 * d * 2 + 2 * rq * (d + 1) * 4
    assert split["flops"] == plain["flops"]
    kg = rocprof.kernel_accounting("attn_fwd_kg_kernel<fp16, 64, 2, 64, 2, 0>")
    assert kg["workload"] == plain["workload"]
    assert kg["bytes"] == plain["bytes"] and kg["flops"] == plain["flops"]
    merge = rocprof.kernel_accounting("attn_fwd_merge_kernel<fp16, 64>", splits=2)
    assert merge["bytes"] == 2 * rq * (d + 1) * 4 + rq * (d * 2 + 4)
    assert merge["flops"] is None
    # THD: 16 sequences of seed 4 (T = 40,702 tokens), H 16, causal.
    thd = rocprof.kernel_accounting("attn_fwd_kernel<bf16, 128, 4, 1, 64, 2, 1, true, false, "
                                    "false>")
    assert thd["bytes"] == 16 * 40702 * (4 * 128 * 2 + 4)
    assert thd["flops"] == pytest.approx(5.116e11, rel=1e-3)
    # Padded: true lengths of seed 5 only (sum 42,230 rows), H 32, causal.
    pad = rocprof.kernel_accounting("attn_fwd_kernel<bf16, 128, 8, 1, 64, 2, 2, true, false, "
                                    "false>")
    assert pad["bytes"] == 32 * 42230 * (4 * 128 * 2 + 4)
    assert pad["flops"] == pytest.approx(1.982e12, rel=1e-3)
    # Backward on the dense bf16 S2048 workload.
    B, H, S, D = 4, 16, 2048, 128
    r = B * H * S
    dq = rocprof.kernel_accounting("attn_bwd_dq_kernel<bf16, 128, 0, false>")
    # Q, O, dO and K, V (bf16), the LSE read; dQ and the two row values written.
    assert dq["bytes"] == r * (4 * D * 2 + 4) + r * 2 * D * 2 + r * 8
    assert dq["flops"] == 3 * 2.0 * S * S * D * B * H
    dkdv = rocprof.kernel_accounting("attn_bwd_dkdv_kernel<bf16, 128, 0, true>")
    assert dkdv["bytes"] == r * 2 * D * 2 + r * 8 + r * 4 * D * 2
    assert dkdv["flops"] == 4 * 2.0 * S * S * D * B * H / 2


def test_derived_counter_metrics():
    c = {"SQ_VALU_MFMA_BUSY_CYCLES": 512.0, "SQ_ACTIVE_INST_VALU": 128.0,
         "SQ_LDS_IDX_ACTIVE": 64.0, "GRBM_GUI_ACTIVE": 8.0, "_duration_ns": 0.5}
    assert rocprof.mfma_busy_pct(c) == pytest.approx(50.0)   # 512 / (1 x 1024)
    assert rocprof.valu_busy_pct(c) == pytest.approx(50.0)   # 128 / 256 / 1
    assert rocprof.lds_util_pct(c) == pytest.approx(25.0)    # 64 / (1 x 256)
    assert rocprof.clock_ghz(c) == pytest.approx(2.0)        # 1 cycle per 0.5 ns
    assert rocprof.clock_ghz({"GRBM_GUI_ACTIVE": 8.0}) is None


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


COUNTER_HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id",
                  "Thread_Id", "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size",
                  "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
                  "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"]


def _counter_rows(entries):
    """entries: (dispatch, kernel, counter, value)."""
    return [[d, d, 1, 0, 7, 7, 1024, 3, k, 256, 0, 0, 128, 64, 40, c, v, 0, 1]
            for d, k, c, v in entries]


def test_counter_parsing_sums_rows_of_a_dispatch_then_averages(tmp_path):
    d = tmp_path / "sq"
    _write_csv(str(d / "host" / "sq_counter_collection.csv"), COUNTER_HEADER, _counter_rows([
        (1, MANGLED_NC, "SQ_VALU_MFMA_BUSY_CYCLES", 300.0),
        (1, MANGLED_NC, "SQ_VALU_MFMA_BUSY_CYCLES", 100.0),  # a second row of dispatch 1
        (1, MANGLED_NC, "GRBM_GUI_ACTIVE", 8.0),
        (2, MANGLED_NC, "SQ_VALU_MFMA_BUSY_CYCLES", 600.0),
        (2, MANGLED_NC, "GRBM_GUI_ACTIVE", 8.0),
    ]))
    c = rocprof.parse_counters(str(d))
    k = rocprof.short_name(MANGLED_NC)
    assert c[k]["SQ_VALU_MFMA_BUSY_CYCLES"] == pytest.approx(500.0)
    assert c[k]["GRBM_GUI_ACTIVE"] == pytest.approx(8.0)
    # 500 busy cycles summed over 1024 SIMDs against 8 / 8 = 1 cycle each.
    assert rocprof.mfma_busy_pct(c[k]) == pytest.approx(100 * 500 / 1024)


def test_counter_parsing_takes_dispatch_durations_from_the_same_run(tmp_path):
    d = tmp_path / "sq"
    _write_csv(str(d / "host" / "sq_counter_collection.csv"), COUNTER_HEADER, _counter_rows([
        (1, MANGLED_NC, "GRBM_GUI_ACTIVE", 8.0e5),
        (2, MANGLED_NC, "GRBM_GUI_ACTIVE", 8.0e5),
    ]))
    _write_csv(str(d / "host" / "sq_kernel_trace.csv"),
               ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               [[1, MANGLED_NC, 1000, 51000], [2, MANGLED_NC, 90000, 140000],
                [3, COPY, 0, 10]])
    c = rocprof.parse_counters(str(d))[rocprof.short_name(MANGLED_NC)]
    assert c["_duration_ns"] == pytest.approx(50000.0)
    assert rocprof.clock_ghz(c) == pytest.approx(2.0)  # 1e5 cycles per XCD in 50 us


def test_stats_parsing(tmp_path):
    d = tmp_path / "trace"
    _write_csv(str(d / "host" / "trace_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                "StdDev"],
               [[MANGLED_NC, 10, 1300000, 130000.0, 60.0, 127000, 166000, 1000.0],
                [COPY, 1, 4700, 4700.0, 0.1, 4700, 4700, 0.0]])
    s = rocprof.parse_stats(str(d))
    assert s[rocprof.short_name(MANGLED_NC)] == pytest.approx((10, 130.0, 127.0, 166.0, 60.0))
    assert s[COPY][1] == pytest.approx(4.7)


def test_traffic_summary_round_trips_into_bench(tmp_path, monkeypatch):
    k = rocprof.short_name(MANGLED_NC)
    n_kib = rocprof.COPY_MIB * 1024
    # The copy reads half its bytes on FETCH_SIZE: fetch readings double.
    fetch = {COPY: {"FETCH_SIZE": n_kib / 2}, k: {"FETCH_SIZE": 50000.0}}
    write = {COPY: {"WRITE_SIZE": float(n_kib)}, k: {"WRITE_SIZE": 33000.0}}
    stats = {k: (10, 130.0, 127.0, 166.0, 60.0)}
    assert rocprof.copy_factors(fetch, write)[:2] == pytest.approx((2.0, 1.0))
    path = tmp_path / rocprof.TRAFFIC_FILE
    rocprof.write_traffic(fetch, write, stats, ["rocprofv3 --pmc FETCH_SIZE -- python3 bench.py"],
                          str(path))
    want = (2 * 50000.0 + 33000.0) * 1024
    assert rocprof.traffic_from_profiles(profiles_dir=str(tmp_path)) == pytest.approx(want, rel=1e-6)
    text = path.read_text()
    assert f"{want / 130e-6 / 1e9:.0f}" in text  # achieved GB/s from the trace's average
    # A summary taken on other kernel sources is not reported.
    path.write_text(text.replace(rocprof.kernel_source_hash(), "0" * 16))
    assert rocprof.traffic_from_profiles(profiles_dir=str(tmp_path)) is None


def test_calibration_uses_the_largest_copy_dispatch(tmp_path):
    # Small uploads share the copy kernel's name; their dispatches must not
    # dilute the calibration copy's reading.
    n_kib = rocprof.COPY_MIB * 1024
    d = tmp_path / "fetch"
    _write_csv(str(d / "host" / "fetch_counter_collection.csv"), COUNTER_HEADER, _counter_rows([
        (1, COPY, "FETCH_SIZE", 0.1), (2, COPY, "FETCH_SIZE", n_kib / 2),
        (3, COPY, "FETCH_SIZE", 0.1), (4, COPY, "FETCH_SIZE", n_kib / 2),
    ]))
    fetch = rocprof.parse_counters(str(d))
    write = {COPY: {"WRITE_SIZE": 1.0, "WRITE_SIZE#max": float(n_kib)}}
    assert rocprof.copy_factors(fetch, write)[:2] == pytest.approx((2.0, 1.0))


def test_missing_calibration_copy_is_an_error():
    with pytest.raises(RuntimeError):
        rocprof.copy_factors({"x": {"FETCH_SIZE": 1.0}}, {"x": {"WRITE_SIZE": 1.0}})


def test_committed_traffic_summary_parses():
    # bench.py's roofline.traffic comes from this file; it must stay readable
    # (it is None only when the kernel sources changed since it was taken).
    path = os.path.join(rocprof.ROOT, "profiles", rocprof.TRAFFIC_FILE)
    text = open(path).read()
    assert "kernel_source_sha:" in text and "hbm_bytes_per_launch:" in text


def test_command_line_defaults_to_every_pass():
    assert rocprof.parse_args([]).passes == ["trace", "counters", "traffic"]
    assert rocprof.parse_args(["traffic"]).passes == ["traffic"]
    with pytest.raises(SystemExit):
        rocprof.parse_args(["nonsense"])
