"""The dispatch-table sweep's selection rule (CPU only, no GPU work)."""

import json
import re
import shutil

from scaled_dot_product_03_amd import sweep


def _table_entries(text, cond):
    """The per-bucket entries the generated table holds for one class."""
    m = re.search(re.escape(cond) + r"\) \{\s*constexpr TableEntry e\[kSeqBuckets\] = \{(.*?)\};",
                  text, re.S)
    assert m, cond
    return [tuple(int(x) for x in e.split(",")) for e in re.findall(r"\{([^{}]*)\}", m.group(1))]


def test_write_picks_per_bucket_fastest_candidate_that_passed_parity(tmp_path):
    results = [
        {"dtype": "bf16", "head_dim": 128, "cand": [8, 64, 3], "parity": False, "ms": None},
        # fastest in the long bucket, slower in the short one
        {"dtype": "bf16", "head_dim": 128, "cand": [4, 64, 2], "parity": True,
         "ms": {"5": {"w": [0.2, 0.1]}, "0": {"s": [0.05]}}},
        {"dtype": "bf16", "head_dim": 128, "cand": [2, 32, 2], "parity": True,
         "ms": {"5": {"w": [0.25, 0.1]}, "0": {"s": [0.03]}}},
        # fastest of all but failed parity: never chosen
        {"dtype": "fp16", "head_dim": 64, "cand": [8, 64, 3], "parity": False,
         "ms": {"3": {"w": [0.01]}}},
        {"dtype": "fp16", "head_dim": 64, "cand": [4, 32, 3], "parity": True,
         "ms": {"3": {"w": [0.3]}}},
        {"dtype": "fp16", "head_dim": 64, "cand": [8, 64, 3, 1], "parity": True,
         "ms": {"3": {"w": [0.4]}}},
    ]
    rp = tmp_path / "results.json"
    rp.write_text(json.dumps(results))
    table = tmp_path / "dispatch_table.inc"
    shutil.copy(sweep.TABLE, table)
    pick = sweep.write(str(rp), str(table))
    assert pick[("bf16", 128, 5)] == (4, 64, 2, 0)
    assert pick[("bf16", 128, 0)] == (2, 32, 2, 0)
    assert pick[("fp16", 64, 3)] == (4, 32, 3, 0)
    # buckets without timings keep the class default
    assert pick[("bf16", 128, 2)] == (4, 64, 2, 0) and pick[("fp16", 64, 0)] == (4, 64, 3, 0)
    # untimed classes follow the timed class of the same head_dim, bucket by bucket
    assert pick[("fp16", 128, 0)] == (2, 32, 2, 0) and pick[("bf16", 64, 3)] == (4, 32, 3, 0)
    text = table.read_text()
    assert _table_entries(text, "dtype_code<T>() == DT_BF16 && D == 128") == [
        (2, 32, 2, 0)] + [(4, 64, 2, 0)] * 7
    assert _table_entries(text, "dtype_code<T>() == DT_F16 && D == 64")[3] == (4, 32, 3, 0)
    assert text.count("// BEGIN TABLE (generated)") == 1 and text.count("// END TABLE") == 1


def test_write_emits_the_pingpong_field(tmp_path):
    results = [
        {"dtype": "bf16", "head_dim": 128, "cand": [4, 64, 2, 0], "parity": True,
         "ms": {"5": {"w": [0.3]}}},
        {"dtype": "bf16", "head_dim": 128, "cand": [8, 64, 3, 1], "parity": True,
         "ms": {"5": {"w": [0.2]}}},
    ]
    rp = tmp_path / "results.json"
    rp.write_text(json.dumps(results))
    table = tmp_path / "dispatch_table.inc"
    shutil.copy(sweep.TABLE, table)
    pick = sweep.write(str(rp), str(table))
    assert pick[("bf16", 128, 5)] == (8, 64, 3, 1) and pick[("fp16", 128, 5)] == (8, 64, 3, 1)
    assert _table_entries(table.read_text(), "dtype_code<T>() == DT_BF16 && D == 128")[5] == \
        (8, 64, 3, 1)
    assert sweep._name(("bf16", 128), (8, 64, 3, 1)) == "bf16_d128_w8_n64_s3_pp"


def test_every_bucket_has_timed_workloads_in_its_own_bucket():
    for cls, per_bucket in sweep.TIMED.items():
        assert sorted(per_bucket) == list(range(len(sweep.BUCKETS)))
        for b, specs in per_bucket.items():
            for name, kind, kw in specs:
                if kind == "named":
                    continue
                if kind == "dense":
                    sq, sk = kw["Sq"], kw["Sk"]
                else:  # compact: the longest sequence is at most len_hi
                    sq = sk = kw["len_hi"]
                qb = 0 if sq <= 128 else (1 if sq <= 512 else (2 if sq <= 4096 else 3))
                kb = 0 if sk <= 512 else 1
                assert 2 * qb + kb == b, (cls, b, name)


def test_written_table_compiles_into_the_committed_format():
    text = open(sweep.TABLE).read()
    for cond in ("dtype_code<T>() == DT_BF16 && D == 128", "dtype_code<T>() == DT_F16 && D == 64",
                 "dtype_code<T>() == DT_BF16 && D == 64", "dtype_code<T>() == DT_F16 && D == 128"):
        assert len(_table_entries(text, cond)) == len(sweep.BUCKETS)


def test_schedule_field_names_defines_and_table_entries(tmp_path):
    # schedule 2 (two 32-row blocks per wave) is named, built and written like the others
    assert sweep._name(("bf16", 128), (4, 32, 3, 2)) == "bf16_d128_w4_n32_s3_rb2"
    assert sweep._name(("fp16", 64), (4, 64, 2, 0)) == "fp16_d64_w4_n64_s2"
    assert "-DSDPA03_SWEEP_SCHEDULE=2" in sweep._defines(("bf16", 128), (4, 32, 3, 2))
    assert "-DSDPA03_SWEEP_SCHEDULE=0" in sweep._defines(("fp16", 64), (4, 64, 2))
    results = [
        {"dtype": "bf16", "head_dim": 128, "cand": [4, 32, 3, 2], "parity": True,
         "ms": {"5": {"w": [0.1]}}},
        {"dtype": "bf16", "head_dim": 128, "cand": [4, 64, 2, 0], "parity": True,
         "ms": {"5": {"w": [0.2]}}},
    ]
    rp = tmp_path / "results.json"
    rp.write_text(json.dumps(results))
    table = tmp_path / "dispatch_table.inc"
    shutil.copy(sweep.TABLE, table)
    pick = sweep.write(str(rp), str(table))
    assert pick[("bf16", 128, 5)] == (4, 32, 3, 2)
    assert _table_entries(table.read_text(), "dtype_code<T>() == DT_BF16 && D == 128")[5] == \
        (4, 32, 3, 2)


def test_every_candidate_class_offers_each_schedule():
    for cls, cands in sweep.CANDIDATES.items():
        scheds = {sweep._cand4(c)[3] for c in cands}
        assert scheds == {0, 1, 2}, (cls, scheds)


def test_child_faults_stop_the_sweep_but_failed_comparisons_do_not():
    # pytest's own outcomes: 0 passed, 1 some test failed (a wrong result).
    assert not sweep.child_faulted(0, "12 passed")
    assert not sweep.child_faulted(1, "1 failed, 11 passed")
    # Signals, time limits, other exit codes and fault text end the sweep.
    assert sweep.child_faulted(-11, "")
    assert sweep.child_faulted(-6, "")
    assert sweep.child_faulted(134, "")
    assert sweep.child_faulted(None, "")
    assert sweep.child_faulted(1, "Memory access fault by GPU node-2")
    assert sweep.child_faulted(1, "+++ Timeout +++")
    assert sweep.child_faulted(0, "hipErrorLaunchFailure")
