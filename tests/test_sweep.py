"""The dispatch-table sweep's selection rule (CPU only, no GPU work)."""

import json
import shutil

from scaled_dot_product_03_amd import sweep


def test_write_picks_fastest_candidate_that_passed_parity(tmp_path):
    results = [
        {"dtype": "bf16", "head_dim": 128, "cand": [8, 64, 3], "parity": False, "ms": None},
        {"dtype": "bf16", "head_dim": 128, "cand": [4, 64, 2], "parity": True,
         "ms": {"w": [0.2, 0.1]}},
        {"dtype": "bf16", "head_dim": 128, "cand": [8, 64, 2], "parity": True,
         "ms": {"w": [0.25, 0.1]}},
        # fastest of all but failed parity: never chosen
        {"dtype": "fp16", "head_dim": 64, "cand": [8, 64, 3], "parity": False,
         "ms": {"w": [0.01]}},
        {"dtype": "fp16", "head_dim": 64, "cand": [4, 32, 3], "parity": True, "ms": {"w": [0.3]}},
        {"dtype": "fp16", "head_dim": 64, "cand": [8, 64, 3, 1], "parity": True, "ms": {"w": [0.4]}},
    ]
    rp = tmp_path / "results.json"
    rp.write_text(json.dumps(results))
    table = tmp_path / "dispatch_table.inc"
    shutil.copy(sweep.TABLE, table)
    pick = sweep.write(str(rp), str(table))
    assert pick[("bf16", 128)] == (4, 64, 2, 0)
    assert pick[("fp16", 64)] == (4, 32, 3, 0)
    # untimed classes follow the timed class of the same head_dim
    assert pick[("fp16", 128)] == (4, 64, 2, 0) and pick[("bf16", 64)] == (4, 32, 3, 0)
    text = table.read_text()
    assert "dtype_code<T>() == DT_F16 && D == 64) {\n    return TableEntry{4, 32, 3, 0};" in text
    assert text.count("// BEGIN TABLE (generated)") == 1 and text.count("// END TABLE") == 1


def test_write_emits_the_pingpong_field(tmp_path):
    results = [
        {"dtype": "bf16", "head_dim": 128, "cand": [4, 64, 2, 0], "parity": True,
         "ms": {"w": [0.3]}},
        {"dtype": "bf16", "head_dim": 128, "cand": [8, 64, 3, 1], "parity": True,
         "ms": {"w": [0.2]}},
    ]
    rp = tmp_path / "results.json"
    rp.write_text(json.dumps(results))
    table = tmp_path / "dispatch_table.inc"
    shutil.copy(sweep.TABLE, table)
    pick = sweep.write(str(rp), str(table))
    assert pick[("bf16", 128)] == (8, 64, 3, 1) and pick[("fp16", 128)] == (8, 64, 3, 1)
    assert "dtype_code<T>() == DT_BF16 && D == 128) {\n    return TableEntry{8, 64, 3, 1};" in \
        table.read_text()
    assert sweep._name(("bf16", 128), (8, 64, 3, 1)) == "bf16_d128_w8_n64_s3_pp"
