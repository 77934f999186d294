"""The dispatch-table sweep's selection rule, table writer and workload plan
(CPU only, no GPU work)."""

import json
import re
import shutil

import numpy as np

from scaled_dot_product_03_amd import sweep


def _table_entries(text, cond):
    """The [bucket][variant] entries the generated table holds for one class."""
    m = re.search(re.escape(cond) + r"\) \{\s*constexpr TableEntry e\[kSeqBuckets\]\[kVariants\] "
                  r"= \{(.*?)\};", text, re.S)
    assert m, cond
    rows = re.findall(r"\{(\{[^{}]*\}(?:, \{[^{}]*\})*)\}", m.group(1))
    return [[tuple(int(x) for x in e.split(",")) for e in re.findall(r"\{([^{}]*)\}", r)]
            for r in rows]


def _ms(per_bucket):
    """{bucket: {workload: {variant: ms}}} with string keys, as results.json has."""
    return {str(b): {w: {str(v): t for v, t in per.items()} for w, per in wl.items()}
            for b, wl in per_bucket.items()}


def _write(tmp_path, results):
    rp = tmp_path / "results.json"
    rp.write_text(json.dumps(results))
    table = tmp_path / "dispatch_table.inc"
    shutil.copy(sweep.TABLE, table)
    summary = tmp_path / "summary.md"
    pick = sweep.write(str(rp), str(table), str(summary))
    return pick, table.read_text(), summary.read_text()


def test_write_picks_per_bucket_and_variant_among_candidates_that_passed_parity(tmp_path):
    results = [
        # fastest everywhere but failed parity: never chosen
        {"dtype": "bf16", "head_dim": 128, "cand": [8, 64, 3, 0], "parity": False, "ms": None},
        # best on the dense non-causal calls of bucket 5, worse causal
        {"dtype": "bf16", "head_dim": 128, "cand": [4, 64, 2, 0], "parity": True,
         "ms": _ms({5: {"a": {0: 0.10, 1: 0.09}, "b": {0: 0.20, 1: 0.12}, "t": {3: 0.5}}})},
        {"dtype": "bf16", "head_dim": 128, "cand": [4, 32, 2, 4], "parity": True,
         "ms": _ms({5: {"a": {0: 0.12, 1: 0.07}, "b": {0: 0.22, 1: 0.10}, "t": {3: 0.4}}})},
        {"dtype": "fp16", "head_dim": 64, "cand": [4, 32, 3, 3], "parity": True,
         "ms": _ms({3: {"c": {0: 0.3}}})},
        {"dtype": "fp16", "head_dim": 64, "cand": [4, 64, 2, 0], "parity": True,
         "ms": _ms({3: {"c": {0: 0.2}}})},
    ]
    pick, text, summary = _write(tmp_path, results)
    assert pick[("bf16", 128, 5, 0)] == (4, 64, 2, 0)
    assert pick[("bf16", 128, 5, 1)] == (4, 32, 2, 4)
    assert pick[("bf16", 128, 5, 3)] == (4, 32, 2, 4)
    # variable-length without the mask has no timing here: dense without the mask
    assert pick[("bf16", 128, 5, 2)] == (4, 64, 2, 0)
    assert pick[("fp16", 64, 3, 0)] == (4, 64, 2, 0)
    # keys no timing reaches (other buckets, untimed classes) keep the default
    assert pick[("bf16", 128, 0, 0)] == sweep.DEFAULT
    assert pick[("fp32", 64, 5, 1)] == sweep.DEFAULT
    ent = _table_entries(text, "dtype_code<T>() == DT_BF16 && D == 128")
    assert len(ent) == len(sweep.BUCKETS) and all(len(r) == len(sweep.VARIANTS) for r in ent)
    assert ent[5] == [(4, 64, 2, 0), (4, 32, 2, 4), (4, 64, 2, 0), (4, 32, 2, 4)]
    assert text.count("// BEGIN TABLE (generated)") == 1 and text.count("// END TABLE") == 1
    # braces balance: one opened per class, one for the default, all closed
    body = text[text.index("// BEGIN TABLE"):text.index("// END TABLE")]
    assert not re.search(r"^\s*\}\}", body, re.M)
    assert body.count("{") == body.count("}")
    # the summary traces each entry to its timings
    assert "| 5 | dense causal | (4, 32, 2, 4) | own timings |" in summary
    assert "| 5 | varlen | (4, 64, 2, 0) | variant dense |" in summary
    assert "FAIL" in summary


def test_scores_count_every_call_alike():
    # one long and one short call: 10% slower on the long one and 20% faster
    # on the short one wins (1.1 + 1.0 < 1.0 + 1.25)
    results = [
        {"dtype": "bf16", "head_dim": 128, "cand": [4, 64, 2, 0], "parity": True,
         "ms": _ms({7: {"long": {0: 2.0}, "short": {0: 0.0125}}})},
        {"dtype": "bf16", "head_dim": 128, "cand": [8, 64, 2, 0], "parity": True,
         "ms": _ms({7: {"long": {0: 2.2}, "short": {0: 0.0100}}})},
    ]
    pick, best = sweep.select(results)
    assert pick[("bf16", 128, 7, 0)][0] == (8, 64, 2, 0)
    assert abs(best[("bf16", 128, 7, 0)][1] - 2.1) < 1e-9


def test_a_candidate_missing_a_call_of_a_key_does_not_compete_for_it():
    # a candidate timed without the mask only wins the unmasked key and is
    # absent from the causal one, though its (missing) causal calls would
    # otherwise make its score look small
    results = [
        {"dtype": "fp16", "head_dim": 64, "cand": [4, 64, 2, 0], "parity": True,
         "ms": _ms({3: {"a": {0: 0.10, 1: 0.05}, "b": {0: 0.20, 1: 0.08}}})},
        {"dtype": "fp16", "head_dim": 64, "cand": [8, 64, 2, 5], "parity": True,
         "ms": _ms({3: {"a": {0: 0.09}, "b": {0: 0.18}}})},
        {"dtype": "fp16", "head_dim": 64, "cand": [4, 32, 2, 0], "parity": True,
         "ms": _ms({3: {"a": {0: 0.12, 1: 0.06}, "b": {1: 0.09}}})},
    ]
    pick, best = sweep.select(results)
    assert pick[("fp16", 64, 3, 0)][0] == (8, 64, 2, 5)
    assert pick[("fp16", 64, 3, 1)][0] == (4, 64, 2, 0)
    assert best[("fp16", 64, 3, 0)][2] == 2
    # (4, 32, 2, 0) lacks workload b's unmasked call: not a runner-up there
    assert best[("fp16", 64, 3, 0)][3][2] == (4, 64, 2, 0)


def test_names_and_defines_of_every_schedule():
    assert sweep._name(("bf16", 128), (4, 32, 3, 2)) == "bf16_d128_w4_n32_s3_rb2"
    assert sweep._name(("bf16", 128), (8, 64, 3, 1)) == "bf16_d128_w8_n64_s3_pp"
    assert sweep._name(("fp16", 64), (4, 32, 3, 3)) == "fp16_d64_w4_n32_s3_lag"
    assert sweep._name(("fp16", 64), (4, 64, 2, 4)) == "fp16_d64_w4_n64_s2_3w"
    assert sweep._name(("fp32", 64), (4, 64, 2)) == "fp32_d64_w4_n64_s2"
    assert "-DSDPA03_SWEEP_SCHEDULE=3" in sweep._defines(("fp16", 64), (4, 32, 3, 3))
    assert "-DSDPA03_SWEEP_DTYPE=0" in sweep._defines(("fp32", 128), (4, 32, 2, 0))
    assert sweep._kernel_prefix(("fp16", 64), (4, 32, 3, 3)).startswith("attn_fwd_lagged_kernel")
    assert sweep._kernel_prefix(("bf16", 128), (4, 32, 2, 4)).startswith("attn_fwd_3w_kernel")


def test_every_class_is_swept_with_several_schedules():
    assert set(sweep.CANDIDATES) == set(sweep.CLASSES)
    for cls, cands in sweep.CANDIDATES.items():
        scheds = {sweep._cand4(c)[3] for c in cands}
        assert len(cands) >= 4, cls
        if cls[0] != "fp32":
            assert {0, 1, 4} <= scheds, (cls, scheds)
        else:  # the ping-pong and lagged schedules are 16-bit only
            assert scheds == {0}


def _lengths(kind, kw):
    if kind == "dense":
        return kw["Sq"], kw["Sk"]
    rng = np.random.default_rng(kw["seed"])
    if kw["k_lo"] is None:
        lq = rng.integers(kw["len_lo"], kw["len_hi"], size=kw["n_seqs"], endpoint=True)
        return int(lq.max()), int(lq.max())
    rng = np.random.default_rng(kw["seed"] + 1)
    lq = rng.integers(kw["len_lo"], kw["len_hi"], size=kw["n_seqs"], endpoint=True)
    lk = rng.integers(kw["k_lo"], kw["k_hi"], size=kw["n_seqs"], endpoint=True)
    return int(lq.max()), int(lk.max())


def test_every_bucket_has_two_dense_and_a_varlen_workload_in_its_own_bucket():
    for cls, per_bucket in sweep.TIMED.items():
        assert sorted(per_bucket) == list(range(len(sweep.BUCKETS)))
        for b, specs in per_bucket.items():
            kinds = [kind for _, kind, _ in specs]
            assert kinds.count("dense") >= 2 and "compact" in kinds, (cls, b)
            for name, kind, kw in specs:
                if kind == "named":
                    continue
                sq, sk = _lengths(kind, kw)
                qb = 0 if sq <= 128 else (1 if sq <= 512 else (2 if sq <= 4096 else 3))
                kb = 0 if sk <= 512 else 1
                assert 2 * qb + kb == b, (cls, b, name, sq, sk)


def test_committed_table_holds_every_class_bucket_and_variant():
    text = open(sweep.TABLE).read()
    for dt, d in sweep.CLASSES:
        ent = _table_entries(text, sweep._cond(dt, d))
        assert len(ent) == len(sweep.BUCKETS), (dt, d)
        assert all(len(r) == len(sweep.VARIANTS) for r in ent), (dt, d)


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
