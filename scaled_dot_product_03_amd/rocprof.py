"""rocprofv3 harness: kernel times, matrix-core, VALU and LDS use, HBM traffic.

    python -m scaled_dot_product_03_amd.rocprof [trace] [counters] [traffic]
        [--out rocprof_out] [--profiles profiles] [--steps 20]

Runs ``bench.py`` under rocprofv3 as child processes (this process never
touches the GPU) and writes short markdown summaries into ``profiles/``,
one row per kernel of the bench run (every forward, split, merge and
backward kernel on the bench line), each tied to the workload it ran on:

* ``trace``: ``--kernel-trace --stats`` over a normal bench run; per kernel
  the call count and the average, min and max duration.
* ``counters``: one ``--pmc`` pass (with ``--kernel-trace`` for per-dispatch
  durations) over every bench workload: matrix-core busy % =
  SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs), VALU
  busy % and LDS use % by the profiler's own derived-metric formulas,
  v_exp_f32 wave-instructions, LDS wait and bank-conflict cycles, and the
  shader clock each kernel ran at (GRBM_GUI_ACTIVE per XCD over the
  dispatch's duration).
* ``traffic``: one ``--pmc FETCH_SIZE`` and one ``--pmc WRITE_SIZE`` pass over
  the same workloads plus a plain device copy of known size, whose readings
  give the factor that turns each counter into bytes.  Bytes per launch
  against each kernel's algorithmic bytes and, with the trace's average
  durations, achieved HBM GB/s against 8 TB/s.

Counter passes stay within one pass's hardware limits (at most 8 SQ, 4 TCC
and 2 GRBM counters) and are never combined with API tracing.  Every
rocprofv3 run is bounded by ``timeout -s KILL``.  The summaries carry the
hash of the kernel sources; ``bench.py`` reports figures from them only
while that hash matches the sources it runs.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import subprocess
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ["scaled_dot_product_03_amd/csrc/attn_fwd.hip",
                  "scaled_dot_product_03_amd/csrc/attn_fwd_bf16.hip",
                  "scaled_dot_product_03_amd/csrc/attn_fwd_f16.hip",
                  "scaled_dot_product_03_amd/csrc/attn_fwd_kernels.h",
                  "scaled_dot_product_03_amd/csrc/attn_bwd.hip",
                  "scaled_dot_product_03_amd/csrc/attn_common.h",
                  "scaled_dot_product_03_amd/csrc/dispatch_table.inc"]
TRAFFIC_FILE = "hbm_traffic_attn_kernels_bench_workloads.md"
COUNTERS_FILE = "counters_attn_kernels_bench_workloads.md"
TRACE_FILE = "kernel_trace_attn_kernels_bench_workloads.md"
HBM_PEAK_GBS = 8000.0
XCDS = 8
CUS = 256
SIMDS = 1024  # 256 CUs x 4 SIMDs
COPY_MIB = 256

SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU_TRANS_F32",
               "SQ_WAIT_INST_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
               "SQ_ACTIVE_INST_LDS", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
# Profiled runs skip the cpu baseline and the untimed settle phases (the
# profiler serialises dispatches; steady clocks are the trace pass's job).
PROFILED = ["--no-cpu-baseline", "--settle-s", "0", "--launch-stats", "0"]
TEMPLATE_NOTE = ("Forward template arguments: <element type, head_dim, waves, row blocks per wave, "
                 "block_n, stages, mode (0 dense, 1 compact, 2 padded), causal, split, bias> "
                 "(attn_fwd_3w_kernel and attn_fwd_lagged_kernel: the same without row blocks; "
                 "attn_fwd_kg_kernel: <element type, head_dim, key groups, block_n, stages, "
                 "mode>); "
                 "merge: <element type, head_dim>; backward: <element type, head_dim, mode[, "
                 "causal]>.")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _summary_value(fname: str, key: str, profiles_dir: str | None):
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"), fname)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha:\s*(\w+)", text)
    val = re.search(key + r":\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def traffic_from_profiles(profiles_dir: str | None = None):
    """HBM bytes per launch of the dominant kernel from the committed traffic
    summary, if it was taken on the current kernel sources; else None."""
    return _summary_value(TRAFFIC_FILE, "hbm_bytes_per_launch", profiles_dir)


def clock_from_profiles(profiles_dir: str | None = None):
    """Shader clock (GHz) the dominant kernel ran at in the committed counter
    pass, if taken on the current kernel sources; else None."""
    return _summary_value(COUNTERS_FILE, "dominant_kernel_shader_clock_ghz", profiles_dir)


# --- kernel names --------------------------------------------------------

_TYPES = {"DF16b": "bf16", "DF16_": "fp16", "f": "fp32", "__bf16": "bf16", "_Float16": "fp16",
          "float": "fp32", "__hip_bfloat16": "bf16", "__half": "fp16"}


def _mangled_args(text: str):
    """Template arguments from their Itanium mangling: a leading element
    type, then integer and bool literals (DF16bLi128ELb0E...)."""
    m = re.match(r"(DF16b|DF16_|f)?((?:L[ib]n?\d+E?)*)", text)
    args = [_TYPES[m.group(1)]] if m.group(1) else []
    for kind, val in re.findall(r"L([ib])(n?\d+)E?", m.group(2)):
        val = val.replace("n", "-")
        args.append(("true" if val == "1" else "false") if kind == "b" else val)
    return args


def short_name(name: str) -> str:
    """'ident<arg, ...>' for a mangled or demangled template kernel name;
    other names are returned without namespace and argument list."""
    name = name.strip()
    if name.startswith("_Z"):
        pos = 3 if name.startswith("_ZN") else 2
        ident = None
        while pos < len(name) and name[pos].isdigit():
            n = re.match(r"\d+", name[pos:]).group(0)
            pos += len(n)
            ident = name[pos:pos + int(n)]
            pos += int(n)
        if ident is None:
            return name
        if pos < len(name) and name[pos] == "I":
            return f"{ident}<{', '.join(_mangled_args(name[pos + 1:]))}>"
        return ident
    m = re.search(r"(\w+)<([^<>]*)>", name)
    if m:
        inner = m.group(2).strip()
        if "," not in inner and re.fullmatch(r"(DF16b|DF16_|f)?(L[ib]n?\d+E?)*", inner):
            args = _mangled_args(inner)
        else:
            args = [_TYPES.get(a.strip(), a.strip()) for a in inner.split(",")]
        return f"{m.group(1)}<{', '.join(args)}>"
    return re.sub(r"\(.*$", "", name).replace("void ", "").split("::")[-1].strip()


def template_args(short: str):
    m = re.match(r"(\w+)<(.*)>$", short)
    return (m.group(1), [a.strip() for a in m.group(2).split(",")]) if m else (short, [])


def is_dominant(short: str) -> bool:
    """The dense bf16 head-dim-128 forward without mask, split or bias."""
    ident, args = template_args(short)
    return (ident == "attn_fwd_kernel" and len(args) == 10 and args[0] == "bf16"
            and args[1] == "128" and args[6] == "0" and args[7:] == ["false"] * 3)


# --- which workload each kernel ran on, and what it must move -------------

# bench.py runs each (element type, head_dim, mode) on exactly one workload.
BENCH_WORKLOADS = {
    ("bf16", 128, 0): "dense_bf16_b4h16s2048d128",
    ("bf16", 128, 1): "thd_bf16_16seq_len1to4096_h16d128_causal",
    ("bf16", 128, 2): "padded_bf16_b8h32smax8192d128_len2048to8192_causal",
    ("fp16", 64, 0): "dense_fp16_b2h32sq512sk8192d64",
}
ELEM_BYTES = {"bf16": 2, "fp16": 2, "fp32": 4}


def workload_geometry(name: str):
    """(H, D, [(Lq, Lk) per batch or sequence]) of a named workload, with
    true lengths for the variable-length ones."""
    from . import inputs
    builder, kw = inputs.WORKLOADS[name]
    if builder is inputs.dense_inputs:
        return kw["H"], kw["D"], [(kw["Sq"], kw["Sk"])] * kw["B"]
    lengths = inputs.workload_lengths(name)
    return kw["H"], kw["D"], [(int(L), int(L)) for L in lengths]


def product_flops(pairs, H, D, causal):
    """FLOPs of one (Lq x Lk x D) matrix product over every (batch or
    sequence, head), halved under the causal mask (Lq == Lk here)."""
    f = sum(2.0 * lq * lk * D * H for lq, lk in pairs)
    return f / 2 if causal else f


def kernel_accounting(short: str, splits: int | None = None, block_m: int | None = None):
    """{workload, bytes, flops} of one launch of a bench kernel: the
    algorithmic HBM bytes (every input element read once, every output
    element written once, over true lengths) and the matrix-product FLOPs the
    kernel executes.  None for kernels that are not the bench's.

    Forward: Q, K, V read, O written, fp32 LSE written; with a bias also the
    bias entries of every key tile a query tile loads (all of them without the
    mask; under the causal mask query tile m of block_m rows loads keys
    0 .. block_m (m + 1) - 1).  Split forward: Q, K, V read and each split's
    fp32 partial output and logsumexp written; merge: those read, O and LSE
    written.  Backward: dQ reads Q, O, dO, K, V and the fp32 LSE and writes
    dQ and two fp32 values per row (rowsum(dO * O) and LSE * log2(e)); dK/dV
    reads Q, dO, K, V and those row values and writes dK, dV.  FLOPs: 2
    products per forward, 3 in the dQ kernel (S, dP, dQ) and 4 in the dK/dV
    kernel (S, dP, dV, dK)."""
    ident, args = template_args(short)
    if len(args) < 2 or args[0] not in ELEM_BYTES:
        return None
    es, D = ELEM_BYTES[args[0]], int(args[1])
    if ident == "attn_fwd_kernel" and len(args) == 10:
        mode, causal = int(args[6]), args[7] == "true"
        split, bias = args[8] == "true", args[9] == "true"
        block_m = 32 * int(args[2]) * int(args[3])
    elif ident in ("attn_fwd_lagged_kernel", "attn_fwd_3w_kernel") and len(args) == 9:
        mode, causal = int(args[5]), args[6] == "true"
        split, bias = args[7] == "true", args[8] == "true"
        block_m = 32 * int(args[2])
    elif ident == "attn_fwd_kg_kernel" and len(args) == 6:
        # <element, head_dim, key groups, block_n, stages, mode>: four waves of
        # 32 rows share the query tile, no mask, bias or split.
        mode, causal, split, bias, block_m = int(args[5]), False, False, False, 128
    elif ident == "attn_fwd_pingpong_kernel" and len(args) == 6:
        mode, causal, split, bias, block_m = int(args[4]), args[5] == "true", False, False, 256
    elif ident == "attn_fwd_merge_kernel":
        mode, causal, split, bias = 0, False, False, False
    elif ident in ("attn_bwd_dq_kernel", "attn_bwd_dkdv_kernel"):
        mode = int(args[2])
        causal = len(args) > 3 and args[3] == "true"
        split = bias = False
    else:
        return None
    name = BENCH_WORKLOADS.get((args[0], D, mode))
    if name is None:
        return None
    H, _, pairs = workload_geometry(name)
    rq = H * sum(lq for lq, _ in pairs)  # query rows over all heads
    rk = H * sum(lk for _, lk in pairs)
    prod = product_flops(pairs, H, D, causal)
    out = {"workload": name, "bytes": None, "flops": None}
    if ident == "attn_bwd_dq_kernel":
        out["bytes"] = rq * (4 * D * es + 4) + rk * 2 * D * es + rq * 2 * 4
        out["flops"] = 3 * prod
    elif ident == "attn_bwd_dkdv_kernel":
        out["bytes"] = rq * 2 * D * es + rq * 2 * 4 + rk * 4 * D * es
        out["flops"] = 4 * prod
    elif ident == "attn_fwd_merge_kernel":
        if splits is None:
            return out
        out["bytes"] = splits * rq * (D + 1) * 4 + rq * (D * es + 4)
    elif split:
        out["flops"] = 2 * prod
        if splits is not None:
            out["bytes"] = rq * D * es + rk * 2 * D * es + splits * rq * (D + 1) * 4
    else:
        out["flops"] = 2 * prod
        nbytes = rq * (2 * D * es + 4) + rk * 2 * D * es
        if bias:
            entries = 0
            for lq, lk in pairs:
                if causal:
                    entries += sum(min(block_m * (m + 1), lk) * min(block_m, lq - block_m * m)
                                   for m in range((lq + block_m - 1) // block_m))
                else:
                    entries += lq * lk
            nbytes += H * entries * es
        out["bytes"] = nbytes
    return out


def algorithmic_bytes(short: str, splits: int | None = None):
    acc = kernel_accounting(short, splits)
    return None if acc is None else acc["bytes"]


# --- rocprofv3 runs ------------------------------------------------------

def _bench_cmd(extra):
    return [sys.executable, os.path.join(ROOT, "bench.py")] + extra


def _rocprof(opts, out_dir, prefix, bench_args, limit_s):
    d = os.path.join(out_dir, prefix)
    cmd = (["timeout", "-s", "KILL", str(limit_s), "rocprofv3"] + opts
           + ["--output-format", "csv", "-d", d, "-o", prefix, "--"] + _bench_cmd(bench_args))
    print("[rocprof] " + " ".join(cmd), flush=True)
    env = dict(os.environ, TMPDIR="/tmp")
    log_path = os.path.join(out_dir, f"{prefix}.log")
    with open(log_path, "w") as log:
        rc = subprocess.call(cmd, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT)
    files = glob.glob(os.path.join(d, "**", "*.csv"), recursive=True)
    finished = '"metric"' in open(log_path, errors="replace").read()
    # rocprofv3 itself may end with a segmentation fault after the program
    # has finished and its results are written: those results are used.
    # Any other failure (a time limit included) ends the harness, so no
    # further GPU run starts after it.
    if rc != 0 and not (rc == 139 and finished and files):
        raise RuntimeError(f"rocprofv3 exited with {rc} ({log_path}): {' '.join(cmd)}")
    print(f"[rocprof] {prefix}: exit {rc}, {len(files)} csv file(s)", flush=True)
    return d, " ".join(["rocprofv3"] + opts + ["--output-format", "csv", "-d",
                                               os.path.relpath(d, ROOT), "-o", prefix, "--",
                                               "python3", "bench.py"] + bench_args), log_path


def bench_record(log_path):
    """The bench JSON line a profiled run printed (None if absent)."""
    for line in open(log_path, errors="replace"):
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    return None


def split_count(record):
    try:
        return int(record["breakdown"]["dense_fp16_sq512_sk8192"]["splits"])
    except (TypeError, KeyError, ValueError):
        return None


def _col(row, *names):
    """A CSV field by any of its known column names (case-insensitive)."""
    low = {k.lower(): v for k, v in row.items() if k}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(f"none of {names} in the columns {sorted(row)}")


def _csv_rows(d, suffix):
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def parse_stats(d):
    """{short kernel name: (calls, avg_us, min_us, max_us, share_pct)}."""
    out = {}
    for r in _csv_rows(d, "kernel_stats.csv"):
        out[short_name(_col(r, "Name", "Kernel_Name"))] = (
            int(_col(r, "Calls")), float(_col(r, "AverageNs")) / 1e3,
            float(_col(r, "MinNs")) / 1e3, float(_col(r, "MaxNs")) / 1e3,
            float(_col(r, "Percentage")))
    return out


def parse_counters(d):
    """{short kernel name: {counter: mean over dispatches, counter#max: the
    largest dispatch's}}; a counter's rows of one dispatch are summed first.  With a kernel trace in the same
    directory, '_duration_ns' is the mean dispatch duration."""
    per_dispatch = defaultdict(float)
    names = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        disp = _col(r, "Dispatch_Id")
        per_dispatch[(disp, _col(r, "Counter_Name"))] += float(_col(r, "Counter_Value"))
        names[disp] = short_name(_col(r, "Kernel_Name", "Name"))
    for r in _csv_rows(d, "kernel_trace.csv"):
        try:
            disp = _col(r, "Dispatch_Id")
            dur = float(_col(r, "End_Timestamp")) - float(_col(r, "Start_Timestamp"))
        except KeyError:
            continue
        if disp in names:
            per_dispatch[(disp, "_duration_ns")] = dur
    acc = defaultdict(lambda: defaultdict(list))
    for (disp, counter), val in per_dispatch.items():
        acc[names[disp]][counter].append(val)
    out = {}
    for k, cs in acc.items():
        out[k] = {c: sum(v) / len(v) for c, v in cs.items()}
        out[k].update({c + "#max": max(v) for c, v in cs.items()})
    return out


def mfma_busy_pct(c):
    """The profiler's MfmaUtil: SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs
    against GRBM_GUI_ACTIVE of one XCD (the reading here is summed over the
    8 XCDs, so it is divided by 8)."""
    return 100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)


def valu_busy_pct(c):
    """The profiler's VALUBusy: SQ_ACTIVE_INST_VALU / CU count / GUI cycles."""
    return 100.0 * c["SQ_ACTIVE_INST_VALU"] / CUS / (c["GRBM_GUI_ACTIVE"] / XCDS)


def lds_util_pct(c):
    """The profiler's LdsUtil: SQ_LDS_IDX_ACTIVE / (GUI cycles x CU count)."""
    return 100.0 * c["SQ_LDS_IDX_ACTIVE"] / ((c["GRBM_GUI_ACTIVE"] / XCDS) * CUS)


def clock_ghz(c):
    """GUI cycles of one XCD over the dispatch duration (GHz)."""
    dur = c.get("_duration_ns")
    return (c["GRBM_GUI_ACTIVE"] / XCDS) / dur if dur else None


# --- summaries -----------------------------------------------------------

def _header(title, cmds, extra=()):
    lines = [f"# {title}", "", f"kernel_source_sha: {kernel_source_hash()}", *extra, ""]
    lines.append("Commands (repository root, one MI355X; written by `python -m "
                 "scaled_dot_product_03_amd.rocprof`, which runs them from /tmp with "
                 "TMPDIR=/tmp):")
    lines.append("")
    lines.extend("    " + c for c in cmds)
    lines.append("")
    return lines


def _fmt(x, f="{:.1f}"):
    return "n/a" if x is None else f.format(x)


def write_trace(stats, cmd, path):
    lines = _header("Kernel trace: the attention kernels of one bench.py run", [cmd])
    lines.append("| kernel | workload | calls | avg us | min us | max us | share % |")
    lines.append("|---|---|---|---|---|---|---|")
    for k, (n, avg, lo, hi, share) in sorted(stats.items(), key=lambda kv: -kv[1][4]):
        acc = kernel_accounting(k)
        wl = acc["workload"] if acc else "-"
        lines.append(f"| `{k}` | {wl} | {n} | {avg:.1f} | {lo:.1f} | {hi:.1f} | {share:.1f} |")
    lines += ["", TEMPLATE_NOTE, "Calls include bench.py's warmup, untimed settle and "
              "per-launch statistics launches."]
    _write(path, lines)


def write_counters(counters, stats, cmd, path, splits=None):
    dominant_clock = None
    rows = []
    for k, c in sorted(counters.items()):
        if "GRBM_GUI_ACTIVE" not in c or "SQ_VALU_MFMA_BUSY_CYCLES" not in c:
            continue
        acc = kernel_accounting(k, splits)
        ghz = clock_ghz(c)
        if is_dominant(k):
            dominant_clock = ghz
        avg_us = stats.get(k, (0, None))[1] if stats else None
        tflops = (acc["flops"] / (avg_us * 1e-6) / 1e12
                  if acc and acc["flops"] and avg_us else None)
        rows.append(
            f"| `{k}` | {acc['workload'] if acc else '-'} | {mfma_busy_pct(c):.1f} | "
            f"{_fmt(valu_busy_pct(c) if 'SQ_ACTIVE_INST_VALU' in c else None)} | "
            f"{_fmt(lds_util_pct(c) if 'SQ_LDS_IDX_ACTIVE' in c else None)} | "
            f"{c.get('SQ_INSTS_VALU_TRANS_F32', 0):.3g} | {c.get('SQ_WAIT_INST_LDS', 0):.3g} | "
            f"{c.get('SQ_LDS_BANK_CONFLICT', 0):.3g} | {_fmt(ghz, '{:.2f}')} | "
            f"{_fmt(tflops, '{:.0f}')} |")
    extra = ([f"dominant_kernel_shader_clock_ghz: {dominant_clock:.4f}"]
             if dominant_clock else [])
    lines = _header("Matrix-core, VALU and LDS counters: every attention kernel of the bench "
                    "workloads", [cmd], extra)
    lines += [
        "MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs); "
        "VALU busy % = SQ_ACTIVE_INST_VALU / 256 CUs / GRBM_GUI_ACTIVE per XCD; LDS use % = "
        "SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE per XCD x 256 CUs) (the profiler's MfmaUtil, "
        "VALUBusy and LdsUtil formulas; GRBM_GUI_ACTIVE is read summed over the 8 XCDs). "
        "Clock = GRBM_GUI_ACTIVE per XCD over the dispatch's duration in the same run. "
        "TFLOP/s = the kernel's matrix-product FLOPs over its average duration in the trace "
        "pass (2 products per forward, 3 for dQ, 4 for dK/dV). Counters are means over the "
        "dispatches of the profiled run.",
        "",
        "| kernel | workload | MFMA busy % | VALU busy % | LDS use % | v_exp_f32 wave-instr | "
        "SQ_WAIT_INST_LDS | LDS bank-conflict cycles | clock GHz | TFLOP/s (trace) |",
        "|---|---|---|---|---|---|---|---|---|---|"] + rows
    lines += ["", TEMPLATE_NOTE]
    _write(path, lines)
    return dominant_clock


def copy_factors(fetch, write):
    """Bytes per KiB of counter reading, from the plain copy's known traffic.
    The copy kernel also serves small uploads (cu_seqlens) in the same run,
    so its largest dispatch -- the calibration copy -- is the one used."""
    n_kib = COPY_MIB * 1024
    fc = [c.get("FETCH_SIZE#max", c.get("FETCH_SIZE")) for k, c in fetch.items()
          if "copyBuffer" in k and "FETCH_SIZE" in c]
    wc = [c.get("WRITE_SIZE#max", c.get("WRITE_SIZE")) for k, c in write.items()
          if "copyBuffer" in k and "WRITE_SIZE" in c]
    if not fc or not wc:
        raise RuntimeError("the calibration copy kernel is missing from the counter results")
    return n_kib / max(fc), n_kib / max(wc), max(fc), max(wc)


def write_traffic(fetch, write, stats, cmds, path, splits=None):
    f_fac, w_fac, f_copy, w_copy = copy_factors(fetch, write)
    rows, dominant = [], None
    for k in sorted(set(fetch) & set(write)):
        acc = kernel_accounting(k, splits)
        if acc is None:
            continue
        rd = fetch[k]["FETCH_SIZE"] * f_fac * 1024
        wr = write[k]["WRITE_SIZE"] * w_fac * 1024
        alg = acc["bytes"]
        avg_us = stats.get(k, (0, 0.0))[1] if stats else 0.0
        gbs = (rd + wr) / (avg_us * 1e-6) / 1e9 if avg_us else None
        rows.append((k, acc["workload"], fetch[k]["FETCH_SIZE"], write[k]["WRITE_SIZE"], rd, wr,
                     alg, avg_us, gbs))
        if is_dominant(k):
            dominant = rd + wr
    extra = [f"hbm_bytes_per_launch: {dominant:.6e}"] if dominant is not None else []
    lines = _header("HBM traffic per launch: every attention kernel of the bench workloads",
                    cmds, extra)
    lines.append(f"Calibration: a {COPY_MIB} MiB device copy ({COPY_MIB * 1024} KiB read and "
                 f"written) reads {f_copy:.0f} KiB on FETCH_SIZE and {w_copy:.0f} KiB on "
                 f"WRITE_SIZE, so FETCH_SIZE is scaled by {f_fac:.3f} and WRITE_SIZE by "
                 f"{w_fac:.3f}.")
    lines.append("")
    lines.append("| kernel | workload | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB read | "
                 "scaled MB written | total MB | algorithmic MB | total / algorithmic | "
                 "avg us (trace) | HBM GB/s | % of 8 TB/s |")
    lines.append("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for k, wl, fk, wk, rd, wr, alg, avg_us, gbs in rows:
        alg_s = f"{alg / 1e6:.1f} | {(rd + wr) / alg:.2f}" if alg else "n/a | n/a"
        gbs_s = f"{gbs:.0f} | {100 * gbs / HBM_PEAK_GBS:.1f}" if gbs else "n/a | n/a"
        avg_s = f"{avg_us:.1f}" if avg_us else "n/a"
        lines.append(f"| `{k}` | {wl} | {fk:.0f} | {wk:.0f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{(rd + wr) / 1e6:.1f} | {alg_s} | {avg_s} | {gbs_s} |")
    lines += ["", "Algorithmic bytes (per launch, over true lengths): forward Q, K, V read "
              "once, O and the fp32 LSE written once; with a bias also the bias entries of "
              "every key tile a query tile loads (all of them without the mask; under the "
              "causal mask query tile m of block_m rows loads keys 0 .. block_m (m + 1) - 1); "
              "split forward: Q, K, V read and every split's fp32 partial output and "
              "logsumexp written; merge: those read, O and LSE written; backward dQ: Q, O, "
              "dO, K, V and the fp32 LSE read, dQ and two fp32 values per row written; dK/dV: "
              "Q, dO, K, V and the row values read, dK and dV written.  HBM GB/s = "
              "scaled bytes over the kernel's average duration in the trace pass.  The dense "
              "non-causal forward without bias is the kernel bench.py reports as "
              "roofline.traffic.", "", TEMPLATE_NOTE]
    _write(path, lines)


def _write(path, lines):
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"[rocprof] wrote {path}", flush=True)


PASSES = ["trace", "counters", "traffic"]


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("passes", nargs="*", help=f"any of {PASSES} (default: all)")
    ap.add_argument("--out", default=os.path.join(ROOT, "rocprof_out"))
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--limit", type=int, default=240, help="seconds per rocprofv3 run")
    ap.add_argument("--summarize", action="store_true",
                    help="run nothing: write the summaries from the results an earlier run "
                         "left under --out (copied back from the machine that ran them)")
    args = ap.parse_args(argv)
    bad = [p for p in args.passes if p not in PASSES]
    if bad:
        ap.error(f"unknown pass(es) {bad}; choose from {PASSES}")
    args.passes = args.passes or list(PASSES)
    return args


def _runs(steps):
    """(profiler options, output prefix, bench arguments) of every pass."""
    short = ["--steps", "3", "--warmup", "1"] + PROFILED
    cal = short + ["--calibrate-copy-mib", str(COPY_MIB)]
    return {
        "trace": [(["--kernel-trace", "--stats"], "trace",
                   ["--steps", str(steps), "--warmup", "5", "--no-cpu-baseline"])],
        "counters": [(["--kernel-trace", "--pmc"] + SQ_COUNTERS, "sq", short)],
        "traffic": [(["--pmc", "FETCH_SIZE"], "fetch", cal), (["--pmc", "WRITE_SIZE"], "write", cal)],
    }


def _command_text(opts, out_dir, prefix, bench_args):
    d = os.path.join(out_dir, prefix)
    return " ".join(["rocprofv3"] + opts + ["--output-format", "csv", "-d",
                                            os.path.relpath(d, ROOT), "-o", prefix, "--",
                                            "python3", "bench.py"] + bench_args)


def main(argv=None):
    args = parse_args(argv)
    out = os.path.abspath(args.out)
    os.makedirs(out, exist_ok=True)
    os.makedirs(args.profiles, exist_ok=True)
    runs = _runs(args.steps)
    if not args.summarize:
        for p in args.passes:
            for opts, prefix, bench_args in runs[p]:
                _rocprof(opts, out, prefix, bench_args, args.limit)

    def dir_cmd_log(opts, prefix, bench_args):
        return (os.path.join(out, prefix), _command_text(opts, out, prefix, bench_args),
                os.path.join(out, f"{prefix}.log"))

    stats, splits = None, None
    if "trace" in args.passes or os.path.isdir(os.path.join(out, "trace")):
        d, cmd, log = dir_cmd_log(*runs["trace"][0])
        stats = parse_stats(d)
        splits = split_count(bench_record(log)) if os.path.exists(log) else None
        if "trace" in args.passes:
            write_trace(stats, cmd, os.path.join(args.profiles, TRACE_FILE))
    if "counters" in args.passes:
        d, cmd, log = dir_cmd_log(*runs["counters"][0])
        splits = splits or split_count(bench_record(log))
        write_counters(parse_counters(d), stats, cmd, os.path.join(args.profiles, COUNTERS_FILE),
                       splits)
    if "traffic" in args.passes:
        (df, cf, logf), (dw, cw, _) = [dir_cmd_log(*r) for r in runs["traffic"]]
        splits = splits or split_count(bench_record(logf))
        write_traffic(parse_counters(df), parse_counters(dw), stats, [cf, cw],
                      os.path.join(args.profiles, TRAFFIC_FILE), splits)
    return 0


if __name__ == "__main__":
    sys.exit(main())
