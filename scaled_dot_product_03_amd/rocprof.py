"""rocprofv3 harness: kernel times, matrix-core utilisation and HBM traffic.

    python -m scaled_dot_product_03_amd.rocprof [trace] [counters] [traffic]
        [--out gpurun_out/prof] [--profiles profiles] [--steps 20]

Runs ``bench.py`` under rocprofv3 as child processes (this process never
touches the GPU) and writes short markdown summaries into ``profiles/``:

* ``trace``: ``--kernel-trace --stats`` over a normal bench run; per kernel
  the call count and the average, min and max duration.
* ``counters``: one ``--pmc`` pass over the dense bf16 B4 H16 S2048 D128
  forward (both masks, with and without a bias): matrix-core busy % =
  SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), LDS
  bank-conflict cycles, v_exp_f32 wave-instructions and LDS wait cycles.
* ``traffic``: one ``--pmc FETCH_SIZE`` and one ``--pmc WRITE_SIZE`` pass over
  the same forwards plus a plain device copy of known size, whose readings
  give the factor that turns each counter into bytes.  Bytes per launch and,
  with the trace's average durations, achieved HBM GB/s against 8 TB/s.

Counter passes stay within one pass's hardware limits (at most 8 SQ, 4 TCC
and 2 GRBM counters) and are never combined with API tracing.  Every
rocprofv3 run is bounded by ``timeout -s KILL``.  The summaries carry the
hash of the forward kernel's sources; ``bench.py`` reports the traffic
figure only while that hash matches the sources it runs.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import subprocess
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ["scaled_dot_product_03_amd/csrc/attn_fwd.hip",
                  "scaled_dot_product_03_amd/csrc/attn_fwd_bf16.hip",
                  "scaled_dot_product_03_amd/csrc/attn_fwd_kernels.h",
                  "scaled_dot_product_03_amd/csrc/attn_common.h",
                  "scaled_dot_product_03_amd/csrc/dispatch_table.inc"]
TRAFFIC_TAG = "dense_bf16_b4h16s2048d128_noncausal"
HBM_PEAK_GBS = 8000.0
XCDS = 8
SIMDS = 1024  # 256 CUs x 4 SIMDs
COPY_MIB = 256

# The dense bf16 workload the counter passes run (bench.py's headline).
B, H, S, D, ELEM = 4, 16, 2048, 128, 2

SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS",
               "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_WAVES", "SQ_BUSY_CYCLES",
               "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE"]
FWD_ONLY = ["--no-cpu-baseline", "--no-varlen", "--no-padded", "--no-splitk", "--no-bwd"]
TEMPLATE_NOTE = ("Forward template arguments: <element type, head_dim, waves, row blocks per wave, "
                 "block_n, stages, mode (0 dense, 1 compact, 2 padded), causal, split, bias>; "
                 "merge and backward kernels: <element type, head_dim[, mode, causal]>.")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(tag: str = TRAFFIC_TAG, profiles_dir: str | None = None):
    """HBM bytes per launch of the dominant kernel from a committed traffic
    summary, if it was taken on the current kernel sources; else None."""
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"), f"hbm_traffic_{tag}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha:\s*(\w+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


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


def algorithmic_bytes(short: str):
    """HBM bytes a forward launch on the dense B4 H16 S2048 D128 bf16
    workload must move: Q, K, V read once, O written, the fp32 LSE written,
    and with a bias the bias entries of every key tile a query tile loads."""
    ident, args = template_args(short)
    if ident != "attn_fwd_kernel" or len(args) != 10 or args[1] != str(D) or args[6] != "0":
        return None
    if args[8] == "true":  # split: partial results go through a workspace
        return None
    qkvo = 4 * B * H * S * D * ELEM + B * H * S * 4
    if args[9] != "true":
        return qkvo
    block_m = 32 * int(args[2]) * int(args[3])
    if args[7] != "true":
        return qkvo + B * H * S * S * ELEM
    keys = sum(min(block_m * (m + 1), S) * min(block_m, S - block_m * m)
               for m in range((S + block_m - 1) // block_m))
    return qkvo + B * H * keys * ELEM


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
                                               "python3", "bench.py"] + bench_args)


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
    """{short kernel name: {counter: mean over dispatches}}; a counter's rows
    of one dispatch are summed first."""
    per_dispatch = defaultdict(float)
    names = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        disp = _col(r, "Dispatch_Id")
        per_dispatch[(disp, _col(r, "Counter_Name"))] += float(_col(r, "Counter_Value"))
        names[disp] = short_name(_col(r, "Kernel_Name", "Name"))
    acc = defaultdict(lambda: defaultdict(list))
    for (disp, counter), val in per_dispatch.items():
        acc[names[disp]][counter].append(val)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def mfma_busy_pct(c):
    return 100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)


# --- summaries -----------------------------------------------------------

def _header(title, cmds):
    lines = [f"# {title}", "", f"kernel_source_sha: {kernel_source_hash()}", ""]
    lines.append("Commands (repository root, one MI355X; written by `python -m "
                 "scaled_dot_product_03_amd.rocprof`, which runs them from /tmp with "
                 "TMPDIR=/tmp):")
    lines.append("")
    lines.extend("    " + c for c in cmds)
    lines.append("")
    return lines


def write_trace(stats, cmd, path):
    lines = _header("Kernel trace: the attention kernels of one bench.py run", [cmd])
    lines.append("| kernel | calls | avg us | min us | max us | share % |")
    lines.append("|---|---|---|---|---|---|")
    for k, (n, avg, lo, hi, share) in sorted(stats.items(), key=lambda kv: -kv[1][4]):
        lines.append(f"| `{k}` | {n} | {avg:.1f} | {lo:.1f} | {hi:.1f} | {share:.1f} |")
    lines += ["", TEMPLATE_NOTE, "Calls include bench.py's warmup and untimed settle launches."]
    _write(path, lines)


def write_counters(counters, cmd, path):
    lines = _header("Matrix-core, VALU and LDS counters: attention forward, dense bf16 B4 H16 "
                    "S2048 D128", [cmd])
    lines.append("MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 "
                 "SIMDs); GRBM_GUI_ACTIVE is summed over the XCDs.")
    lines.append("")
    lines.append("| kernel | MFMA busy % | LDS bank-conflict cycles | v_exp_f32 wave-instr | "
                 "SQ_WAIT_INST_LDS | GRBM_GUI_ACTIVE |")
    lines.append("|---|---|---|---|---|---|")
    for k, c in sorted(counters.items()):
        if "GRBM_GUI_ACTIVE" not in c or "SQ_VALU_MFMA_BUSY_CYCLES" not in c:
            continue
        lines.append(f"| `{k}` | {mfma_busy_pct(c):.1f} | {c.get('SQ_LDS_BANK_CONFLICT', 0):.3g} | "
                     f"{c.get('SQ_INSTS_VALU_TRANS_F32', 0):.3g} | "
                     f"{c.get('SQ_WAIT_INST_LDS', 0):.3g} | {c['GRBM_GUI_ACTIVE']:.3g} |")
    lines += ["", TEMPLATE_NOTE]
    _write(path, lines)


def copy_factors(fetch, write):
    """Bytes per KiB of counter reading, from the plain copy's known traffic."""
    n_kib = COPY_MIB * 1024
    fc = [c["FETCH_SIZE"] for k, c in fetch.items() if "copyBuffer" in k and "FETCH_SIZE" in c]
    wc = [c["WRITE_SIZE"] for k, c in write.items() if "copyBuffer" in k and "WRITE_SIZE" in c]
    if not fc or not wc:
        raise RuntimeError("the calibration copy kernel is missing from the counter results")
    return n_kib / max(fc), n_kib / max(wc), max(fc), max(wc)


def write_traffic(fetch, write, stats, cmds, path):
    f_fac, w_fac, f_copy, w_copy = copy_factors(fetch, write)
    lines = _header("HBM traffic per launch: attention forward, dense bf16 B4 H16 S2048 D128",
                    cmds)
    rows, dominant = [], None
    for k in sorted(set(fetch) & set(write)):
        if not k.startswith("attn_fwd_kernel"):
            continue
        rd = fetch[k]["FETCH_SIZE"] * f_fac * 1024
        wr = write[k]["WRITE_SIZE"] * w_fac * 1024
        alg = algorithmic_bytes(k)
        avg_us = stats.get(k, (0, 0.0))[1] if stats else 0.0
        gbs = (rd + wr) / (avg_us * 1e-6) / 1e9 if avg_us else None
        rows.append((k, fetch[k]["FETCH_SIZE"], write[k]["WRITE_SIZE"], rd, wr, alg, avg_us, gbs))
        if is_dominant(k):
            dominant = rd + wr
    if dominant is not None:
        lines.insert(3, f"hbm_bytes_per_launch: {dominant:.6e}")
    lines.append(f"Calibration: a {COPY_MIB} MiB device copy ({COPY_MIB * 1024} KiB read and "
                 f"written) reads {f_copy:.0f} KiB on FETCH_SIZE and {w_copy:.0f} KiB on "
                 f"WRITE_SIZE, so FETCH_SIZE is scaled by {f_fac:.3f} and WRITE_SIZE by "
                 f"{w_fac:.3f}.")
    lines.append("")
    lines.append("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB read | scaled MB written | "
                 "total MB | algorithmic MB | avg us (trace) | HBM GB/s | % of 8 TB/s |")
    lines.append("|---|---|---|---|---|---|---|---|---|---|")
    for k, fk, wk, rd, wr, alg, avg_us, gbs in rows:
        alg_s = f"{alg / 1e6:.1f}" if alg else "n/a"
        gbs_s = f"{gbs:.0f} | {100 * gbs / HBM_PEAK_GBS:.1f}" if gbs else "n/a | n/a"
        avg_s = f"{avg_us:.1f}" if avg_us else "n/a"
        lines.append(f"| `{k}` | {fk:.0f} | {wk:.0f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{(rd + wr) / 1e6:.1f} | {alg_s} | {avg_s} | {gbs_s} |")
    lines += ["", "Algorithmic bytes: Q, K, V read once and O written (4 x 33.55 MB) plus the "
              "fp32 LSE (0.52 MB); with a bias, the bias entries of every key tile a query "
              "tile loads (all of them without the mask; under the causal mask query tile m "
              "of block_m rows loads keys 0 .. block_m (m + 1) - 1).  HBM GB/s = scaled bytes "
              "over the kernel's average duration in the trace pass.  The dense non-causal "
              "kernel without bias is the one bench.py reports as roofline.traffic.",
              "", TEMPLATE_NOTE]
    _write(path, lines)


def _write(path, lines):
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"[rocprof] wrote {path}", flush=True)


PASSES = ["trace", "counters", "traffic"]


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("passes", nargs="*", help=f"any of {PASSES} (default: all)")
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "prof"))
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--limit", type=int, default=170, help="seconds per rocprofv3 run")
    args = ap.parse_args(argv)
    bad = [p for p in args.passes if p not in PASSES]
    if bad:
        ap.error(f"unknown pass(es) {bad}; choose from {PASSES}")
    args.passes = args.passes or list(PASSES)
    return args


def main(argv=None):
    args = parse_args(argv)
    out = os.path.abspath(args.out)
    os.makedirs(out, exist_ok=True)
    os.makedirs(args.profiles, exist_ok=True)

    stats = None
    if "trace" in args.passes:
        d, cmd = _rocprof(["--kernel-trace", "--stats"], out, "trace",
                          ["--steps", str(args.steps), "--warmup", "5", "--no-cpu-baseline"],
                          args.limit)
        stats = parse_stats(d)
        write_trace(stats, cmd, os.path.join(args.profiles,
                                             "kernel_trace_attn_fwd_bench_workloads.md"))
    short = ["--steps", "3", "--warmup", "1"] + FWD_ONLY
    if "counters" in args.passes:
        d, cmd = _rocprof(["--pmc"] + SQ_COUNTERS, out, "sq", short, args.limit)
        write_counters(parse_counters(d), cmd,
                       os.path.join(args.profiles, "counters_attn_fwd_dense_bf16_s2048_d128.md"))
    if "traffic" in args.passes:
        cal = short + ["--calibrate-copy-mib", str(COPY_MIB)]
        df, cf = _rocprof(["--pmc", "FETCH_SIZE"], out, "fetch", cal, args.limit)
        dw, cw = _rocprof(["--pmc", "WRITE_SIZE"], out, "write", cal, args.limit)
        write_traffic(parse_counters(df), parse_counters(dw), stats, [cf, cw],
                      os.path.join(args.profiles, f"hbm_traffic_{TRAFFIC_TAG}.md"))
    return 0


if __name__ == "__main__":
    sys.exit(main())
