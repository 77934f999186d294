"""Offline sweep that writes the compiled-in dispatch table.

For every problem class (dtype, head_dim) a set of candidate kernel shapes
(waves per workgroup, keys per tile, LDS stages, schedule: 0 single group,
1 ping-pong of two wave groups) is compiled into its own
build of libsdpa03.so.  A candidate counts only if its build has no register
spills, keeps two waves per SIMD, and then passes the GPU parity tests
(tests/test_gpu_parity.py, run against that build); only then is it timed
on the workloads of its class.  The fastest candidate per class goes into
csrc/dispatch_table.inc.  There is no tuning at run time.

    python -m scaled_dot_product_03_amd.sweep build   # CPU: compile candidates
    python -m scaled_dot_product_03_amd.sweep run     # GPU: parity, then timing
    python -m scaled_dot_product_03_amd.sweep write   # rewrite dispatch_table.inc

`run` writes _sweep/results.json; `write` reads it.
"""

from __future__ import annotations

import json
import os
import re
import subprocess
import sys
import time

from .build import CSRC, DEVICE_FLAGS, HIPCC, ROOT, SOURCES, ARCH

SWEEP_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_sweep")
RESULTS = os.path.join(SWEEP_DIR, "results.json")
TABLE = os.path.join(CSRC, "dispatch_table.inc")
DTYPE_CODES = {"fp32": 0, "fp16": 1, "bf16": 2}

# Candidate (waves, block_n, stages, pingpong) per class.
CANDIDATES = {
    ("bf16", 128): [(4, 64, 2, 0), (4, 32, 3, 0), (8, 64, 2, 0), (8, 64, 3, 0), (8, 32, 3, 0),
                    (8, 64, 3, 1), (8, 128, 2, 1)],
    ("fp16", 64): [(4, 64, 2, 0), (4, 64, 3, 0), (4, 32, 3, 0), (8, 64, 3, 0), (8, 64, 3, 1),
                   (8, 128, 2, 1)],
}

# Timed workloads per class: (workload name from inputs.WORKLOADS, weight).
TIMED = {
    ("bf16", 128): ["dense_bf16_b4h16s2048d128", "thd_bf16_16seq_len1to4096_h16d128_causal",
                    "padded_bf16_b8h32smax8192d128_len2048to8192_causal"],
    ("fp16", 64): ["dense_fp16_b2h32sq512sk8192d64"],
}


def _cand4(cand):
    """Candidates recorded before the schedule field existed are single-group."""
    return tuple(cand) + (0,) * (4 - len(cand))


def _name(cls, cand):
    w, n, st, pp = _cand4(cand)
    return f"{cls[0]}_d{cls[1]}_w{w}_n{n}_s{st}" + ("_pp" if pp else "")


def _lib_path(cls, cand):
    return os.path.join(SWEEP_DIR, f"libsdpa03_{_name(cls, cand)}.so")


def _resources(cls, cand):
    """(max VGPRs, spills, waves/SIMD) of the candidate's kernels for its class."""
    defs = _defines(cls, cand)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-c",
           *DEVICE_FLAGS, "-I", os.path.join(ROOT, "include"), "-x", "hip",
           os.path.join(CSRC, "attn_fwd.hip"), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", *defs]
    out = subprocess.run(cmd, capture_output=True, text=True).stderr
    dt_tag = {"bf16": "DF16b", "fp16": "DF16_", "fp32": "f"}[cls[0]]
    w, n, st, pp = _cand4(cand)
    want = (f"attn_fwd_pingpong_kernelI{dt_tag}Li{cls[1]}ELi{n}ELi{st}E" if pp else
            f"attn_fwd_kernelI{dt_tag}Li{cls[1]}ELi{w}ELi{n}ELi{st}E")
    vg, sp, occ, cur = 0, 0, 99, None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            continue
        if cur is None or want not in cur:
            continue
        m = re.search(r"remark:\s+(VGPRs|VGPRs Spill|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m:
            val = int(m.group(2))
            if m.group(1) == "VGPRs":
                vg = max(vg, val)
            elif m.group(1) == "VGPRs Spill":
                sp = max(sp, val)
            else:
                occ = min(occ, val)
    return vg, sp, occ


def _defines(cls, cand):
    w, n, st, pp = _cand4(cand)
    return [f"-DSDPA03_SWEEP_DTYPE={DTYPE_CODES[cls[0]]}", f"-DSDPA03_SWEEP_HEAD_DIM={cls[1]}",
            f"-DSDPA03_SWEEP_WAVES={w}", f"-DSDPA03_SWEEP_BLOCK_N={n}",
            f"-DSDPA03_SWEEP_STAGES={st}", f"-DSDPA03_SWEEP_PINGPONG={pp}"]


def build(only=None):
    """Compile the candidates (those whose name contains one of `only`, if given)."""
    os.makedirs(SWEEP_DIR, exist_ok=True)
    plan = []
    for cls, cands in CANDIDATES.items():
        for cand in cands:
            if only and not any(o in _name(cls, cand) for o in only):
                continue
            vg, sp, occ = _resources(cls, cand)
            ok = sp == 0 and occ >= 2
            print(f"{_name(cls, cand):28s} vgpr={vg} spill={sp} waves/simd={occ} "
                  f"{'build' if ok else 'skip'}", flush=True)
            if not ok:
                continue
            cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
                   *DEVICE_FLAGS, "-I", os.path.join(ROOT, "include"), "-x", "hip",
                   *[os.path.join(CSRC, s) for s in SOURCES], "-o", _lib_path(cls, cand),
                   *_defines(cls, cand)]
            plan.append((cls, cand, subprocess.Popen(cmd, stdout=subprocess.DEVNULL,
                                                     stderr=subprocess.PIPE, text=True)))
    built = []
    for cls, cand, proc in plan:
        _, err = proc.communicate()
        if proc.returncode != 0:
            raise RuntimeError(f"build of {_name(cls, cand)} failed:\n{err}")
        built.append({"dtype": cls[0], "head_dim": cls[1], "cand": list(cand)})
    with open(os.path.join(SWEEP_DIR, "built.json"), "w") as f:
        json.dump(built, f)
    print(f"built {len(built)} candidates", flush=True)


def _time_workload(binding, torch, inputs, name, reps=10):
    x = inputs.workload(name)
    dev = torch.device("cuda:0")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    calls = []
    if x.mode == "dense":
        for causal in x.causal_modes:
            calls.append(lambda c=causal: binding.attn_fwd(q, k, v, scale=x.scale, causal=c))
    elif x.mode == "compact":
        cu = torch.from_numpy(x.cu_seqlens_q).to(dev)
        mx = int(max(x.meta["lengths_q"]))
        calls.append(lambda: binding.attn_fwd_compact_varlen(q, k, v, cu, cu, mx, mx,
                                                             scale=x.scale, causal=True))
    else:
        cu = torch.from_numpy(x.cu_seqlens_q).to(dev)
        calls.append(lambda: binding.attn_fwd_padded_varlen(q, k, v, cu, cu, scale=x.scale,
                                                            causal=True))
    out = []
    for call in calls:
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / reps)
    return out


def _timing_child(lib):
    """Runs in a fresh process with SDPA03_LIBRARY set: prints JSON timings."""
    import torch
    from . import binding, inputs
    binding.load_library(lib)
    cls = json.loads(os.environ["SDPA03_SWEEP_CLASS"])
    res = {}
    for name in TIMED.get(tuple(cls), []):
        res[name] = _time_workload(binding, torch, inputs, name)
    print("SWEEP_TIMINGS " + json.dumps(res), flush=True)


def run():
    with open(os.path.join(SWEEP_DIR, "built.json")) as f:
        built = json.load(f)
    results = []
    for b in built:
        cls, cand = (b["dtype"], b["head_dim"]), _cand4(b["cand"])
        if cls not in TIMED:
            continue
        lib = _lib_path(cls, cand)
        env = dict(os.environ, SDPA03_LIBRARY=lib, SDPA03_SWEEP_CLASS=json.dumps(list(cls)))
        print(f"== {_name(cls, cand)}: parity", flush=True)
        t0 = time.time()
        par = subprocess.run([sys.executable, "-u", "-m", "pytest", "-x", "-q", "-m", "gpu",
                              "--timeout", "300", "--timeout-method", "thread",
                              os.path.join(ROOT, "tests", "test_gpu_parity.py")],
                             cwd=ROOT, env=env, capture_output=True, text=True)
        tail = par.stdout.strip().splitlines()[-1:] if par.stdout else []
        print(f"   parity rc={par.returncode} {tail} ({time.time() - t0:.0f} s)", flush=True)
        entry = {"dtype": cls[0], "head_dim": cls[1], "cand": list(cand),
                 "parity": par.returncode == 0, "ms": None}
        if par.returncode == 0:
            tim = subprocess.run([sys.executable, "-u", "-c",
                                  "import sys; sys.path.insert(0, %r); "
                                  "from scaled_dot_product_03_amd import sweep; "
                                  "sweep._timing_child(%r)" % (ROOT, lib)],
                                 cwd=ROOT, env=env, capture_output=True, text=True)
            m = re.search(r"SWEEP_TIMINGS (.*)", tim.stdout)
            if tim.returncode != 0 or not m:
                raise RuntimeError(f"timing of {_name(cls, cand)} failed: {tim.stderr[-2000:]}")
            entry["ms"] = json.loads(m.group(1))
            print(f"   ms {entry['ms']}", flush=True)
        else:
            print(par.stdout[-3000:], flush=True)
        results.append(entry)
        with open(RESULTS, "w") as f:
            json.dump(results, f, indent=1)


def write(results_path=RESULTS, table_path=TABLE):
    with open(results_path) as f:
        results = json.load(f)
    best = {}
    for r in results:
        if not r["parity"] or not r["ms"]:
            continue
        cls = (r["dtype"], r["head_dim"])
        total = sum(sum(v) for v in r["ms"].values())
        if cls not in best or total < best[cls][0]:
            best[cls] = (total, _cand4(r["cand"]), r["ms"])
    fallback = {("bf16", 128): (4, 64, 2, 0), ("fp16", 128): (4, 64, 2, 0),
                ("bf16", 64): (4, 64, 3, 0), ("fp16", 64): (4, 64, 3, 0)}
    pick = {cls: (best[cls][1] if cls in best else fallback[cls]) for cls in fallback}
    # classes without their own timed workload follow the timed class of the same head_dim
    if ("bf16", 128) in best:
        pick[("fp16", 128)] = best[("bf16", 128)][1]
    if ("fp16", 64) in best:
        pick[("bf16", 64)] = best[("fp16", 64)][1]
    lines = ["  // BEGIN TABLE (generated)"]
    for cls, (total, cand, ms) in sorted(best.items()):
        lines.append(f"  // {cls[0]} d{cls[1]}: (waves, block_n, stages, pingpong) = {cand}; "
                     f"sum of timed workloads {total:.3f} ms")
    lines += ["  if constexpr (sizeof(T) == 4) {", "    return TableEntry{4, 32, 2, 0};"]
    for dt in ("bf16", "fp16"):
        for d in (128, 64):
            w, n, st, pp = pick[(dt, d)]
            cond = (f"dtype_code<T>() == {'DT_BF16' if dt == 'bf16' else 'DT_F16'} && D == {d}")
            lines += [f"  }} else if constexpr ({cond}) {{",
                      f"    return TableEntry{{{w}, {n}, {st}, {pp}}};"]
    lines += ["  } else {", "    return TableEntry{4, 64, 2, 0};", "  }", "  // END TABLE"]
    text = open(table_path).read()
    text = re.sub(r"  // BEGIN TABLE \(generated\).*  // END TABLE", "\n".join(lines), text,
                  flags=re.S)
    with open(table_path, "w") as f:
        f.write(text)
    print("\n".join(lines))
    return pick


if __name__ == "__main__":
    if sys.argv[1] == "build":
        build(sys.argv[2:] or None)
    else:
        {"run": run, "write": write}[sys.argv[1]]()
