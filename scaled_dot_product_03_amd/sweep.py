"""Offline sweep that writes the compiled-in dispatch table.

The dispatch key is (dtype, head_dim, sequence-length bucket): four query
buckets (<= 128, <= 512, <= 4096, longer) by two key buckets (<= 512,
longer), as
AOTriton's tuning database probes sequence lengths, head dim and dtype
(AOTriton issue #12, the maintainer's replies).  For every class (dtype,
head_dim) a set of candidate kernel shapes (waves per workgroup, keys per
tile, LDS stages, schedule: 0 single group, 1 ping-pong of two wave groups,
2 single group with two 32-row blocks per wave)
is compiled into its own build of libsdpa03.so, the shape applied to every
bucket of the class.  A candidate counts only if its build has no register
spills (an occupancy the LDS or the two-row-block schedule limits to one wave
per SIMD is left to the timing), and then passes the GPU parity tests
(tests/test_gpu_parity.py, run against that build): the same page warns that
a kernel built with some configurations runs but gives wrong results.  Only
then is it timed, on workloads of every bucket.  Per bucket, the passing
candidate with the lowest score on that bucket's workloads (its time over the
best time, summed over the timed calls) goes into csrc/dispatch_table.inc.  There is no tuning at run time.

    python -m scaled_dot_product_03_amd.sweep build [name ...]  # CPU: compile candidates
    python -m scaled_dot_product_03_amd.sweep run [name ...]    # GPU: parity, then timing
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

# Candidate (waves, block_n, stages, schedule) per class; schedule 0 single
# group, 1 ping-pong, 2 single group with two 32-row blocks per wave.
CANDIDATES = {
    ("bf16", 128): [(2, 32, 2, 0), (4, 32, 2, 0), (4, 64, 2, 0), (4, 32, 3, 0), (8, 64, 2, 0),
                    (8, 64, 3, 0), (8, 64, 4, 0), (8, 32, 3, 0), (8, 64, 3, 1), (8, 128, 2, 1),
                    (4, 32, 3, 2)],
    ("fp16", 64): [(2, 32, 2, 0), (4, 32, 2, 0), (4, 64, 2, 0), (4, 64, 3, 0), (4, 64, 4, 0),
                   (4, 32, 3, 0), (8, 64, 3, 0), (8, 64, 3, 1), (8, 128, 2, 1), (4, 64, 3, 2)],
}

BUCKETS = ["q<=128,k<=512", "q<=128,k>512", "q<=512,k<=512", "q<=512,k>512",
           "q<=4096,k<=512", "q<=4096,k>512", "q>4096,k<=512", "q>4096,k>512"]


def _bucket_workloads(dtype, d):
    """Timed workloads per bucket: (name, builder, kwargs).  The five named
    workloads sit in their buckets; the others are seeded synthetic shapes of
    the same recipe (inputs.py) that fill the short buckets."""
    dense = lambda B, H, Sq, Sk, causal=(False, True): (
        f"dense_{dtype}_b{B}h{H}sq{Sq}sk{Sk}d{d}", "dense",
        dict(B=B, H=H, Sq=Sq, Sk=Sk, D=d, dtype=dtype, seed=11, causal_modes=causal))
    thd = lambda n, hi: (f"thd_{dtype}_{n}seq_len1to{hi}_h16d{d}_causal", "compact",
                         dict(n_seqs=n, H=16, D=d, dtype=dtype, seed=12, len_lo=1, len_hi=hi))
    w = {
        0: [dense(128, 16, 64, 64), dense(64, 16, 128, 128), thd(256, 128)],
        1: [dense(16, 16, 128, 4096, (False,))],
        2: [dense(16, 16, 256, 256), dense(8, 16, 512, 512), thd(128, 256), thd(64, 512)],
        3: [dense(2, 32, 512, 8192, (False,))],
        4: [dense(4, 16, 2048, 512, (False,))],
        5: [dense(4, 16, 2048, 2048), thd(16, 4096)],
        6: [dense(1, 16, 8192, 512, (False,))],
        7: [dense(1, 16, 8192, 8192)],
    }
    if (dtype, d) == ("bf16", 128):
        w[7].append(("padded_bf16_b8h32smax8192d128_len2048to8192_causal", "named", {}))
    return w


TIMED = {cls: _bucket_workloads(*cls) for cls in CANDIDATES}


def _cand4(cand):
    """Candidates recorded before the schedule field existed are single-group."""
    return tuple(cand) + (0,) * (4 - len(cand))


def _name(cls, cand):
    w, n, st, sched = _cand4(cand)
    return f"{cls[0]}_d{cls[1]}_w{w}_n{n}_s{st}" + {0: "", 1: "_pp", 2: "_rb2"}[sched]


def _lib_path(cls, cand):
    return os.path.join(SWEEP_DIR, f"libsdpa03_{_name(cls, cand)}.so")


def _resources(cls, cand):
    """(max VGPRs, spills, waves/SIMD) of the candidate's kernels for its class."""
    defs = _defines(cls, cand)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-c",
           *DEVICE_FLAGS, "-I", os.path.join(ROOT, "include"), "-x", "hip",
           os.path.join(CSRC, f"attn_fwd_{ {'bf16': 'bf16', 'fp16': 'f16', 'fp32': 'f32'}[cls[0]] }.hip"),
           "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", *defs]
    out = subprocess.run(cmd, capture_output=True, text=True).stderr
    dt_tag = {"bf16": "DF16b", "fp16": "DF16_", "fp32": "f"}[cls[0]]
    w, n, st, sched = _cand4(cand)
    rb = 2 if sched == 2 else 1
    want = (f"attn_fwd_pingpong_kernelI{dt_tag}Li{cls[1]}ELi{n}ELi{st}E" if sched == 1 else
            f"attn_fwd_kernelI{dt_tag}Li{cls[1]}ELi{w}ELi{rb}ELi{n}ELi{st}E")
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
    w, n, st, sched = _cand4(cand)
    return [f"-DSDPA03_SWEEP_DTYPE={DTYPE_CODES[cls[0]]}", f"-DSDPA03_SWEEP_HEAD_DIM={cls[1]}",
            f"-DSDPA03_SWEEP_WAVES={w}", f"-DSDPA03_SWEEP_BLOCK_N={n}",
            f"-DSDPA03_SWEEP_STAGES={st}", f"-DSDPA03_SWEEP_SCHEDULE={sched}"]


def build(only=None):
    """Compile the candidates (those whose name contains one of `only`, if given),
    two at a time (each build runs one compiler per source file)."""
    from concurrent.futures import ThreadPoolExecutor

    from .build import build_library

    os.makedirs(SWEEP_DIR, exist_ok=True)
    plan = []
    for cls, cands in CANDIDATES.items():
        for cand in cands:
            if only and not any(o in _name(cls, cand) for o in only):
                continue
            vg, sp, occ = _resources(cls, cand)
            ok = sp == 0 and occ >= 1
            print(f"{_name(cls, cand):28s} vgpr={vg} spill={sp} waves/simd={occ} "
                  f"{'build' if ok else 'skip'}", flush=True)
            if ok:
                plan.append((cls, cand))
    with ThreadPoolExecutor(max_workers=2) as pool:
        futs = [pool.submit(build_library, False, _lib_path(cls, cand), _defines(cls, cand))
                for cls, cand in plan]
        for f in futs:
            f.result()
    built = [{"dtype": cls[0], "head_dim": cls[1], "cand": list(cand)} for cls, cand in plan]
    with open(os.path.join(SWEEP_DIR, "built.json"), "w") as f:
        json.dump(built, f)
    print(f"built {len(built)} candidates", flush=True)


def _make_inputs(inputs, kind, kwargs, name):
    if kind == "named":
        return inputs.workload(name)
    if kind == "dense":
        return inputs.dense_inputs(**kwargs)
    return inputs.compact_inputs(**kwargs, causal_modes=(True,))


def _time_workload(binding, torch, inputs, spec, reps=10):
    name, kind, kwargs = spec
    x = _make_inputs(inputs, kind, kwargs, name)
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
        # Untimed sustained load first: the GPU raises its clocks only after
        # ~0.1 s of it, and inputs were just generated on the host.
        t_end = time.time() + 0.2
        n = 0
        while n < 3 or time.time() < t_end:
            call()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
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
    """Runs in a fresh process with SDPA03_LIBRARY set: prints JSON timings
    per bucket and workload."""
    import torch
    from . import binding, inputs
    binding.load_library(lib)
    cls = tuple(json.loads(os.environ["SDPA03_SWEEP_CLASS"]))
    res = {}
    for bucket, specs in TIMED.get(cls, {}).items():
        for spec in specs:
            res.setdefault(str(bucket), {})[spec[0]] = _time_workload(binding, torch, inputs, spec)
            print(f"   timed bucket {bucket} {spec[0]}", file=sys.stderr, flush=True)
    print("SWEEP_TIMINGS " + json.dumps(res), flush=True)


def run(only=None):
    """Parity, then timing, of the built candidates (those whose name contains
    one of `only`, if given: their results replace earlier ones of the same
    candidate in results.json, the others are kept)."""
    with open(os.path.join(SWEEP_DIR, "built.json")) as f:
        built = json.load(f)
    results = []
    if only and os.path.exists(RESULTS):
        with open(RESULTS) as f:
            results = json.load(f)
    for b in built:
        cls, cand = (b["dtype"], b["head_dim"]), _cand4(b["cand"])
        if cls not in TIMED:
            continue
        if only and not any(o in _name(cls, cand) for o in only):
            continue
        results = [r for r in results
                   if not ((r["dtype"], r["head_dim"]) == cls and _cand4(r["cand"]) == cand)]
        lib = _lib_path(cls, cand)
        env = dict(os.environ, SDPA03_LIBRARY=lib, SDPA03_SWEEP_CLASS=json.dumps(list(cls)))
        print(f"== {_name(cls, cand)}: parity", flush=True)
        t0 = time.time()
        try:
            par = subprocess.run([sys.executable, "-u", "-m", "pytest", "-x", "-q", "-m", "gpu",
                                  "--timeout", "300", "--timeout-method", "thread",
                                  os.path.join(ROOT, "tests", "test_gpu_parity.py")],
                                 cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
        except subprocess.TimeoutExpired as e:
            raise SweepFault(f"parity run of {_name(cls, cand)} exceeded 900 s") from e
        tail = par.stdout.strip().splitlines()[-1:] if par.stdout else []
        print(f"   parity rc={par.returncode} {tail} ({time.time() - t0:.0f} s)", flush=True)
        if child_faulted(par.returncode, par.stdout + par.stderr):
            print(par.stdout[-3000:] + par.stderr[-3000:], flush=True)
            raise SweepFault(f"parity run of {_name(cls, cand)} ended abnormally "
                             f"(rc {par.returncode}); no further candidate is run")
        entry = {"dtype": cls[0], "head_dim": cls[1], "cand": list(cand),
                 "parity": par.returncode == 0, "ms": None}
        if par.returncode == 0:
            try:
                tim = subprocess.run([sys.executable, "-u", "-c",
                                      "import sys; sys.path.insert(0, %r); "
                                      "from scaled_dot_product_03_amd import sweep; "
                                      "sweep._timing_child(%r)" % (ROOT, lib)],
                                     cwd=ROOT, env=env, capture_output=True, text=True,
                                     timeout=600)
            except subprocess.TimeoutExpired as e:
                raise SweepFault(f"timing of {_name(cls, cand)} exceeded 600 s") from e
            m = re.search(r"SWEEP_TIMINGS (.*)", tim.stdout)
            if tim.returncode != 0 or not m:
                raise SweepFault(f"timing of {_name(cls, cand)} failed (rc {tim.returncode}): "
                                 f"{tim.stderr[-2000:]}")
            entry["ms"] = json.loads(m.group(1))
            print(f"   ms {entry['ms']}", flush=True)
        else:
            print(par.stdout[-3000:], flush=True)
        results.append(entry)
        with open(RESULTS, "w") as f:
            json.dump(results, f, indent=1)


# Text that marks a child run as ended by the GPU or the runtime rather than
# by a failed comparison.
_FAULT_MARKS = ("Memory access fault", "GPU core dump", "hipError", "HIP error",
                "Segmentation fault", "Aborted", "core dumped", "Timeout", "timed out",
                "HSA_STATUS_ERROR")


def child_faulted(returncode, text):
    """True when a child process (a parity or timing run) ended by a signal, a
    time limit, a return code other than pytest's 0 (passed) and 1 (tests
    failed), or with fault text in its output: the sweep must stop there and
    launch no further GPU work.  Plain test failures are not faults."""
    if returncode is None or returncode < 0 or returncode not in (0, 1):
        return True
    return any(m in (text or "") for m in _FAULT_MARKS)


class SweepFault(RuntimeError):
    """A candidate's GPU run ended abnormally; the sweep stops."""


def _entry(cand):
    w, n, st, sched = cand
    return f"{{{w}, {n}, {st}, {sched}}}"


def write(results_path=RESULTS, table_path=TABLE):
    """Per (class, bucket): the passing candidate with the smallest score, the
    sum over that bucket's timed calls of its time divided by the best time
    any passing candidate reached on the call (so every workload counts
    alike, whatever its length).  Classes without timed workloads follow the
    timed class of the same head_dim."""
    with open(results_path) as f:
        results = json.load(f)
    passing = [r for r in results if r["parity"] and r["ms"]]
    fastest = {}  # (dtype, d, bucket, workload, call index) -> best ms
    for r in passing:
        for bucket, times in r["ms"].items():
            for name, calls in times.items():
                for i, t in enumerate(calls):
                    k = (r["dtype"], r["head_dim"], int(bucket), name, i)
                    fastest[k] = min(fastest.get(k, t), t)
    best = {}  # (dtype, d, bucket) -> (score, cand)
    for r in passing:
        for bucket, times in r["ms"].items():
            key = (r["dtype"], r["head_dim"], int(bucket))
            score = sum(t / fastest[key + (name, i)]
                        for name, calls in times.items() for i, t in enumerate(calls))
            if key not in best or score < best[key][0]:
                best[key] = (score, _cand4(r["cand"]))
    default = {128: (4, 64, 2, 0), 64: (4, 64, 3, 0)}
    timed_class = {128: "bf16", 64: "fp16"}
    pick = {}
    for dt in ("bf16", "fp16"):
        for d in (128, 64):
            for b in range(len(BUCKETS)):
                src = (dt, d, b) if (dt, d, b) in best else (timed_class[d], d, b)
                pick[(dt, d, b)] = best[src][1] if src in best else default[d]
    lines = ["  // BEGIN TABLE (generated)",
             "  // buckets: " + ", ".join(f"({b})" for b in BUCKETS)]
    for (dt, d, b), (score, cand) in sorted(best.items()):
        n_calls = sum(1 for k in fastest if k[:3] == (dt, d, b))
        lines.append(f"  // {dt} d{d} bucket {b}: (waves, block_n, stages, schedule) = {cand}; "
                     f"score {score:.3f} over {n_calls} timed calls (1 per call is best)")
    lines += ["  if constexpr (sizeof(T) == 4) {", "    return TableEntry{4, 32, 2, 0};"]
    for dt in ("bf16", "fp16"):
        for d in (128, 64):
            cond = f"dtype_code<T>() == {'DT_BF16' if dt == 'bf16' else 'DT_F16'} && D == {d}"
            ents = [_entry(pick[(dt, d, b)]) for b in range(len(BUCKETS))]
            lines += [f"  }} else if constexpr ({cond}) {{",
                      "    constexpr TableEntry e[kSeqBuckets] = {" + ", ".join(ents[:3]) + ",",
                      "                                           " + ", ".join(ents[3:]) + "};",
                      "    return e[BUCKET];"]
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
    elif sys.argv[1] == "run":
        run(sys.argv[2:] or None)
    else:
        write()
