"""Offline sweep that writes the compiled-in dispatch table.

The dispatch key is (dtype, head_dim, sequence-length bucket, variant): four
query buckets (<= 128, <= 512, <= 4096, longer) by two key buckets (<= 512,
longer), and four variants (dense without mask, dense causal,
variable-length without mask, variable-length causal).  AOTriton's tuning
database probes sequence lengths, head dim and dtype (AOTriton issue #12,
the maintainer's replies); the mask and layout join the key here because
they change the work per query tile.

For every class (dtype, head_dim) a set of candidate kernel shapes (waves
per workgroup, keys per tile, LDS stages, schedule: 0 single group, 1
ping-pong of two wave groups, 2 single group with two 32-row blocks per wave,
3 the lagged schedule, 4 single group at three waves per SIMD) is compiled
into its own build of libsdpa03.so, the shape applied to every bucket and
variant of the class.  A candidate counts only if its build has no register
spills, and then passes the GPU parity tests (tests/test_gpu_parity.py,
test_gpu_splitk.py and test_gpu_bias.py at their small shapes, run against
that build): the same page warns that a kernel built with some
configurations runs but gives wrong results.  Only then is it timed, on at
least two workloads of every bucket for the dense variants (both masks) and
on variable-length workloads of every bucket.  Per (bucket, variant), the
passing candidate with the lowest score on that bucket's calls of that
variant (its time over the best time any candidate reached on the call,
summed) goes into csrc/dispatch_table.inc.  There is no tuning at run time.

    python -m scaled_dot_product_03_amd.sweep build [name ...]  # CPU: compile candidates
    python -m scaled_dot_product_03_amd.sweep run [name ...]    # GPU: parity, then timing
    python -m scaled_dot_product_03_amd.sweep write   # rewrite the table and its summary

`run` writes _sweep/results.json; `write` reads it and also writes the
per-entry summary profiles/dispatch_sweep_attn_fwd_every_class.md.
"""

from __future__ import annotations

import hashlib
import json
import os
import re
import subprocess
import sys
import time

from .build import ARCH, CSRC, HIPCC, ROOT, SOURCES, object_command

SWEEP_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_sweep")
RESULTS = os.path.join(SWEEP_DIR, "results.json")
TABLE = os.path.join(CSRC, "dispatch_table.inc")
SUMMARY = os.path.join(ROOT, "profiles", "dispatch_sweep_attn_fwd_every_class.md")
DTYPE_CODES = {"fp32": 0, "fp16": 1, "bf16": 2}
TU_OF = {"bf16": "attn_fwd_bf16.hip", "fp16": "attn_fwd_f16.hip", "fp32": "attn_fwd_f32.hip"}
SCHED_TAG = {0: "", 1: "_pp", 2: "_rb2", 3: "_lag", 4: "_3w"}

CLASSES = [("bf16", 128), ("fp16", 128), ("bf16", 64), ("fp16", 64), ("fp32", 64), ("fp32", 128)]

# Candidate (waves, block_n, stages, schedule) per class.
CANDIDATES = {
    ("bf16", 128): [(4, 32, 2, 0), (4, 64, 2, 0), (4, 32, 3, 0), (2, 32, 2, 0), (8, 64, 2, 0),
                    (8, 64, 3, 0), (4, 32, 2, 4), (8, 64, 3, 1), (4, 32, 3, 2)],
    ("fp16", 128): [(4, 32, 2, 0), (4, 64, 2, 0), (4, 32, 3, 0), (8, 64, 2, 0), (4, 32, 2, 4),
                    (8, 64, 3, 1)],
    ("bf16", 64): [(4, 32, 2, 0), (4, 64, 2, 0), (4, 64, 3, 0), (4, 64, 2, 4), (8, 128, 2, 1),
                   (4, 32, 3, 3)],
    ("fp16", 64): [(4, 32, 2, 0), (4, 64, 2, 0), (4, 64, 3, 0), (2, 32, 2, 0), (8, 64, 3, 0),
                   (4, 32, 2, 4), (4, 64, 2, 4), (8, 128, 2, 1), (4, 32, 3, 3), (4, 64, 3, 2)],
    ("fp32", 64): [(4, 32, 2, 0), (4, 64, 2, 0), (2, 32, 2, 0), (8, 32, 2, 0)],
    ("fp32", 128): [(4, 32, 2, 0), (4, 64, 2, 0), (2, 32, 2, 0), (8, 32, 2, 0)],
}
# The entry of a class before any sweep (and for keys no timing reaches).
DEFAULT = (4, 64, 2, 0)

BUCKETS = ["q<=128,k<=512", "q<=128,k>512", "q<=512,k<=512", "q<=512,k>512",
           "q<=4096,k<=512", "q<=4096,k>512", "q>4096,k<=512", "q>4096,k>512"]
VARIANTS = ["dense", "dense causal", "varlen", "varlen causal"]


def variant_of(mode: str, causal: bool) -> int:
    return (2 if mode != "dense" else 0) + (1 if causal else 0)


def _bucket_workloads(dtype, d):
    """Timed workloads per bucket: (name, kind, kwargs).  Every bucket has two
    dense shapes, each timed with both masks, and variable-length workloads
    whose longest sequence falls in the bucket (compact THD; for bf16 head
    dim 128 also the bench's compact THD workload in its bucket and its padded
    workload in the longest one).  The
    named workloads sit in their buckets; the others are seeded synthetic
    shapes of the same recipe (inputs.py)."""
    def dense(B, H, Sq, Sk):
        return (f"dense_{dtype}_b{B}h{H}sq{Sq}sk{Sk}d{d}", "dense",
                dict(B=B, H=H, Sq=Sq, Sk=Sk, D=d, dtype=dtype, seed=11,
                     causal_modes=(False, True)))

    def thd(n, q_lo, q_hi, k_lo=None, k_hi=None, H=16):
        same = k_lo is None
        name = (f"thd_{dtype}_{n}seq_q{q_lo}to{q_hi}" + ("" if same else f"_k{k_lo}to{k_hi}")
                + f"_h{H}d{d}")
        return (name, "compact", dict(n_seqs=n, H=H, D=d, dtype=dtype, seed=12, len_lo=q_lo,
                                      len_hi=q_hi, k_lo=k_lo, k_hi=k_hi))

    w = {
        0: [dense(128, 16, 64, 64), dense(64, 16, 128, 128), thd(256, 1, 128)],
        1: [dense(16, 16, 128, 4096), dense(32, 16, 64, 2048), thd(64, 1, 128, 1000, 4000)],
        2: [dense(16, 16, 256, 256), dense(8, 16, 512, 512), thd(128, 129, 256),
            thd(64, 1, 512)],
        3: [dense(2, 32, 512, 8192), dense(8, 16, 384, 2048), thd(32, 129, 512, 2000, 8000)],
        4: [dense(4, 16, 2048, 512), dense(2, 16, 4096, 256), thd(16, 600, 4000, 1, 512)],
        5: [dense(4, 16, 2048, 2048), dense(1, 16, 4096, 4096), thd(16, 1, 4096)],
        6: [dense(1, 16, 8192, 512), dense(1, 8, 16384, 256), thd(4, 4200, 8192, 1, 512)],
        7: [dense(1, 16, 8192, 8192), dense(2, 8, 6144, 6144), thd(4, 4200, 8192)],
    }
    if (dtype, d) == ("bf16", 128):
        w[5].append(("thd_bf16_16seq_len1to4096_h16d128_causal", "named", {}))
        w[7].append(("padded_bf16_b8h32smax8192d128_len2048to8192_causal", "named", {}))
    return w


TIMED = {cls: _bucket_workloads(*cls) for cls in CLASSES}


def _cand4(cand):
    """Candidates recorded before the schedule field existed are single-group."""
    return tuple(cand) + (0,) * (4 - len(cand))


def _name(cls, cand):
    w, n, st, sched = _cand4(cand)
    return f"{cls[0]}_d{cls[1]}_w{w}_n{n}_s{st}" + SCHED_TAG[sched]


def _lib_path(cls, cand):
    return os.path.join(SWEEP_DIR, f"libsdpa03_{_name(cls, cand)}.so")


def _defines(cls, cand):
    w, n, st, sched = _cand4(cand)
    return [f"-DSDPA03_SWEEP_DTYPE={DTYPE_CODES[cls[0]]}", f"-DSDPA03_SWEEP_HEAD_DIM={cls[1]}",
            f"-DSDPA03_SWEEP_WAVES={w}", f"-DSDPA03_SWEEP_BLOCK_N={n}",
            f"-DSDPA03_SWEEP_STAGES={st}", f"-DSDPA03_SWEEP_SCHEDULE={sched}"]


def _kernel_prefix(cls, cand):
    """Mangled-name prefix of the candidate's forward kernels."""
    dt_tag = {"bf16": "DF16b", "fp16": "DF16_", "fp32": "f"}[cls[0]]
    w, n, st, sched = _cand4(cand)
    d = cls[1]
    if sched == 1:
        return f"attn_fwd_pingpong_kernelI{dt_tag}Li{d}ELi{n}ELi{st}E"
    if sched == 3:
        return f"attn_fwd_lagged_kernelI{dt_tag}Li{d}ELi{w}ELi{n}ELi{st}E"
    if sched == 4:
        return f"attn_fwd_3w_kernelI{dt_tag}Li{d}ELi{w}ELi{n}ELi{st}E"
    rb = 2 if sched == 2 else 1
    return f"attn_fwd_kernelI{dt_tag}Li{d}ELi{w}ELi{rb}ELi{n}ELi{st}E"


# Spilled registers the forward with a bias may have (its bias tile adds 16
# registers to the kernel; a couple of spills there cost less than a shape
# the other kernels cannot use).
BIAS_SPILL_LIMIT = 8


def _resources(cls, cand):
    """(max VGPRs, spills of the kernels without a bias, spills of those with
    one, waves/SIMD) of the candidate's forward kernels for its class."""
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-c",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-x", "hip", os.path.join(CSRC, TU_OF[cls[0]]),
           "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage", *_defines(cls, cand)]
    out = subprocess.run(cmd, capture_output=True, text=True).stderr
    want = _kernel_prefix(cls, cand)
    vg, sp, sp_bias, occ, cur = 0, 0, 0, 99, None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            continue
        if cur is None or want not in cur:
            continue
        # the bias flag is the last template argument of every forward kernel
        bias = cur.endswith("ELb1EEEvNS_7FwdArgsE")
        m = re.search(r"remark:\s+(VGPRs|VGPRs Spill|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m:
            val = int(m.group(2))
            if m.group(1) == "VGPRs":
                vg = max(vg, val)
            elif m.group(1) == "VGPRs Spill":
                if bias:
                    sp_bias = max(sp_bias, val)
                else:
                    sp = max(sp, val)
            elif not bias:
                occ = min(occ, val)
    if occ == 99:
        raise RuntimeError(f"no kernel {want} in the resource report of {_name(cls, cand)}")
    return vg, sp, sp_bias, occ


def _source_digest():
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    with open(os.path.join(ROOT, "include", "sdpa03.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def _build_candidate(cls, cand, cache):
    """Links the candidate's library from cached objects: only the units that
    read the table with the candidate's defines (the dispatch unit and the
    class's element type) are compiled per candidate."""
    digest = _source_digest()
    objs = []
    for src in SOURCES:
        defs = _defines(cls, cand) if src in ("attn_fwd.hip", TU_OF[cls[0]]) else []
        key = hashlib.sha256((digest + src + " ".join(defs)).encode()).hexdigest()[:20]
        obj = os.path.join(cache, f"{src}.{key}.o")
        if not os.path.exists(obj):
            res = subprocess.run(object_command(src, obj + ".tmp", defs), capture_output=True,
                                 text=True)
            if res.returncode != 0:
                raise RuntimeError(f"{_name(cls, cand)}: {src} failed\n{res.stderr[-3000:]}")
            os.replace(obj + ".tmp", obj)
        objs.append(obj)
    lib = _lib_path(cls, cand)
    res = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o",
                          lib + ".tmp"], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(res.stderr[-3000:])
    os.replace(lib + ".tmp", lib)
    return lib


def build(only=None):
    """Compile the candidates (those whose name contains one of `only`, if
    given), four at a time."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(SWEEP_DIR, exist_ok=True)
    cache = os.path.join(SWEEP_DIR, "objcache")
    os.makedirs(cache, exist_ok=True)
    plan, skipped = [], []
    todo = [(cls, cand) for cls in CLASSES for cand in CANDIDATES[cls]
            if not only or any(o in _name(cls, cand) for o in only)]
    with ThreadPoolExecutor(max_workers=6) as pool:
        res = list(pool.map(lambda cc: _resources(*cc), todo))
    for (cls, cand), (vg, sp, sp_bias, occ) in zip(todo, res):
        ok = sp == 0 and sp_bias <= BIAS_SPILL_LIMIT and occ >= 1
        print(f"{_name(cls, cand):30s} vgpr={vg} spill={sp} bias-kernel spill={sp_bias} "
              f"waves/simd={occ} {'build' if ok else 'skip'}", flush=True)
        rec = {"dtype": cls[0], "head_dim": cls[1], "cand": list(_cand4(cand)), "vgpr": vg,
               "spill": sp, "bias_spill": sp_bias, "waves_per_simd": occ}
        (plan if ok else skipped).append(rec)
    # the units shared by every candidate first, then the candidates in parallel
    if plan:
        first = plan[0]
        _build_candidate((first["dtype"], first["head_dim"]), first["cand"], cache)
    with ThreadPoolExecutor(max_workers=4) as pool:
        futs = [pool.submit(_build_candidate, (r["dtype"], r["head_dim"]), r["cand"], cache)
                for r in plan[1:]]
        for f in futs:
            f.result()
    path = os.path.join(SWEEP_DIR, "built.json")
    old = json.load(open(path)) if (only and os.path.exists(path)) else []
    # records of schedules this source no longer has are dropped
    old = [r for r in old if _cand4(r["cand"])[3] in SCHED_TAG]
    keep = [r for r in old if not any(o in _name((r["dtype"], r["head_dim"]), r["cand"])
                                      for o in (only or []))]
    with open(path, "w") as f:
        json.dump(keep + plan + [dict(r, skipped=True) for r in skipped], f, indent=1)
    print(f"built {len(plan)} candidates, skipped {len(skipped)} (spills)", flush=True)


def _make_inputs(inputs, kind, kwargs, name):
    if kind == "named":
        return inputs.workload(name)
    if kind == "dense":
        return inputs.dense_inputs(**kwargs)
    kw = dict(kwargs)
    k_lo, k_hi = kw.pop("k_lo"), kw.pop("k_hi")
    if k_lo is None:
        return inputs.compact_inputs(**kw, causal_modes=(False, True))
    import numpy as np
    rng = np.random.default_rng(kw["seed"] + 1)
    lq = rng.integers(kw["len_lo"], kw["len_hi"], size=kw["n_seqs"], endpoint=True)
    lk = rng.integers(k_lo, k_hi, size=kw["n_seqs"], endpoint=True)
    return inputs.compact_inputs(**kw, lengths_q=lq, lengths_k=lk, causal_modes=(False, True))


def _time_workload(binding, torch, inputs, spec, reps=10):
    """{variant: ms} of one workload (each of its masks)."""
    name, kind, kwargs = spec
    x = _make_inputs(inputs, kind, kwargs, name)
    dev = torch.device("cuda:0")
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    calls = {}
    if x.mode == "dense":
        for causal in x.causal_modes:
            calls[variant_of("dense", causal)] = (
                lambda c=causal: binding.attn_fwd(q, k, v, scale=x.scale, causal=c))
    elif x.mode == "compact":
        cq = torch.from_numpy(x.cu_seqlens_q).to(dev)
        ck = torch.from_numpy(x.cu_seqlens_k).to(dev)
        mq, mk = int(max(x.meta["lengths_q"])), int(max(x.meta["lengths_k"]))
        for causal in x.causal_modes:
            calls[variant_of("compact", causal)] = (
                lambda c=causal: binding.attn_fwd_compact_varlen(q, k, v, cq, ck, mq, mk,
                                                                 scale=x.scale, causal=c))
    else:
        cu = torch.from_numpy(x.cu_seqlens_q).to(dev)
        calls[variant_of("padded", True)] = (
            lambda: binding.attn_fwd_padded_varlen(q, k, v, cu, cu, scale=x.scale, causal=True))
    out = {}
    for var, call in calls.items():
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
        out[str(var)] = e0.elapsed_time(e1) / reps
    return out


def _timing_child(lib):
    """Runs in a fresh process with SDPA03_LIBRARY set: prints JSON timings
    per bucket, workload and variant."""
    import torch
    from . import binding, inputs
    binding.load_library(lib)
    cls = tuple(json.loads(os.environ["SDPA03_SWEEP_CLASS"]))
    res = {}
    for bucket, specs in TIMED.get(cls, {}).items():
        for spec in specs:
            res.setdefault(str(bucket), {})[spec[0]] = _time_workload(binding, torch, inputs,
                                                                      spec)
            print(f"   timed bucket {bucket} {spec[0]}", file=sys.stderr, flush=True)
    print("SWEEP_TIMINGS " + json.dumps(res), flush=True)


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


PARITY_TESTS = ["tests/test_gpu_parity.py", "tests/test_gpu_splitk.py", "tests/test_gpu_bias.py"]
PARITY_FILTER = "not workload and not s2048"


def run(only=None):
    """Parity, then timing, of the built candidates (those whose name contains
    one of `only`, if given: their results replace earlier ones of the same
    candidate in results.json, the others are kept)."""
    with open(os.path.join(SWEEP_DIR, "built.json")) as f:
        records = json.load(f)
    built = [b for b in records if not b.get("skipped")]
    results = []
    if os.path.exists(RESULTS):
        with open(RESULTS) as f:
            results = json.load(f)
    # A candidate the last build skipped (it spills with the current source)
    # keeps no timing from an earlier source.
    skipped = {((b["dtype"], b["head_dim"]), _cand4(b["cand"])) for b in records
               if b.get("skipped")}
    results = [r for r in results
               if ((r["dtype"], r["head_dim"]), _cand4(r["cand"])) not in skipped]
    for b in built:
        cls, cand = (b["dtype"], b["head_dim"]), _cand4(b["cand"])
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
                                  "-k", PARITY_FILTER,
                                  *[os.path.join(ROOT, t) for t in PARITY_TESTS]],
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
                 "parity": par.returncode == 0, "parity_summary": tail[0] if tail else "",
                 "ms": None, "vgpr": b.get("vgpr"), "waves_per_simd": b.get("waves_per_simd")}
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
            print(f"   timed in {time.time() - t0:.0f} s", flush=True)
        else:
            print(par.stdout[-3000:], flush=True)
        results.append(entry)
        with open(RESULTS, "w") as f:
            json.dump(results, f, indent=1)


# When a (bucket, variant) has no timed call, the entry follows the first
# variant in this list that has one (the variable-length variants fall back
# to the dense ones of the same mask, then to dense without the mask).
FALLBACK = {0: [], 1: [0], 2: [0], 3: [1, 0]}


def select(results):
    """Per (dtype, d, bucket, variant): (candidate, score, calls, runner-up)
    among the candidates that passed parity, from their timings.  The score is
    the sum over the key's timed calls of the candidate's time over the best
    time any passing candidate reached on that call.  A candidate competes
    for a key only if it was timed on every call of that key."""
    passing = [r for r in results if r["parity"] and r["ms"]]
    fastest = {}
    for r in passing:
        for bucket, per_wl in r["ms"].items():
            for wl, per_var in per_wl.items():
                for var, t in per_var.items():
                    k = (r["dtype"], r["head_dim"], int(bucket), int(var), wl)
                    fastest[k] = min(fastest.get(k, t), t)
    calls_of = {}
    for k in fastest:
        calls_of.setdefault(k[:4], set()).add(k[4])
    scores = {}
    for r in passing:
        acc = {}
        for bucket, per_wl in r["ms"].items():
            for wl, per_var in per_wl.items():
                for var, t in per_var.items():
                    key = (r["dtype"], r["head_dim"], int(bucket), int(var))
                    s, n, seen = acc.get(key, (0.0, 0, frozenset()))
                    acc[key] = (s + t / fastest[key + (wl,)], n + 1, seen | {wl})
        for key, (s, n, seen) in acc.items():
            if seen == calls_of[key]:
                scores.setdefault(key, []).append((s, n, _cand4(r["cand"])))
    best = {}
    for key, lst in scores.items():
        lst.sort()
        best[key] = (lst[0][2], lst[0][0], lst[0][1], lst[1] if len(lst) > 1 else None)
    pick = {}
    for dt, d in CLASSES:
        for b in range(len(BUCKETS)):
            for v in range(len(VARIANTS)):
                src = next(((dt, d, b, w) for w in [v] + FALLBACK[v] if (dt, d, b, w) in best),
                           None)
                pick[(dt, d, b, v)] = (best[src][0] if src else DEFAULT, src)
    return pick, best


def _entry(cand):
    w, n, st, sched = cand
    return f"{{{w}, {n}, {st}, {sched}}}"


def _cond(dt, d):
    return f"dtype_code<T>() == {dict(bf16='DT_BF16', fp16='DT_F16', fp32='DT_F32')[dt]} && D == {d}"


def write(results_path=RESULTS, table_path=TABLE, summary_path=SUMMARY):
    """Rewrites the generated part of dispatch_table.inc from the sweep's
    results and the per-entry summary; returns {(dtype, d, bucket, variant):
    candidate}."""
    with open(results_path) as f:
        results = json.load(f)
    pick, best = select(results)
    lines = ["  // BEGIN TABLE (generated)",
             "  // per class: [bucket][variant]; buckets " + ", ".join(f"({b})" for b in BUCKETS),
             "  // variants: " + ", ".join(f"{i} {v}" for i, v in enumerate(VARIANTS))]
    first = True
    for dt, d in CLASSES:
        opener = "if" if first else "} else if"
        lines.append(f"  {opener} constexpr ({_cond(dt, d)}) {{")
        first = False
        lines.append("    constexpr TableEntry e[kSeqBuckets][kVariants] = {")
        for b in range(len(BUCKETS)):
            ents = ", ".join(_entry(pick[(dt, d, b, v)][0]) for v in range(len(VARIANTS)))
            lines.append(f"        {{{ents}}}{',' if b + 1 < len(BUCKETS) else '};'}")
        lines.append("    return e[BUCKET][VARIANT];")
    lines += ["  } else {", f"    return TableEntry{_entry(DEFAULT)};", "  }", "  // END TABLE"]
    text = open(table_path).read()
    text = re.sub(r"  // BEGIN TABLE \(generated\).*  // END TABLE", lambda _: "\n".join(lines),
                  text, flags=re.S)
    with open(table_path, "w") as f:
        f.write(text)
    if summary_path:
        write_summary(results, pick, best, summary_path)
    return {k: v[0] for k, v in pick.items()}


def write_summary(results, pick, best, path):
    """The committed trace of every table entry: each candidate's resources,
    parity outcome and time per workload and variant, and per key the chosen
    candidate, its score, the number of timed calls and the runner-up."""
    out = ["# Dispatch-table sweep: every class of the attention forward", "",
           "Written by `python -m scaled_dot_product_03_amd.sweep write` from the results of "
           "`python -m scaled_dot_product_03_amd.sweep build` (CPU) and `... sweep run` (one "
           "MI355X).  Candidates: (waves, block_n, stages, schedule) with schedule 0 single "
           "group, 1 ping-pong, 2 two row blocks per wave, 3 lagged P.V, 4 three waves per SIMD, "
           "'-' marks a call a candidate was not timed on.  A four-wave single-group candidate "
           "runs as two key groups on grids of at most 256 workgroups.  Times in microseconds, the mean of 10 back-to-back calls after 0.2 s of untimed "
           "calls.  Score = sum over the key's calls of time / best time among passing "
           "candidates (1.000 per call is best).", ""]
    for dt, d in CLASSES:
        rs = [r for r in results if (r["dtype"], r["head_dim"]) == (dt, d)]
        if not rs:
            continue
        out += [f"## {dt}, head_dim {d}", "", "| candidate | VGPRs | waves/SIMD | parity |",
                "|---|---|---|---|"]
        for r in rs:
            out.append(f"| {tuple(_cand4(r['cand']))} | {r.get('vgpr', '')} | "
                       f"{r.get('waves_per_simd', '')} | "
                       f"{'pass' if r['parity'] else 'FAIL'} {r.get('parity_summary', '')} |")
        cands = [r for r in rs if r["parity"] and r["ms"]]
        out += ["", "| bucket | workload | variant | " +
                " | ".join(str(tuple(_cand4(r["cand"]))) for r in cands) + " |",
                "|---|---|---|" + "---|" * len(cands)]
        for b in range(len(BUCKETS)):
            wls = sorted({(wl, var) for r in cands for wl, pv in r["ms"].get(str(b), {}).items()
                          for var in pv})
            for wl, var in wls:
                ts = [r["ms"].get(str(b), {}).get(wl, {}).get(var) for r in cands]
                out.append(f"| {b} | {wl} | {VARIANTS[int(var)]} | " +
                           " | ".join("-" if t is None else f"{t * 1e3:.1f}" for t in ts) + " |")
        out += ["", "| bucket | variant | entry | from | score | timed calls | runner-up |",
                "|---|---|---|---|---|---|---|"]
        for b in range(len(BUCKETS)):
            for v in range(len(VARIANTS)):
                cand, src = pick[(dt, d, b, v)]
                if src is None:
                    out.append(f"| {b} | {VARIANTS[v]} | {cand} | default (no timing) | | | |")
                    continue
                c, score, n, ru = best[src]
                frm = "own timings" if src[3] == v else f"variant {VARIANTS[src[3]]}"
                ru_s = f"{ru[2]} ({ru[0]:.3f})" if ru else ""
                out.append(f"| {b} | {VARIANTS[v]} | {cand} | {frm} | {score:.3f} | {n} | "
                           f"{ru_s} |")
        out.append("")
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(f"wrote {path}", flush=True)


if __name__ == "__main__":
    if sys.argv[1] == "build":
        build(sys.argv[2:] or None)
    elif sys.argv[1] == "run":
        run(sys.argv[2:] or None)
    else:
        write()
