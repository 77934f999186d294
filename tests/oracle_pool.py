"""The float64 oracle over every (batch or sequence, head) of a full-size
workload, in a pool of host processes, compared with the GPU's outputs.

The parent (a test that has run the library on the GPU) writes the inputs
and the GPU's O and LSE as .npy files into a temporary directory (bf16 as
its raw 16-bit patterns, fp16 and float32 as they are); each worker
memory-maps them, widens the slices it needs exactly to float64,
runs ``oracle.attention_head`` on one (batch or sequence, head) and returns
the error sums and maxima of that head, so only a few numbers travel back.
Workers are started with the ``spawn`` method: fresh interpreters that never
touch the GPU.  Each uses one BLAS thread.
"""

from __future__ import annotations

import multiprocessing
import os
import shutil
import tempfile
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

# Box processes (16 CPUs per GPU there); this container has fewer.
MAX_WORKERS = 16


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _save(d, name, a):
    """Writes one array; bf16 goes as raw uint16 patterns with a marker."""
    import torch
    if isinstance(a, torch.Tensor):
        a = a.detach().to("cpu")
        if a.dtype == torch.bfloat16:
            np.save(os.path.join(d, f"{name}.bf16.npy"), a.contiguous().view(torch.int16).numpy())
            return
        a = a.numpy()
    np.save(os.path.join(d, f"{name}.npy"), np.ascontiguousarray(a))


def _load(d, name):
    p = os.path.join(d, f"{name}.bf16.npy")
    if os.path.exists(p):
        return np.load(p, mmap_mode="r"), True
    return np.load(os.path.join(d, f"{name}.npy"), mmap_mode="r"), False


def _wide(arr_flag, sl):
    """float64 copy of arr[sl]; bf16 patterns shifted into float32's high half."""
    arr, bf16 = arr_flag
    x = np.asarray(arr[sl])
    if bf16:
        x = (x.astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float64)


def _head(task):
    """(sum |dO|, max |dO|, max |dLSE|, elements, all finite) of one head."""
    from oracle import attention_head

    d, kind, idx, scale, causal = task
    q, k, v, o, lse = (_load(d, n) for n in ("q", "k", "v", "o", "lse"))
    if kind == "dense":
        b, h = idx
        sl = (b, h)
        sl_lse = (b, h)
    elif kind == "compact":
        h, s, e = idx
        sl = (slice(s, e), h)
        sl_lse = (0, h, slice(s, e))
    else:
        b, h, L = idx
        sl = (b, h, slice(0, L))
        sl_lse = (b, h, slice(0, L))
    ro, rl = attention_head(_wide(q, sl), _wide(k, sl), _wide(v, sl), scale, causal)
    go = _wide(o, sl)
    gl = _wide(lse, sl_lse)
    finite = bool(np.isfinite(go).all() and np.isfinite(gl).all())
    do = np.abs(go - ro)
    dl = np.abs(gl - rl)
    return float(do.sum()), float(do.max(initial=0.0)), float(dl.max(initial=0.0)), do.size, finite


def compare_all_heads(kind, arrays, tasks, scale, causal):
    """Runs the oracle on every task's head against the GPU outputs in
    ``arrays`` (q, k, v, o, lse as torch or numpy arrays).  Returns
    {max_o, mean_o, max_lse, elements, all_finite, workers, oracle_s}."""
    d = tempfile.mkdtemp(prefix="sdpa03_oracle_")
    try:
        for name, a in arrays.items():
            _save(d, name, a)
        workers = max(1, min(MAX_WORKERS, os.cpu_count() or 1, len(tasks)))
        t0 = time.perf_counter()
        with ProcessPoolExecutor(max_workers=workers, initializer=_worker_init,
                                 mp_context=multiprocessing.get_context("spawn")) as pool:
            res = list(pool.map(_head, [(d, kind, t, scale, causal) for t in tasks],
                                chunksize=1))
        dt = time.perf_counter() - t0
    finally:
        shutil.rmtree(d, ignore_errors=True)
    n = sum(r[3] for r in res)
    return {"max_o": max(r[1] for r in res), "mean_o": sum(r[0] for r in res) / max(n, 1),
            "max_lse": max(r[2] for r in res), "elements": n,
            "all_finite": all(r[4] for r in res), "workers": workers, "oracle_s": dt}
