"""Helpers for comparing the HIP library with the float64 oracle."""

import numpy as np
import torch

# max |dO|, mean |dO| per input dtype, and max |dLSE| (all dtypes).
O_TOL = {"fp32": (1e-4, 1e-4), "fp16": (2e-2, 2e-3), "bf16": (2e-2, 2e-3)}
LSE_TOL = 1e-3


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label=""):
    """Element-wise comparison over all given entries; returns the stats."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert lse_gpu.shape == lse_ref.shape, (lse_gpu.shape, lse_ref.shape)
    assert np.isfinite(o_gpu).all(), f"{label}: non-finite O"
    d = np.abs(o_gpu - o_ref)
    both_inf = np.isneginf(lse_gpu) & np.isneginf(lse_ref)
    with np.errstate(invalid="ignore"):
        dl = np.where(both_inf, 0.0, np.abs(lse_gpu - lse_ref))
    stats = dict(max_o=float(d.max(initial=0.0)), mean_o=float(d.mean()) if d.size else 0.0,
                 max_lse=float(dl.max(initial=0.0)))
    max_tol, mean_tol = O_TOL[dtype]
    assert stats["max_o"] <= max_tol, f"{label}: max|dO| {stats['max_o']:.3e} > {max_tol}"
    assert stats["mean_o"] <= mean_tol, f"{label}: mean|dO| {stats['mean_o']:.3e} > {mean_tol}"
    assert stats["max_lse"] <= LSE_TOL, f"{label}: max|dLSE| {stats['max_lse']:.3e} > {LSE_TOL}"
    return stats


def sample_rows(length, rng, tile=128, extra=12):
    """Rows at tile edges, the ends, and a few random ones (unique, sorted)."""
    cand = {0, 1, length - 1, length - 2}
    for t in range(tile, length, tile * 3):
        cand.update({t - 1, t, t + 1})
    cand.update(rng.integers(0, length, size=extra).tolist())
    return np.array(sorted(r for r in cand if 0 <= r < length), dtype=np.int64)
