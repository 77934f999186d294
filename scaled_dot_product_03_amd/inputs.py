"""Seeded synthetic inputs shared by the tests, the bench and the CPU oracle.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both sides of every parity check (the HIP library and
the float64 oracle) receive the same tensors from here.

Recipe (one ``numpy.random.default_rng(seed)``, a PCG64 stream, per input set):

1. variable-length workloads draw their lengths first, with
   ``rng.integers(lo, hi, size=n, endpoint=True)`` (both ends inclusive);
2. then Q, K and V, in that order, each with
   ``rng.standard_normal(shape, dtype=float32)`` over the full tensor,
   padding included;
3. each is rounded to the target dtype with round-to-nearest-even
   (``torch.Tensor.to``).

The five named workloads are the ones the flash-attention forward is checked
and measured on; their sizes are spelt out in ``WORKLOADS``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class AttnInputs:
    """One seeded input set.  Tensors are host (CPU) tensors in ``dtype``."""

    mode: str  # "dense" | "compact" | "padded"
    dtype: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    scale: float
    causal_modes: tuple
    cu_seqlens_q: np.ndarray | None = None
    cu_seqlens_k: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[-1])


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim), rounded to the float32 value the library receives."""
    return float(np.float32(1.0 / np.sqrt(np.float64(head_dim))))


def _draw(rng, shape, dtype: str) -> torch.Tensor:
    x = rng.standard_normal(shape, dtype=np.float32)
    return torch.from_numpy(x).to(DTYPES[dtype])


def cu_from_lengths(lengths) -> np.ndarray:
    """int32 exclusive prefix sums with a leading 0 (length n+1)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("token count does not fit int32")
    return cu.astype(np.int32)


def dense_inputs(B, H, Sq, Sk, D, dtype, seed, scale=None, causal_modes=(False, True)):
    """BHSD contiguous Q (B,H,Sq,D) and K, V (B,H,Sk,D)."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, H, Sq, D), dtype)
    k = _draw(rng, (B, H, Sk, D), dtype)
    v = _draw(rng, (B, H, Sk, D), dtype)
    return AttnInputs(
        "dense", dtype, q, k, v,
        default_scale(D) if scale is None else float(np.float32(scale)),
        tuple(causal_modes),
        meta=dict(B=B, H=H, Sq=Sq, Sk=Sk, D=D, seed=seed),
    )


def bias_tensor(shape, dtype, seed, neg_inf_frac=0.0, key_pad=8):
    """A seeded standard-normal additive bias of ``shape`` (rank 4), stored
    with its last dimension padded to a multiple of ``key_pad`` elements (the
    library needs row strides in multiples of 4) and returned as the
    unpadded view.  ``neg_inf_frac`` of the entries become -inf."""
    rng = np.random.default_rng(seed)
    *lead, sk = shape
    padded = (sk + key_pad - 1) // key_pad * key_pad if sk else key_pad
    x = rng.standard_normal((*lead, padded), dtype=np.float32)
    if neg_inf_frac > 0:
        x[rng.random(x.shape) < neg_inf_frac] = -np.inf
    return torch.from_numpy(x).to(DTYPES[dtype])[..., :sk]


def compact_inputs(n_seqs, H, D, dtype, seed, len_lo, len_hi, same_kv_lengths=True,
                   lengths_q=None, lengths_k=None, extra_tokens=0, causal_modes=(True,)):
    """Packed THD tokens: Q (Tq,H,D), K/V (Tk,H,D) plus int32 cu_seqlens.

    Lengths are drawn (query lengths first, then key lengths when they differ)
    unless given.  ``extra_tokens`` appends that many unused tokens after the
    last sequence, so a test can check they are never read or written.
    """
    rng = np.random.default_rng(seed)
    if lengths_q is None:
        lengths_q = rng.integers(len_lo, len_hi, size=n_seqs, endpoint=True)
    if lengths_k is None:
        lengths_k = lengths_q if same_kv_lengths else rng.integers(
            len_lo, len_hi, size=n_seqs, endpoint=True)
    cu_q = cu_from_lengths(lengths_q)
    cu_k = cu_from_lengths(lengths_k)
    tq = int(cu_q[-1]) + extra_tokens
    tk = int(cu_k[-1]) + extra_tokens
    q = _draw(rng, (tq, H, D), dtype)
    k = _draw(rng, (tk, H, D), dtype)
    v = _draw(rng, (tk, H, D), dtype)
    return AttnInputs(
        "compact", dtype, q, k, v, default_scale(D), tuple(causal_modes), cu_q, cu_k,
        meta=dict(H=H, D=D, seed=seed, n_seqs=n_seqs,
                  lengths_q=np.asarray(lengths_q).tolist(),
                  lengths_k=np.asarray(lengths_k).tolist()),
    )


def padded_inputs(B, H, Sq_max, Sk_max, D, dtype, seed, len_lo, len_hi,
                  same_kv_lengths=True, lengths_q=None, lengths_k=None,
                  causal_modes=(True,)):
    """Rank-4 BHSD slabs (B,H,S_max,D) with per-batch true lengths in cu_seqlens."""
    rng = np.random.default_rng(seed)
    if lengths_q is None:
        lengths_q = rng.integers(len_lo, len_hi, size=B, endpoint=True)
    if lengths_k is None:
        lengths_k = lengths_q if same_kv_lengths else rng.integers(
            len_lo, len_hi, size=B, endpoint=True)
    q = _draw(rng, (B, H, Sq_max, D), dtype)
    k = _draw(rng, (B, H, Sk_max, D), dtype)
    v = _draw(rng, (B, H, Sk_max, D), dtype)
    return AttnInputs(
        "padded", dtype, q, k, v, default_scale(D), tuple(causal_modes),
        cu_from_lengths(lengths_q), cu_from_lengths(lengths_k),
        meta=dict(B=B, H=H, Sq_max=Sq_max, Sk_max=Sk_max, D=D, seed=seed,
                  lengths_q=np.asarray(lengths_q).tolist(),
                  lengths_k=np.asarray(lengths_k).tolist()),
    )


# The five workloads: name -> (builder, kwargs).  The headline seed of the
# k-th workload is k.
WORKLOADS = {
    "tiny_dense_fp32_b1h2s128d64": (
        dense_inputs, dict(B=1, H=2, Sq=128, Sk=128, D=64, dtype="fp32", seed=1,
                           causal_modes=(False, True))),
    "dense_bf16_b4h16s2048d128": (
        dense_inputs, dict(B=4, H=16, Sq=2048, Sk=2048, D=128, dtype="bf16", seed=2,
                           causal_modes=(False, True))),
    "dense_fp16_b2h32sq512sk8192d64": (
        dense_inputs, dict(B=2, H=32, Sq=512, Sk=8192, D=64, dtype="fp16", seed=3,
                           causal_modes=(False,))),
    "thd_bf16_16seq_len1to4096_h16d128_causal": (
        compact_inputs, dict(n_seqs=16, H=16, D=128, dtype="bf16", seed=4,
                             len_lo=1, len_hi=4096, causal_modes=(True,))),
    "padded_bf16_b8h32smax8192d128_len2048to8192_causal": (
        padded_inputs, dict(B=8, H=32, Sq_max=8192, Sk_max=8192, D=128, dtype="bf16",
                            seed=5, len_lo=2048, len_hi=8192, causal_modes=(True,))),
}


def workload(name: str, seed: int | None = None) -> AttnInputs:
    """Build a named workload, optionally with another seed."""
    builder, kwargs = WORKLOADS[name]
    kwargs = dict(kwargs)
    if seed is not None:
        kwargs["seed"] = seed
    return builder(**kwargs)


def workload_lengths(name: str, seed: int | None = None) -> list:
    """The per-sequence (or per-batch) true lengths of a variable-length
    workload without drawing its tensors: step 1 of the recipe alone (the
    lengths come first out of the generator, so they equal those of
    ``workload(name, seed)``)."""
    builder, kwargs = WORKLOADS[name]
    if builder is dense_inputs:
        raise ValueError(f"{name} is a dense workload")
    n = kwargs["n_seqs"] if builder is compact_inputs else kwargs["B"]
    rng = np.random.default_rng(kwargs["seed"] if seed is None else seed)
    return rng.integers(kwargs["len_lo"], kwargs["len_hi"], size=n, endpoint=True).tolist()
