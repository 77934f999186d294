"""GPU parity of the backward (attn_bwd and its compact and padded varlen
forms) against the float64 oracle.

The forward's own outputs (O and LSE from the GPU forward) feed the
backward, as in training; the oracle's gradients are computed from Q, K, V
and dO alone.  Every gradient element of small and ragged shapes is compared
(both masks, D 64 and 128, bf16 and fp16); whole heads of the dense bf16
B4 H16 S2048 D128 workload, a whole S8192 head and whole (sequence, head)
pairs of the THD and padded workloads are compared in full.  Also: determinism, empty query or key
axes, untouched rows outside every sequence, no gradient crossing a sequence
boundary, the fp32 refusal, a too-small workspace, and a workspace whose old
contents (NaN bytes) are never read.

Tolerance.  The gradients are sums of products whose factors were rounded to
the input type (P and dS before the matrix products, O before delta), so the
error of an element is a few units of that type's rounding (u = 2^-8 for
bf16, 2^-11 for fp16) times the magnitude of the terms.  The checks bound
the error relative to the largest reference element of each gradient,
floored at 0.1 (a gradient that is exactly zero, such as dQ with a single key,
still carries the rounding of O inside delta):
max|err| <= MAX_REL * s and mean|err| <= MEAN_REL * s, s = max(max|ref|, 0.1).
MAX_REL is about 5 u for bf16 and 10 u for fp16, MEAN_REL about u/2 and u;
the measured errors sit 3 to 10 times below them.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import (attention_head_bwd, sdpa_compact_varlen_bwd, sdpa_dense_bwd,
                    sdpa_padded_varlen_bwd)
from parity import to64
from scaled_dot_product_03_amd import binding, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_REL = {"bf16": 2e-2, "fp16": 5e-3}
MEAN_REL = {"bf16": 2e-3, "fp16": 5e-4}


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()
    yield
    torch.cuda.synchronize()


def _grad_check(got, ref, dt, label):
    got = to64(got)
    err = np.abs(got - ref)
    scale = max(float(np.abs(ref).max()), 0.1)
    mx, mean = float(err.max()), float(err.mean())
    _log(f"  {label}: max|ref| {scale:.3g} max|err| {mx:.3g} ({mx / scale:.2e}) "
         f"mean|err| {mean:.3g} ({mean / scale:.2e})")
    assert np.isfinite(got).all(), label
    assert mx <= MAX_REL[dt] * scale, label
    assert mean <= MEAN_REL[dt] * scale, label


def _dev(t):
    return t.to(DEV)


def _run(B, H, Sq, Sk, D, dt, causal, seed, heads=None):
    x = inputs.dense_inputs(B, H, Sq, Sk, D, dt, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    do = torch.from_numpy(rng.standard_normal((B, H, Sq, D), dtype=np.float32)).to(
        inputs.DTYPES[dt])
    q, k, v, dod = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV), do.to(DEV)
    o, lse = binding.attn_fwd(q, k, v, scale=x.scale, causal=causal)
    dq, dk, dv = binding.attn_bwd(q, k, v, o, dod, lse, scale=x.scale, causal=causal)
    torch.cuda.synchronize()
    ref = sdpa_dense_bwd(to64(x.q), to64(x.k), to64(x.v), to64(do), x.scale, causal, heads=heads)
    return (dq, dk, dv), ref


SMALL = [
    # B, H, Sq, Sk, D, dtype
    (1, 2, 64, 64, 64, "bf16"),
    (2, 1, 127, 129, 128, "bf16"),
    (1, 2, 129, 127, 64, "fp16"),
    (1, 1, 300, 520, 128, "fp16"),
    (1, 1, 1, 200, 128, "bf16"),
    (1, 2, 200, 1, 64, "bf16"),
    (2, 2, 257, 257, 128, "bf16"),
    (1, 1, 33, 700, 64, "fp16"),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_bwd_small(shape, causal):
    B, H, Sq, Sk, D, dt = shape
    _log(f"bwd {shape} causal={causal}")
    got, ref = _run(B, H, Sq, Sk, D, dt, causal, seed=Sq * 3 + Sk + D)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        _grad_check(g, r, dt, f"{shape} causal={causal} {name}")


def test_bwd_workload_dense_bf16_s2048_heads():
    heads = [(0, 0), (3, 15)]
    for causal in (False, True):
        _log(f"bwd B4H16S2048D128 causal={causal} heads {heads}")
        got, ref = _run(4, 16, 2048, 2048, 128, "bf16", causal, seed=2, heads=heads)
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            gg = torch.stack([g[b, h] for b, h in heads])
            rr = np.stack([r[b, h] for b, h in heads])
            _grad_check(gg, rr, "bf16", f"S2048 causal={causal} {name}")


def test_bwd_long_sequence_bf16_s8192_one_head():
    """A sequence four times the workload's (bf16 B1 H1 S8192 D128), both
    masks, every gradient element of the head against the oracle."""
    for causal in (False, True):
        _log(f"bwd B1H1S8192D128 causal={causal}")
        got, ref = _run(1, 1, 8192, 8192, 128, "bf16", causal, seed=107)
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            _grad_check(g, r, "bf16", f"S8192 causal={causal} {name}")


def test_bwd_deterministic():
    x = inputs.dense_inputs(1, 2, 300, 300, 128, "bf16", seed=4)
    q, k, v = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV)
    do = torch.randn_like(q)
    o, lse = binding.attn_fwd(q, k, v, causal=True)
    a = binding.attn_bwd(q, k, v, o, do, lse, causal=True)
    b = binding.attn_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    for ga, gb in zip(a, b):
        assert torch.equal(ga, gb)


def test_bwd_empty_axes():
    # no keys: dq = 0 (every row's weights are empty); no queries: dk = dv = 0
    x = inputs.dense_inputs(1, 2, 70, 0, 64, "bf16", seed=5)
    q, k, v = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV)
    o, lse = binding.attn_fwd(q, k, v)
    dq = torch.full_like(q, 3.0)
    binding.attn_bwd(q, k, v, o, torch.ones_like(q), lse, dq=dq)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq) == 0
    y = inputs.dense_inputs(1, 2, 0, 90, 64, "fp16", seed=6)
    q, k, v = y.q.to(DEV), y.k.to(DEV), y.v.to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device=DEV)
    dk = torch.full_like(k, 3.0)
    dv = torch.full_like(v, 3.0)
    binding.attn_bwd(q, k, v, o, o, lse, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk) == 0 and torch.count_nonzero(dv) == 0


def test_bwd_refusals_leave_outputs_untouched():
    x = inputs.dense_inputs(1, 1, 64, 64, 64, "fp32", seed=7)
    q, k, v = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV)
    o, lse = binding.attn_fwd(q, k, v)
    dq = torch.full_like(q, 5.0)
    with pytest.raises(binding.SdpaError) as e:
        binding.attn_bwd(q, k, v, o, o, lse, dq=dq)
    assert e.value.status == 2
    y = inputs.dense_inputs(1, 1, 64, 64, 64, "bf16", seed=7)
    q, k, v = y.q.to(DEV), y.k.to(DEV), y.v.to(DEV)
    o, lse = binding.attn_fwd(q, k, v)
    dq = torch.full_like(q, 5.0)
    ws = torch.empty(binding.bwd_workspace_bytes(1, 1, 64) - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(binding.SdpaError) as e:
        binding.attn_bwd(q, k, v, o, o, lse, dq=dq, workspace=ws)
    assert e.value.status == 11
    torch.cuda.synchronize()
    assert (dq == 5.0).all()


# ---------------------------------------------------------------------------
# Variable-length backward
# ---------------------------------------------------------------------------

def _dout_like(shape, dt, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(inputs.DTYPES[dt])


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("fp16", 64), ("bf16", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_compact_small(dt, D, causal):
    lengths_q = [1, 128, 129, 300, 0, 77, 255]
    lengths_k = [1, 128, 129, 300, 5, 0, 400]
    H = 3
    _log(f"bwd compact small {dt} D{D} causal={causal}")
    x = inputs.compact_inputs(len(lengths_q), H, D, dt, seed=61, len_lo=1, len_hi=2,
                              lengths_q=lengths_q, lengths_k=lengths_k, extra_tokens=5)
    do = _dout_like(tuple(x.q.shape), dt, 62)
    q, k, v, dod = _dev(x.q), _dev(x.k), _dev(x.v), _dev(do)
    o, lse = binding.attn_fwd_compact_varlen(q, k, v, x.cu_seqlens_q, x.cu_seqlens_k,
                                             scale=x.scale, causal=causal)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    binding.attn_bwd_compact_varlen(q, k, v, o, dod, lse, x.cu_seqlens_q, x.cu_seqlens_k,
                                    scale=x.scale, causal=causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = sdpa_compact_varlen_bwd(to64(x.q), to64(x.k), to64(x.v), to64(do), x.cu_seqlens_q,
                                  x.cu_seqlens_k, x.scale, causal)
    tq, tk = int(x.cu_seqlens_q[-1]), int(x.cu_seqlens_k[-1])
    # tokens past the last sequence are neither read nor written
    assert torch.isnan(dq[tq:]).all()
    assert torch.isnan(dk[tk:]).all() and torch.isnan(dv[tk:]).all()
    for name, g, r, t in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, (tq, tk, tk)):
        _grad_check(g[:t], r[:t], dt, f"compact {dt} D{D} causal={causal} {name}")


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("fp16", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_padded_small(dt, D, causal):
    B, H, Sq, Sk = 4, 2, 300, 270
    lengths_q = [300, 1, 129, 0]
    lengths_k = [270, 64, 1, 33]
    _log(f"bwd padded small {dt} D{D} causal={causal}")
    x = inputs.padded_inputs(B, H, Sq, Sk, D, dt, seed=71, len_lo=1, len_hi=2,
                             lengths_q=lengths_q, lengths_k=lengths_k)
    do = _dout_like((B, H, Sq, D), dt, 72)
    q, k, v, dod = _dev(x.q), _dev(x.k), _dev(x.v), _dev(do)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Sq), float("nan"), device=DEV)
    binding.attn_fwd_padded_varlen(q, k, v, x.cu_seqlens_q, x.cu_seqlens_k, scale=x.scale,
                                   causal=causal, out=o, lse=lse)
    # poison every input past the true lengths: it must never be read
    for b in range(B):
        q[b, :, lengths_q[b]:] = float("nan")
        dod[b, :, lengths_q[b]:] = float("nan")
        k[b, :, lengths_k[b]:] = float("inf")
        v[b, :, lengths_k[b]:] = float("nan")
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    binding.attn_bwd_padded_varlen(q, k, v, o, dod, lse, x.cu_seqlens_q, x.cu_seqlens_k,
                                   scale=x.scale, causal=causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = sdpa_padded_varlen_bwd(to64(x.q), to64(x.k), to64(x.v), to64(do), x.cu_seqlens_q,
                                 x.cu_seqlens_k, x.scale, causal)
    for b in range(B):
        lq, lk = lengths_q[b], lengths_k[b]
        assert torch.isnan(dq[b, :, lq:]).all()
        assert torch.isnan(dk[b, :, lk:]).all() and torch.isnan(dv[b, :, lk:]).all()
        for name, g, r, n in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, (lq, lk, lk)):
            if n:
                _grad_check(g[b, :, :n], r[b, :, :n], dt,
                            f"padded {dt} D{D} causal={causal} b={b} {name}")


@pytest.mark.parametrize("layout", ["dense", "compact", "padded"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_workspace_contents_never_read_before_written(layout, causal):
    """The dQ kernel writes each query row's row values (and the padding rows
    the dK/dV kernel's tiles reach) into the caller's workspace before the
    dK/dV kernel reads them: a workspace full of NaN bytes and one full of
    zeros give bit-identical, finite gradients.  Ragged lengths (not multiples
    of 64 or 256), an empty sequence and tokens past the last sequence."""
    dt, D, H = "bf16", 128, 2
    _log(f"bwd workspace poison {layout} causal={causal}")
    if layout == "dense":
        x = inputs.dense_inputs(1, H, 300, 333, D, dt, seed=91)
        do = _dout_like(tuple(x.q.shape), dt, 92)
        q, k, v, dod = _dev(x.q), _dev(x.k), _dev(x.v), _dev(do)
        o, lse = binding.attn_fwd(q, k, v, scale=x.scale, causal=causal)
        nbytes = binding.bwd_workspace_bytes(1, H, 300)
        call = lambda ws: binding.attn_bwd(q, k, v, o, dod, lse, scale=x.scale, causal=causal,
                                           workspace=ws)
    elif layout == "compact":
        lengths = [70, 0, 257, 130]
        x = inputs.compact_inputs(len(lengths), H, D, dt, seed=93, len_lo=1, len_hi=2,
                                  lengths_q=lengths, lengths_k=lengths, extra_tokens=7)
        do = _dout_like(tuple(x.q.shape), dt, 94)
        q, k, v, dod = _dev(x.q), _dev(x.k), _dev(x.v), _dev(do)
        o, lse = binding.attn_fwd_compact_varlen(q, k, v, x.cu_seqlens_q, x.cu_seqlens_k,
                                                 scale=x.scale, causal=causal)
        nbytes = binding.bwd_workspace_bytes(1, H, int(q.shape[0]))
        call = lambda ws: binding.attn_bwd_compact_varlen(
            q, k, v, o, dod, lse, x.cu_seqlens_q, x.cu_seqlens_k, scale=x.scale, causal=causal,
            workspace=ws)
    else:
        lengths = [300, 0, 65, 190]
        x = inputs.padded_inputs(4, H, 300, 300, D, dt, seed=95, len_lo=1, len_hi=2,
                                 lengths_q=lengths, lengths_k=lengths)
        do = _dout_like(tuple(x.q.shape), dt, 96)
        q, k, v, dod = _dev(x.q), _dev(x.k), _dev(x.v), _dev(do)
        o, lse = binding.attn_fwd_padded_varlen(q, k, v, x.cu_seqlens_q, x.cu_seqlens_k,
                                                scale=x.scale, causal=causal)
        nbytes = binding.bwd_workspace_bytes(4, H, 300)
        call = lambda ws: binding.attn_bwd_padded_varlen(
            q, k, v, o, dod, lse, x.cu_seqlens_q, x.cu_seqlens_k, scale=x.scale, causal=causal,
            workspace=ws)
    zeros = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    poison = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
    a = call(zeros)
    b = call(poison)
    torch.cuda.synchronize()
    if layout == "compact":
        tq, tk = int(x.cu_seqlens_q[-1]), int(x.cu_seqlens_k[-1])
        a = (a[0][:tq], a[1][:tk], a[2][:tk])
        b = (b[0][:tq], b[1][:tk], b[2][:tk])
    elif layout == "padded":
        a = tuple(torch.cat([g[i, :, :n] for i, n in enumerate(lengths)], dim=1) for g in a)
        b = tuple(torch.cat([g[i, :, :n] for i, n in enumerate(lengths)], dim=1) for g in b)
    for name, ga, gb in zip(("dq", "dk", "dv"), a, b):
        assert torch.isfinite(ga).all(), name
        assert torch.equal(ga, gb), name


def test_bwd_compact_no_cross_sequence_leak_bit_exact():
    """Sequence z's Q, K and dO rows are multiples of the unit vector e_z, so
    each of its gradients lies along e_z: a weight or gradient term taken
    across a sequence boundary would make another column non-zero."""
    lengths = [5, 130, 1, 257, 64, 63, 200]
    H, D = 2, 64
    x = inputs.compact_inputs(len(lengths), H, D, "bf16", seed=81, len_lo=1, len_hi=2,
                              lengths_q=lengths, lengths_k=lengths)
    cu = x.cu_seqlens_q
    rng = np.random.default_rng(82)
    q = torch.zeros_like(x.q)
    k = torch.zeros_like(x.k)
    do = torch.zeros_like(x.q)
    for z in range(len(lengths)):
        s, e = int(cu[z]), int(cu[z + 1])
        for t, scale in ((q, 2.0), (k, 2.0), (do, 1.0)):
            t[s:e, :, z] = torch.from_numpy(
                rng.uniform(0.5, 1.0, size=(e - s, H)).astype(np.float32) * scale).to(t.dtype)
    q, k, v, dod = _dev(q), _dev(k), _dev(x.v), _dev(do)
    for causal in (False, True):
        o, lse = binding.attn_fwd_compact_varlen(q, k, v, cu, cu, scale=x.scale, causal=causal)
        grads = binding.attn_bwd_compact_varlen(q, k, v, o, dod, lse, cu, cu, scale=x.scale,
                                                causal=causal)
        torch.cuda.synchronize()
        for name, g in zip(("dq", "dk", "dv"), grads):
            g = g.cpu().float()
            for z in range(len(lengths)):
                blk = g[cu[z]:cu[z + 1]]
                others = torch.cat([blk[..., :z], blk[..., z + 1:]], dim=-1)
                assert torch.count_nonzero(others) == 0, f"{name} of sequence {z} leaked"
            assert torch.count_nonzero(g) > 0, name


def test_bwd_compact_deterministic():
    x = inputs.compact_inputs(5, 2, 128, "fp16", seed=91, len_lo=1, len_hi=400)
    q, k, v = _dev(x.q), _dev(x.k), _dev(x.v)
    do = torch.randn_like(q)
    o, lse = binding.attn_fwd_compact_varlen(q, k, v, x.cu_seqlens_q, x.cu_seqlens_k, causal=True)
    a = binding.attn_bwd_compact_varlen(q, k, v, o, do, lse, x.cu_seqlens_q, x.cu_seqlens_k,
                                        causal=True)
    b = binding.attn_bwd_compact_varlen(q, k, v, o, do, lse, x.cu_seqlens_q, x.cu_seqlens_k,
                                        causal=True)
    torch.cuda.synchronize()
    for ga, gb in zip(a, b):
        assert torch.equal(ga, gb)


def test_bwd_workload_compact_thd_pairs():
    """THD workload (16 sequences of 1 to 4096 tokens, H16 D128, causal bf16):
    the whole gradients of one head of four sequences, the longest among
    them."""
    x = inputs.workload("thd_bf16_16seq_len1to4096_h16d128_causal")
    lengths = x.meta["lengths_q"]
    _log(f"bwd compact THD lengths {lengths}")
    do = _dout_like(tuple(x.q.shape), "bf16", 104)
    q, k, v, dod = _dev(x.q), _dev(x.k), _dev(x.v), _dev(do)
    o, lse = binding.attn_fwd_compact_varlen(q, k, v, x.cu_seqlens_q, x.cu_seqlens_k,
                                             scale=x.scale, causal=True)
    # NaN-filled gradients: the sequences cover every token, so every row of
    # dQ, dK and dV must be written (both kernels' causal launches take each
    # XCD's heads in parts here).
    grads = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    binding.attn_bwd_compact_varlen(q, k, v, o, dod, lse, x.cu_seqlens_q, x.cu_seqlens_k,
                                    scale=x.scale, causal=True, dq=grads[0], dk=grads[1],
                                    dv=grads[2])
    torch.cuda.synchronize()
    assert int(x.cu_seqlens_q[-1]) == q.shape[0]
    for g in grads:
        assert torch.isfinite(g).all()
    cu = x.cu_seqlens_q
    order = np.argsort(lengths)
    picks = list(dict.fromkeys([int(order[-1]), int(order[0]), int(order[len(order) // 2]), 5]))
    for z in picks:
        s, e = int(cu[z]), int(cu[z + 1])
        h = (3 * z + 1) % 16
        _log(f"  sequence {z} (length {e - s}) head {h}")
        ref = attention_head_bwd(to64(x.q[s:e, h]), to64(x.k[s:e, h]), to64(x.v[s:e, h]),
                                 to64(do[s:e, h]), x.scale, True)
        for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
            _grad_check(g[s:e, h], r, "bf16", f"THD z={z} h={h} {name}")


def test_bwd_workload_padded_pairs():
    """Padded workload (B8 H32, 8192-row slabs, true lengths 2048 to 8192,
    causal bf16): the whole gradients of one head of the two shortest
    batches; padding rows stay untouched everywhere."""
    x = inputs.workload("padded_bf16_b8h32smax8192d128_len2048to8192_causal")
    lengths = x.meta["lengths_q"]
    _log(f"bwd padded lengths {lengths}")
    B, H, S, D = x.q.shape
    do = _dout_like((B, H, S, D), "bf16", 105)
    q, k, v, dod = _dev(x.q), _dev(x.k), _dev(x.v), _dev(do)
    o, lse = binding.attn_fwd_padded_varlen(q, k, v, x.cu_seqlens_q, x.cu_seqlens_k,
                                            scale=x.scale, causal=True)
    scale = x.scale
    del x  # keep host memory to the sampled heads below
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    binding.attn_bwd_padded_varlen(q, k, v, o, dod, lse, inputs.cu_from_lengths(lengths),
                                   inputs.cu_from_lengths(lengths), causal=True, dq=dq, dk=dk,
                                   dv=dv, scale=scale)
    torch.cuda.synchronize()
    for b, L in enumerate(lengths):
        for g in (dq, dk, dv):
            assert torch.isnan(g[b, :, L:]).all()
            assert torch.isfinite(g[b, :, :L]).all()
    for b in [int(i) for i in np.argsort(lengths)[:2]]:
        L, h = lengths[b], (5 * b + 2) % H
        _log(f"  batch {b} (length {L}) head {h}")
        ref = attention_head_bwd(to64(q[b, h, :L]), to64(k[b, h, :L]), to64(v[b, h, :L]),
                                 to64(dod[b, h, :L]), scale, True)
        for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            _grad_check(g[b, h, :L], r, "bf16", f"padded b={b} h={h} {name}")
