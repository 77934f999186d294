"""The split forward on the library's static scratch, attn_fwd_splitk_noalloc,
called through the C ABI: its output must equal attn_fwd_splitk's (the same
kernels and split plan with a caller workspace) and the float64 oracle's, on
two calls in a row, the second on a smaller problem -- the buffer keeps the
first call's partial results, which must not leak into the second.  A
problem whose plan exceeds the scratch is refused before any launch."""

import sys

import numpy as np
import pytest
import torch

from oracle import attention_head, sdpa_dense
from parity import check, sample_rows, to64
from scaled_dot_product_03_amd import binding, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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


def _both(x, causal, splits):
    """(split forward with a workspace, the same without one) on x."""
    q, k, v = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV)
    o_ws, lse_ws = binding.attn_fwd_splitk(q, k, v, scale=x.scale, causal=causal,
                                           num_splits=splits)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=DEV)
    binding.attn_fwd_splitk_noalloc(q, k, v, scale=x.scale, causal=causal, num_splits=splits,
                                    out=o, lse=lse)
    torch.cuda.synchronize()
    return o_ws, lse_ws, o, lse


def test_noalloc_equals_split_forward_on_two_calls_in_a_row():
    # Call 1: the fp16 Sq 512 Sk 8192 D 64 workload in the library's default
    # split (17 MB of the 32 MiB scratch).
    x = inputs.workload("dense_fp16_b2h32sq512sk8192d64")
    B, H, Sq, D = x.q.shape
    Sk = x.k.shape[2]
    used, nbytes = binding.splitk_plan(x.q.dtype, B, H, Sq, Sk, D)
    _log(f"call 1: fp16 B{B} H{H} Sq{Sq} Sk{Sk} D{D}, {used} splits, {nbytes} scratch bytes")
    assert used > 1 and nbytes <= binding.NOALLOC_SCRATCH_BYTES
    o_ws, lse_ws, o, lse = _both(x, False, 0)
    assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws)
    rng = np.random.default_rng(31)
    og, lg = to64(o), to64(lse)
    for b, h in [(0, 0), (1, H - 1), (1, 7)]:
        rows = sample_rows(Sq, rng, extra=16)
        ro, rl = attention_head(x.q[b, h].double().numpy()[rows], x.k[b, h].double().numpy(),
                                x.v[b, h].double().numpy(), x.scale, False)
        check(og[b, h, rows], lg[b, h, rows], ro, rl, "fp16", f"call 1 (b={b}, h={h})")
    del o_ws, lse_ws, o, lse

    # Call 2: a smaller bf16 problem with ragged sizes under the causal mask,
    # more splits than call 1; every element against the oracle.
    y = inputs.dense_inputs(1, 3, 300, 1900, 128, "bf16", seed=32)
    used2, nbytes2 = binding.splitk_plan(y.q.dtype, 1, 3, 300, 1900, 128, 5)
    _log(f"call 2: bf16 B1 H3 Sq300 Sk1900 D128 causal, {used2} splits, {nbytes2} bytes")
    assert used2 > 1 and nbytes2 < nbytes
    o_ws, lse_ws, o, lse = _both(y, True, 5)
    assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws)
    ro, rl = sdpa_dense(y.q.double().numpy(), y.k.double().numpy(), y.v.double().numpy(),
                        y.scale, True)
    stats = check(to64(o), to64(lse), ro, rl, "bf16", "call 2")
    _log(f"call 2: max|dO| {stats['max_o']:.2e} mean|dO| {stats['mean_o']:.2e} "
         f"max|dLSE| {stats['max_lse']:.2e}")


def test_noalloc_refuses_a_plan_larger_than_the_scratch():
    B, H, S, D = 4, 16, 2048, 128
    used, nbytes = binding.splitk_plan(torch.bfloat16, B, H, S, S, D, 8)
    assert nbytes > binding.NOALLOC_SCRATCH_BYTES
    q = torch.randn((B, H, S, D), device=DEV).bfloat16()
    o = torch.full_like(q, 3.0)
    lse = torch.full((B, H, S), 5.0, device=DEV)
    with pytest.raises(binding.SdpaError) as e:
        binding.attn_fwd_splitk_noalloc(q, q, q, num_splits=8, out=o, lse=lse)
    assert e.value.status == 12
    torch.cuda.synchronize()
    assert (o == 3.0).all() and (lse == 5.0).all()
