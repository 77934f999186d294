"""Pins for the float64 oracle, against things other than the oracle itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped scale, a
wrong sign, a transposed operand, the causal mask pointing the wrong way, a
log in the wrong base, a missing normalisation, keys leaking across
sequences) fails at least one of them:

* an exact rational worked example (scale = ln 2, integer Q/K/V);
* a pure-Python brute force written in a different algebraic form;
* PyTorch's CPU attention routines in float64 (library check);
* closed forms: zero queries, a single key, two keys, the first causal row,
  constant V;
* invariants: V = identity exposes P, per-row score shifts, key permutation,
  linearity in V;
* variable-length modes equal dense attention on slices, and equal one
  block-diagonal masked attention over the packed tokens.
"""

import json
import math
import os
import subprocess
import sys
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (
    attention_head,
    lengths_from_cu,
    sdpa_compact_varlen,
    sdpa_dense,
    sdpa_padded_varlen,
)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Exact worked example
# ---------------------------------------------------------------------------

def _load_pow2():
    with open(os.path.join(GOLDEN, "pow2_attention_example.json")) as f:
        return json.load(f)


def test_pow2_fixture_is_current():
    """The stored fixture is what its exact-arithmetic script writes."""
    sys.path.insert(0, GOLDEN)
    try:
        import make_pow2_example as gen
    finally:
        sys.path.pop(0)
    assert gen.build() == _load_pow2()


@pytest.mark.parametrize("causal", [False, True])
def test_pow2_worked_example_exact(causal):
    ex = _load_pow2()
    key = "causal" if causal else "noncausal"
    q, k, v = (np.array(ex[n], dtype=np.float64) for n in ("Q", "K", "V"))
    o, lse = attention_head(q, k, v, math.log(2.0), causal)
    want_o = np.array([[float(Fraction(x)) for x in row] for row in ex[key]["O"]])
    want_lse = np.array([math.log(Fraction(r)) for r in ex[key]["R"]])
    np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Brute force: scalar loops, no max subtraction, weights as 1/sum exp(S_ik - S_ij)
# ---------------------------------------------------------------------------

def _brute(q, k, v, scale, causal):
    lq, lk, dv = len(q), len(k), len(v[0])
    out, lse = [], []
    for i in range(lq):
        keys = [j for j in range(lk) if not (causal and j > i)]
        s = {j: scale * math.fsum(q[i][d] * k[j][d] for d in range(len(q[i]))) for j in keys}
        if not keys:
            out.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        weights = {j: 1.0 / math.fsum(math.exp(s[kk] - s[j]) for kk in keys) for j in keys}
        out.append([math.fsum(weights[j] * v[j][c] for j in keys) for c in range(dv)])
        lse.append(math.log(math.fsum(math.exp(s[j]) for j in keys)))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny(seed):
    rng = _rng(1000 + seed)
    lq, lk = rng.integers(1, 9, size=2)
    d, dv = rng.integers(1, 7, size=2)
    q = rng.standard_normal((lq, d))
    k = rng.standard_normal((lk, d))
    v = rng.standard_normal((lk, dv))
    scale = float(rng.uniform(0.2, 1.5))
    for causal in (False, True):
        o, lse = attention_head(q, k, v, scale, causal)
        bo, blse = _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Library routines (PyTorch CPU, float64)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(2, 3, 37, 53, 16), (1, 2, 64, 64, 64), (1, 1, 70, 20, 8),
                                   (2, 2, 1, 33, 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_sdpa_fp64(shape, causal):
    b, h, sq, sk, d = shape
    rng = _rng(sum(shape) + causal)
    q = rng.standard_normal((b, h, sq, d))
    k = rng.standard_normal((b, h, sk, d))
    v = rng.standard_normal((b, h, sk, d))
    scale = 1.0 / math.sqrt(d)
    o, lse = sdpa_dense(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref_o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, ref_o.numpy(), rtol=0, atol=1e-12)
    # PyTorch's CPU flash routine also returns the natural-log logsumexp.
    f_o, f_lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq, tk, tv, 0.0, causal, scale=scale)[:2]
    np.testing.assert_allclose(o, f_o.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, f_lse.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def test_zero_queries_give_uniform_attention():
    rng = _rng(7)
    lq, lk, d = 9, 13, 5
    q = np.zeros((lq, d))
    k = rng.standard_normal((lk, d))
    v = rng.standard_normal((lk, 4))
    o, lse = attention_head(q, k, v, 0.7, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, np.full(lq, math.log(lk)), atol=1e-14)
    o, lse = attention_head(q, k, v, 0.7, True)
    for i in range(lq):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), atol=1e-14)
        assert abs(lse[i] - math.log(i + 1)) < 1e-14


def test_single_key():
    rng = _rng(8)
    q = rng.standard_normal((6, 7))
    k = rng.standard_normal((1, 7))
    v = rng.standard_normal((1, 3))
    o, lse = attention_head(q, k, v, 0.3, False)
    np.testing.assert_allclose(o, np.repeat(v, 6, axis=0), atol=1e-15)
    for i in range(6):
        assert abs(lse[i] - 0.3 * math.fsum(q[i] * k[0])) < 1e-14


def test_two_keys_logistic():
    """Two keys: weight of key 0 is the logistic function of S_i0 - S_i1."""
    rng = _rng(9)
    q = rng.standard_normal((5, 4))
    k = rng.standard_normal((2, 4))
    v = rng.standard_normal((2, 3))
    scale = 0.9
    o, lse = attention_head(q, k, v, scale, False)
    for i in range(5):
        s0 = scale * math.fsum(q[i] * k[0])
        s1 = scale * math.fsum(q[i] * k[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(o[i], w0 * v[0] + (1 - w0) * v[1], atol=1e-14)
        assert abs(lse[i] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-14


def test_causal_first_row_is_first_value():
    rng = _rng(10)
    q = rng.standard_normal((8, 6))
    k = rng.standard_normal((11, 6))
    v = rng.standard_normal((11, 6))
    o, lse = attention_head(q, k, v, 0.5, True)
    assert np.array_equal(o[0], v[0])
    assert abs(lse[0] - 0.5 * math.fsum(q[0] * k[0])) < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_return_the_constant(causal):
    rng = _rng(11)
    q = 3 * rng.standard_normal((10, 8))
    k = 3 * rng.standard_normal((12, 8))
    v = np.full((12, 5), -2.75)
    o, _ = attention_head(q, k, v, 0.35, causal)
    np.testing.assert_allclose(o, -2.75, rtol=0, atol=1e-13)


def test_no_keys_gives_zero_and_minus_inf():
    q = np.ones((3, 4))
    o, lse = attention_head(q, np.zeros((0, 4)), np.zeros((0, 2)), 0.5, False)
    assert o.shape == (3, 2) and (o == 0).all() and np.isneginf(lse).all()


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_expose_softmax(causal):
    """With V = I the output rows are the weights P: nonnegative, rows sum to
    one, zero where masked, and P_ij / P_ik = exp(S_ij - S_ik)."""
    rng = _rng(12)
    lq, lk, d = 7, 9, 5
    q = rng.standard_normal((lq, d))
    k = rng.standard_normal((lk, d))
    scale = 0.8
    p, lse = attention_head(q, k, np.eye(lk), scale, causal)
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    for i in range(lq):
        top = i if causal else lk - 1
        if causal:
            assert (p[i, i + 1:] == 0).all()
        for j in range(top + 1):
            # exp(S_ij - LSE_i) is the weight itself.
            s_ij = scale * math.fsum(q[i] * k[j])
            assert abs(p[i, j] - math.exp(s_ij - lse[i])) < 1e-14
        if top >= 1:
            s0 = scale * math.fsum(q[i] * k[0])
            s1 = scale * math.fsum(q[i] * k[1])
            assert abs(p[i, 0] / p[i, 1] - math.exp(s0 - s1)) < 1e-12 * max(1, math.exp(s0 - s1))


@pytest.mark.parametrize("causal", [False, True])
def test_row_shift_changes_only_lse(causal):
    """Adding c_i to every score of row i (via one extra feature) leaves O
    alone and adds c_i to LSE."""
    rng = _rng(13)
    lq, lk, d = 6, 10, 4
    q = rng.standard_normal((lq, d))
    k = rng.standard_normal((lk, d))
    v = rng.standard_normal((lk, 3))
    scale = 0.6
    a = rng.uniform(-20, 20, size=lq)
    o0, lse0 = attention_head(q, k, v, scale, causal)
    q1 = np.concatenate([q, a[:, None]], axis=1)
    k1 = np.concatenate([k, np.ones((lk, 1))], axis=1)
    o1, lse1 = attention_head(q1, k1, v, scale, causal)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse1, lse0 + scale * a, rtol=0, atol=1e-12)


def test_key_permutation_equivariance():
    rng = _rng(14)
    q = rng.standard_normal((8, 6))
    k = rng.standard_normal((15, 6))
    v = rng.standard_normal((15, 4))
    perm = rng.permutation(15)
    o0, lse0 = attention_head(q, k, v, 0.4, False)
    o1, lse1 = attention_head(q, k[perm], v[perm], 0.4, False)
    np.testing.assert_allclose(o1, o0, atol=1e-13)
    np.testing.assert_allclose(lse1, lse0, atol=1e-13)


def test_linear_in_values():
    rng = _rng(15)
    q = rng.standard_normal((5, 6))
    k = rng.standard_normal((9, 6))
    v1 = rng.standard_normal((9, 4))
    v2 = rng.standard_normal((9, 4))
    for causal in (False, True):
        a = attention_head(q, k, v1, 0.5, causal)[0]
        b = attention_head(q, k, v2, 0.5, causal)[0]
        c = attention_head(q, k, 2 * v1 - 3 * v2, 0.5, causal)[0]
        np.testing.assert_allclose(c, 2 * a - 3 * b, atol=1e-12)


def test_rows_argument_matches_full():
    rng = _rng(16)
    q = rng.standard_normal((20, 8))
    k = rng.standard_normal((25, 8))
    v = rng.standard_normal((25, 8))
    rows = np.array([0, 3, 19, 7])
    for causal in (False, True):
        o, lse = attention_head(q, k, v, 0.3, causal)
        o_r, lse_r = attention_head(q, k, v, 0.3, causal, rows=rows)
        np.testing.assert_array_equal(o_r, o[rows])
        np.testing.assert_array_equal(lse_r, lse[rows])


# ---------------------------------------------------------------------------
# Variable-length modes
# ---------------------------------------------------------------------------

def test_lengths_from_cu_validation():
    assert lengths_from_cu([0, 3, 3, 7]).tolist() == [3, 0, 4]
    with pytest.raises(ValueError):
        lengths_from_cu([1, 3])
    with pytest.raises(ValueError):
        lengths_from_cu([0, 5, 4])
    with pytest.raises(ValueError):
        lengths_from_cu([0, 5], total=4)


def _packed(rng, lengths_q, lengths_k, h, d):
    cu_q = np.concatenate([[0], np.cumsum(lengths_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lengths_k)]).astype(np.int32)
    q = rng.standard_normal((int(cu_q[-1]) + 3, h, d))
    k = rng.standard_normal((int(cu_k[-1]) + 2, h, d))
    v = rng.standard_normal((int(cu_k[-1]) + 2, h, d))
    return q, k, v, cu_q, cu_k


@pytest.mark.parametrize("causal", [False, True])
def test_compact_equals_dense_on_slices(causal):
    rng = _rng(17)
    lq = [5, 1, 17, 9, 0]
    lk = [5, 3, 17, 12, 4]
    q, k, v, cu_q, cu_k = _packed(rng, lq, lk, 3, 8)
    o, lse = sdpa_compact_varlen(q, k, v, cu_q, cu_k, 0.4, causal)
    for z in range(len(lq)):
        qs = slice(cu_q[z], cu_q[z + 1])
        ks = slice(cu_k[z], cu_k[z + 1])
        # THD slice -> (1, H, L, D)
        to_bhsd = lambda x: np.transpose(x, (1, 0, 2))[None]
        do, dl = sdpa_dense(to_bhsd(q[qs]), to_bhsd(k[ks]), to_bhsd(v[ks]), 0.4, causal)
        np.testing.assert_array_equal(o[qs], np.transpose(do[0], (1, 0, 2)))
        np.testing.assert_array_equal(lse[:, qs], dl[0])
    # tokens past the last sequence are never produced
    assert np.isnan(o[cu_q[-1]:]).all() and np.isnan(lse[:, cu_q[-1]:]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_compact_equals_block_diagonal_library_attention(causal):
    """Second formulation: one masked attention over all packed tokens, done by
    PyTorch's float64 SDPA with a block-diagonal (plus causal) boolean mask."""
    rng = _rng(18)
    lengths = [7, 1, 19, 12, 30]
    q, k, v, cu, _ = _packed(rng, lengths, lengths, 2, 16)
    t = int(cu[-1])
    q, k, v = q[:t], k[:t], v[:t]
    o, lse = sdpa_compact_varlen(q, k, v, cu, cu, 0.25, causal)
    seq = np.repeat(np.arange(len(lengths)), lengths)
    pos = np.arange(t) - cu[seq]
    mask = seq[:, None] == seq[None, :]
    if causal:
        mask &= pos[None, :] <= pos[:, None]
    to_bhsd = lambda x: torch.from_numpy(np.transpose(x, (1, 0, 2))[None].copy())
    ref = torch.nn.functional.scaled_dot_product_attention(
        to_bhsd(q), to_bhsd(k), to_bhsd(v), attn_mask=torch.from_numpy(mask), scale=0.25)
    np.testing.assert_allclose(o, np.transpose(ref[0].numpy(), (1, 0, 2)), atol=1e-12)
    ref_lse = torch.logsumexp(
        torch.where(torch.from_numpy(mask), 0.25 * to_bhsd(q)[0] @ to_bhsd(k)[0].transpose(-1, -2),
                    torch.tensor(-math.inf, dtype=torch.float64)), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_padded_equals_dense_truncated(causal):
    rng = _rng(19)
    b, h, sq, sk, d = 3, 2, 20, 24, 8
    q = rng.standard_normal((b, h, sq, d))
    k = rng.standard_normal((b, h, sk, d))
    v = rng.standard_normal((b, h, sk, d))
    lq = [20, 1, 13]
    lk = [24, 9, 13]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    # poison everything past the true lengths: it must never be read
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for i in range(b):
        q2[i, :, lq[i]:] = np.nan
        k2[i, :, lk[i]:] = np.inf
        v2[i, :, lk[i]:] = np.nan
    o, lse = sdpa_padded_varlen(q2, k2, v2, cu_q, cu_k, 0.3, causal)
    for i in range(b):
        do, dl = sdpa_dense(q[i:i + 1, :, : lq[i]], k[i:i + 1, :, : lk[i]],
                            v[i:i + 1, :, : lk[i]], 0.3, causal)
        np.testing.assert_array_equal(o[i, :, : lq[i]], do[0])
        np.testing.assert_array_equal(lse[i, :, : lq[i]], dl[0])
        assert np.isnan(o[i, :, lq[i]:]).all()


def test_golden_example_script_runs_standalone(tmp_path):
    """The fixture script needs nothing from the repository to run."""
    script = os.path.join(GOLDEN, "make_pow2_example.py")
    env = dict(os.environ, PYTHONPATH="")
    res = subprocess.run([sys.executable, "-c",
                          "import runpy,sys; sys.argv=['x']; "
                          f"g=runpy.run_path({script!r}); print(len(g['build']()['Q']))"],
                         cwd=str(tmp_path), env=env, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "4"
