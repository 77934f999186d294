"""Pins for the oracle's backward (CPU), against things other than itself.

* PyTorch's float64 autograd through its CPU scaled_dot_product_attention
  (library check), both masks, Sq != Sk;
* central finite differences of sum(dO * O) computed with the oracle's
  forward only (independent of the backward formulas);
* closed forms and invariants: zero upstream gradient, constant V (O does not
  depend on Q or K), a common shift of every key row (softmax is invariant to
  it, so the dK rows sum to zero), dV rows summing to the dO rows, keys no
  row may see under the causal mask;
* the variable-length modes equal the dense backward on slices, with zero
  gradients outside every sequence.

A plausible slip -- a dropped scale, delta with the wrong sign, dS not
transposed for dK, the causal mask the wrong way round, unnormalised P --
fails at least one of these.
"""

import numpy as np
import pytest
import torch

from oracle import (
    attention_head,
    attention_head_bwd,
    sdpa_compact_varlen_bwd,
    sdpa_dense_bwd,
    sdpa_padded_varlen_bwd,
)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lq,lk,d", [(5, 5, 4), (3, 7, 8), (9, 4, 16), (1, 1, 2), (6, 6, 1)])
def test_bwd_matches_torch_autograd(lq, lk, d, causal):
    rng = np.random.default_rng(lq * 31 + lk * 7 + d)
    q, k, v, do = (_rand(rng, n, d) for n in (lq, lk, lk, lq))
    scale = 0.37
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], is_causal=causal, scale=scale)[0, 0]
    out.backward(torch.tensor(do, dtype=torch.float64))
    dq, dk, dv = attention_head_bwd(q, k, v, do, scale, causal)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_finite_differences(causal):
    rng = np.random.default_rng(5)
    lq, lk, d = 3, 4, 3
    q, k, v, do = _rand(rng, lq, d), _rand(rng, lk, d), _rand(rng, lk, d), _rand(rng, lq, d)
    scale = 0.8

    def loss(q_, k_, v_):
        o, _ = attention_head(q_, k_, v_, scale, causal)
        return float((o * do).sum())

    grads = attention_head_bwd(q, k, v, do, scale, causal)
    h = 1e-6
    for which, g in enumerate(grads):
        for idx in np.ndindex(*g.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            up = loss(*args)
            args[which][idx] -= 2 * h
            dn = loss(*args)
            assert abs((up - dn) / (2 * h) - g[idx]) < 1e-7, (which, idx)


def test_bwd_zero_upstream_gives_zero():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 4, 8), _rand(rng, 6, 8), _rand(rng, 6, 8)
    for g in attention_head_bwd(q, k, v, np.zeros((4, 8)), 0.5, True):
        assert not g.any()


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_constant_v_has_no_query_or_key_gradient(causal):
    rng = np.random.default_rng(3)
    q, k = _rand(rng, 5, 4), _rand(rng, 5, 4)
    v = np.tile(_rand(rng, 1, 4), (5, 1))
    do = _rand(rng, 5, 4)
    dq, dk, dv = attention_head_bwd(q, k, v, do, 0.9, causal)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(causal):
    rng = np.random.default_rng(4)
    lq, lk, d = 7, 9, 5
    q, k, v, do = _rand(rng, lq, d), _rand(rng, lk, d), _rand(rng, lk, d), _rand(rng, lq, d)
    dq, dk, dv = attention_head_bwd(q, k, v, do, 0.6, causal)
    # shifting every key row by the same vector leaves every softmax unchanged
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # the weights of each row sum to one: dV's rows add up to dO's rows
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)
    if causal:
        # keys past the last query row are seen by no row
        assert not dk[lq:].any() and not dv[lq:].any()


def test_bwd_varlen_equals_dense_slices():
    rng = np.random.default_rng(8)
    h, d = 2, 4
    lens = [3, 0, 5, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t = int(cu[-1]) + 2  # two tokens past the last sequence
    q, k, v, do = (_rand(rng, t, h, d) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = sdpa_compact_varlen_bwd(q, k, v, do, cu, cu, 0.7, causal)
        for z in range(len(lens)):
            s, e = cu[z], cu[z + 1]
            for hh in range(h):
                ref = attention_head_bwd(q[s:e, hh], k[s:e, hh], v[s:e, hh], do[s:e, hh], 0.7,
                                         causal)
                for got, r in zip((dq, dk, dv), ref):
                    np.testing.assert_array_equal(got[s:e, hh], r)
        for g in (dq, dk, dv):
            assert not g[cu[-1]:].any()
    # padded: batch b keeps rows/keys 0..len-1 of its own slab
    b_, smax = 3, 6
    lq = [4, 6, 1]
    cu_p = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    qp, kp, vp, dop = (_rand(rng, b_, h, smax, d) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = sdpa_padded_varlen_bwd(qp, kp, vp, dop, cu_p, cu_p, 0.7, causal)
        ref = sdpa_dense_bwd(qp[:, :, :4], kp[:, :, :4], vp[:, :, :4], dop[:, :, :4], 0.7,
                             causal, heads=[(0, 0), (0, 1)])
        for got, r in zip((dq, dk, dv), ref):
            np.testing.assert_array_equal(got[0, :, :4], r[0])
        for g in (dq, dk, dv):
            assert not g[0, :, 4:].any() and not g[2, :, 1:].any()
