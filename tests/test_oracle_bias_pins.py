"""Pins for the oracle's additive bias (scores = scale * Q K^T + bias), against
things other than the oracle itself.

The AOTriton PR #31 keeps a rank-4 bias input in its forward calls (opening
comment, note 1); the nvFuser issue #2278 points at PyTorch's
scaled_dot_product_attention, whose floating attn_mask is added to the scaled
scores.  A slip in the bias path (added before the scale, added to the wrong
index, transposed, dropped from the logsumexp, the -inf entries mishandled,
the wrong block taken in a varlen mode) fails at least one pin:

* PyTorch's CPU attention with a float attn_mask, in float64 (library check);
* a pure-Python brute force in another algebraic form (weights as exp of
  each score over the sum of exps, logsumexp through math.fsum);
* closed forms: zero queries with bias log(w) give the w-weighted mean of V
  and LSE = log(sum w); a -inf bias everywhere but one key selects that key's
  value; a row-constant bias shifts only the logsumexp;
* a bias of 0 / -inf above the diagonal equals the causal mask; a fully -inf
  row behaves as a row with no key;
* broadcast (stride-0) biases equal their materialised copies;
* the varlen modes equal dense attention with the bias block of each
  sequence.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_head, sdpa_compact_varlen, sdpa_dense, sdpa_padded_varlen


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(rng, lq, lk, d, dv=None):
    dv = d if dv is None else dv
    return (rng.standard_normal((lq, d)), rng.standard_normal((lk, d)),
            rng.standard_normal((lk, dv)))


@pytest.mark.parametrize("shape", [(1, 1, 5, 7, 4), (2, 3, 33, 20, 16), (1, 2, 64, 130, 8)])
def test_bias_against_torch_sdpa_fp64(shape):
    B, H, Sq, Sk, D = shape
    rng = _rng(sum(shape))
    q = rng.standard_normal((B, H, Sq, D))
    k = rng.standard_normal((B, H, Sk, D))
    v = rng.standard_normal((B, H, Sk, D))
    bias = rng.standard_normal((B, H, Sq, Sk)) * 2.0
    scale = 0.37
    o, lse = sdpa_dense(q, k, v, scale, False, bias=bias)
    tq, tk, tv, tb = (torch.from_numpy(x) for x in (q, k, v, bias))
    ref_o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tb,
                                                             scale=scale)
    ref_lse = torch.logsumexp(torch.matmul(tq, tk.transpose(-1, -2)) * scale + tb, dim=-1)
    np.testing.assert_allclose(o, ref_o.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=0, atol=1e-12)


def _brute(q, k, v, scale, causal, bias):
    """Pure-Python loops: each weight is exp(s_ij) / sum_j exp(s_ij) taken
    after subtracting the plain Python max, and the logsumexp through
    math.fsum."""
    lq, lk = len(q), len(k)
    out, lse = [], []
    for i in range(lq):
        scores = []
        for j in range(lk):
            if causal and j > i:
                continue
            if bias[i][j] == -math.inf:
                continue
            dot = math.fsum(q[i][d] * k[j][d] for d in range(len(q[i])))
            scores.append((j, dot * scale + bias[i][j]))
        if not scores:
            out.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        top = max(sc for _, sc in scores)
        ex = [(j, math.exp(sc - top)) for j, sc in scores]
        tot = math.fsum(e for _, e in ex)
        out.append([math.fsum(e * v[j][d] for j, e in ex) / tot for d in range(len(v[0]))])
        lse.append(top + math.log(tot))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_bias_brute_force_tiny(seed, causal):
    rng = _rng(100 + seed)
    lq, lk, d = int(rng.integers(1, 7)), int(rng.integers(1, 8)), int(rng.integers(1, 6))
    q, k, v = _qkv(rng, lq, lk, d, dv=3)
    bias = rng.standard_normal((lq, lk)) * 3.0
    bias[rng.random((lq, lk)) < 0.2] = -np.inf
    o, lse = attention_head(q, k, v, 0.6, causal, bias=bias)
    bo, bl = _brute(q.tolist(), k.tolist(), v.tolist(), 0.6, causal, bias.tolist())
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=0, atol=1e-12)


def test_zero_queries_log_weights_give_weighted_mean():
    """Q = 0 leaves only the bias: with bias_ij = log w_ij the output is the
    w-weighted mean of V and LSE_i = log sum_j w_ij."""
    rng = _rng(7)
    lq, lk, d = 6, 9, 5
    w = rng.uniform(0.1, 3.0, size=(lq, lk))
    v = rng.standard_normal((lk, d))
    o, lse = attention_head(np.zeros((lq, d)), rng.standard_normal((lk, d)), v, 0.9, False,
                            bias=np.log(w))
    np.testing.assert_allclose(o, (w @ v) / w.sum(axis=1, keepdims=True), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(w.sum(axis=1)), rtol=0, atol=1e-13)


def test_one_open_key_per_row_selects_it():
    rng = _rng(8)
    lq, lk, d = 7, 11, 4
    q, k, v = _qkv(rng, lq, lk, d)
    pick = rng.integers(0, lk, size=lq)
    bias = np.full((lq, lk), -np.inf)
    extra = rng.standard_normal(lq)
    bias[np.arange(lq), pick] = extra
    o, lse = attention_head(q, k, v, 0.5, False, bias=bias)
    np.testing.assert_array_equal(o, v[pick])
    s = 0.5 * np.einsum("id,id->i", q, k[pick]) + extra
    np.testing.assert_allclose(lse, s, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_row_constant_bias_shifts_only_lse(causal):
    rng = _rng(9)
    q, k, v = _qkv(rng, 12, 12, 6)
    c = rng.standard_normal(12) * 5.0
    o0, l0 = attention_head(q, k, v, 0.4, causal)
    o1, l1 = attention_head(q, k, v, 0.4, causal, bias=np.repeat(c[:, None], 12, axis=1))
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l0 + c, rtol=0, atol=1e-12)


def test_causal_bias_equals_causal_mask():
    rng = _rng(10)
    q, k, v = _qkv(rng, 10, 14, 5)
    b = rng.standard_normal((10, 14))
    upper = np.triu(np.ones((10, 14), dtype=bool), k=1)
    o1, l1 = attention_head(q, k, v, 0.7, False, bias=np.where(upper, -np.inf, b))
    o2, l2 = attention_head(q, k, v, 0.7, True, bias=b)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)


def test_fully_masked_row_has_no_key():
    rng = _rng(11)
    q, k, v = _qkv(rng, 4, 5, 3)
    bias = rng.standard_normal((4, 5))
    bias[2] = -np.inf
    bias[0, 1:] = -np.inf  # row 0 under the causal mask: key 0 only, and it stays open
    o, lse = attention_head(q, k, v, 1.0, True, bias=bias)
    assert (o[2] == 0).all() and lse[2] == -np.inf
    np.testing.assert_array_equal(o[0], v[0])
    bias[0, 0] = -np.inf  # now row 0 sees nothing either
    o, lse = attention_head(q, k, v, 1.0, True, bias=bias)
    assert (o[0] == 0).all() and lse[0] == -np.inf


def test_bias_validation():
    q, k, v = _qkv(_rng(12), 3, 4, 2)
    with pytest.raises(ValueError):
        attention_head(q, k, v, 1.0, False, bias=np.zeros((4, 3)))
    with pytest.raises(ValueError):
        attention_head(q, k, v, 1.0, False, bias=np.full((3, 4), np.nan))
    with pytest.raises(ValueError):
        attention_head(q, k, v, 1.0, False, bias=np.full((3, 4), np.inf))


def test_broadcast_bias_equals_materialised():
    rng = _rng(13)
    B, H, Sq, Sk, D = 2, 3, 9, 11, 4
    q = rng.standard_normal((B, H, Sq, D))
    k = rng.standard_normal((B, H, Sk, D))
    v = rng.standard_normal((B, H, Sk, D))
    for shape in [(1, 1, 1, Sk), (B, 1, Sq, Sk), (1, H, 1, Sk)]:
        small = rng.standard_normal(shape)
        full = np.ascontiguousarray(np.broadcast_to(small, (B, H, Sq, Sk)))
        a = sdpa_dense(q, k, v, 0.5, True, bias=small)
        b = sdpa_dense(q, k, v, 0.5, True, bias=full)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_compact_bias_equals_dense_on_blocks(causal):
    rng = _rng(14)
    lq, lk = [3, 0, 17, 8], [5, 2, 17, 1]
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    cu_k = np.concatenate([[0], np.cumsum(lk)])
    H, D = 2, 6
    q = rng.standard_normal((cu_q[-1], H, D))
    k = rng.standard_normal((cu_k[-1], H, D))
    v = rng.standard_normal((cu_k[-1], H, D))
    bias = rng.standard_normal((1, H, cu_q[-1], cu_k[-1]))
    o, lse = sdpa_compact_varlen(q, k, v, cu_q, cu_k, 0.3, causal, bias=bias)
    for z in range(len(lq)):
        qs, qe, ks, ke = cu_q[z], cu_q[z + 1], cu_k[z], cu_k[z + 1]
        if qe == qs:
            continue
        ro, rl = sdpa_dense(q[None, qs:qe].transpose(0, 2, 1, 3), k[None, ks:ke].transpose(0, 2, 1, 3),
                            v[None, ks:ke].transpose(0, 2, 1, 3), 0.3, causal,
                            bias=bias[:, :, qs:qe, ks:ke])
        np.testing.assert_array_equal(o[qs:qe], ro[0].transpose(1, 0, 2))
        np.testing.assert_array_equal(lse[:, qs:qe], rl[0])


@pytest.mark.parametrize("causal", [False, True])
def test_padded_bias_equals_dense_truncated(causal):
    rng = _rng(15)
    B, H, S, D = 3, 2, 12, 5
    lq, lk = [12, 4, 1], [7, 12, 3]
    q = rng.standard_normal((B, H, S, D))
    k = rng.standard_normal((B, H, S, D))
    v = rng.standard_normal((B, H, S, D))
    bias = rng.standard_normal((B, H, S, S))
    cu = lambda ls: np.concatenate([[0], np.cumsum(ls)])
    o, lse = sdpa_padded_varlen(q, k, v, cu(lq), cu(lk), 0.45, causal, bias=bias)
    for b in range(B):
        ro, rl = sdpa_dense(q[b:b + 1, :, :lq[b]], k[b:b + 1, :, :lk[b]], v[b:b + 1, :, :lk[b]],
                            0.45, causal, bias=bias[b:b + 1, :, :lq[b], :lk[b]])
        np.testing.assert_array_equal(o[b, :, :lq[b]], ro[0])
        np.testing.assert_array_equal(lse[b, :, :lq[b]], rl[0])
