"""Plain float64 CPU oracle for the attention forward pass (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module.  It shares no code with the HIP library and
imports nothing from it.

What is computed
----------------
The pages name the operation without writing it out: the nvFuser issue #2278
"Investigate a new SDPA IR node" (Priya2698's meeting summary) pairs a forward
SDPA node with a backward one and points at PyTorch's
``scaled_dot_product_attention``; the AOTriton PR #31 "Add varlen support to
AOTriton's Flash Attention" (opening comment) adds the variable-length forward.
The plainest reading, used here, is for one (batch or sequence, head) with
``Lq`` query rows and ``Lk`` key rows::

    S[i, j]  = scale * sum_d Q[i, d] * K[j, d]
    allowed  = (j < Lk) and (not causal or j <= i)      # top-left causal
    m[i]     = max_{allowed j} S[i, j]
    P[i, j]  = exp(S[i, j] - m[i]) if allowed else 0
    l[i]     = sum_j P[i, j]
    O[i, :]  = sum_j (P[i, j] / l[i]) * V[j, :]
    LSE[i]   = m[i] + ln(l[i])                          # natural log

A row with no allowed key (only possible when ``Lk == 0``) has ``O = 0`` and
``LSE = -inf``.  The forward returns LSE because the nvFuser issue's discussion
(IvanYashchuk's and jjsjann123's replies) leaves it to the forward to hand the
backward what it cannot cheaply recompute; one number per query row is enough
to rebuild P.

Additive bias.  The AOTriton PR #31 (opening comment, note 1) keeps a rank-4
bias tensor input ``b`` in every forward call, reserved there; the nvFuser
issue points at PyTorch's ``scaled_dot_product_attention``, whose floating
``attn_mask`` is added to the scaled scores.  With a bias the scores are::

    S[i, j]  = scale * sum_d Q[i, d] * K[j, d] + bias[i, j]

and everything else is unchanged.  Bias entries may be -inf (a key the row
must not see); a row whose allowed scores are all -inf is treated like a row
with no allowed key (``O = 0``, ``LSE = -inf``).  The bias view is indexed
like the scores of the rank-4 view: in the compact layout it is (1, H, Tq,
Tk) and sequence z reads the block at rows ``cu_q[z]..`` and columns
``cu_k[z]..``; in the padded layout batch b reads rows and columns from 0.

Causal alignment when ``Lq != Lk`` is not stated on the pages; this oracle
takes the top-left reading (query i sees keys 0..i, local indices), which is
what PyTorch's ``is_causal`` does.

The three modes differ only in which rows and keys form each (sequence, head):

* dense BHSD: batch b uses all ``Sq`` rows of Q[b, h] and ``Sk`` rows of K/V;
* compact varlen (AOTriton PR #31, opening comment): one batch of packed
  tokens; sequence z owns query tokens ``[cu_q[z], cu_q[z+1])`` and key tokens
  ``[cu_k[z], cu_k[z+1])``; no attention crosses sequences;
* padded varlen (AOTriton PR #31, the fwd_kernel.py excerpt in xinyazhang's
  last code reply): batch b keeps its own rank-4 slab, its true lengths are the
  differences ``cu[b+1] - cu[b]`` and its rows and keys start at offset 0.

Everything is float64.  Inputs of lower precision convert exactly.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "attention_head",
    "sdpa_dense",
    "sdpa_compact_varlen",
    "sdpa_padded_varlen",
    "lengths_from_cu",
]


def attention_head(q, k, v, scale, causal, rows=None, bias=None):
    """Attention of one (sequence, head) in float64, score matrix materialised.

    q: (Lq, D), k: (Lk, D), v: (Lk, Dv).  ``rows`` optionally selects which
    local query indices to compute (their causal limit is still their own
    index).  ``bias`` (optional) is (Lq, Lk), added to the scaled scores.
    Returns ``(O, LSE)`` with shapes ``(len(rows), Dv)`` and ``(len(rows),)``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    if v.shape[0] != lk:
        raise ValueError("K and V must have the same number of rows")
    if q.ndim != 2 or k.ndim != 2 or q.shape[1] != k.shape[1]:
        raise ValueError("Q and K must be (rows, D) with the same D")
    if rows is None:
        rows = np.arange(lq)
    rows = np.asarray(rows, dtype=np.int64)
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float64)
        if bias.shape != (lq, lk):
            raise ValueError(f"bias must be (Lq, Lk) = {(lq, lk)}, got {bias.shape}")
        if np.isnan(bias).any() or (bias == np.inf).any():
            raise ValueError("bias entries must be finite or -inf")
    dv = v.shape[1]
    out = np.zeros((rows.size, dv), dtype=np.float64)
    lse = np.full((rows.size,), -np.inf, dtype=np.float64)
    if rows.size == 0 or lk == 0:
        return out, lse

    # Step 1: scaled scores (one library matmul), plus the bias.
    s = float(scale) * (q[rows] @ k.T)
    if bias is not None:
        s = s + bias[rows]
    # Step 2: which keys each row may see (a -inf score is never seen).
    key_idx = np.arange(lk)[None, :]
    allowed = np.ones((rows.size, lk), dtype=bool)
    if causal:
        allowed = key_idx <= rows[:, None]
    allowed = allowed & (s > -np.inf)
    has_key = allowed.any(axis=1)
    # Step 3: row max over allowed keys, exponentials, row sums.
    s_masked = np.where(allowed, s, -np.inf)
    m = s_masked.max(axis=1)
    m_safe = np.where(has_key, m, 0.0)
    p = np.where(allowed, np.exp(s_masked - m_safe[:, None]), 0.0)
    l = p.sum(axis=1)
    # Step 4: normalised weights times V, and the natural-log logsumexp.
    l_safe = np.where(has_key, l, 1.0)
    out = (p / l_safe[:, None]) @ v
    lse = np.where(has_key, m_safe + np.log(l_safe), -np.inf)
    out[~has_key] = 0.0
    return out, lse


def lengths_from_cu(cu, total=None):
    """Per-sequence lengths from an int32 exclusive prefix-sum array.

    The AOTriton PR #31 excerpt takes each length as the difference of two
    neighbouring ``cu_seqlens`` entries.  ``cu`` must start at 0 and never
    decrease; ``total`` (if given) bounds the last entry.
    """
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2:
        raise ValueError("cu_seqlens needs at least two entries")
    if cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0")
    lengths = np.diff(cu)
    if (lengths < 0).any():
        raise ValueError("cu_seqlens must be non-decreasing")
    if total is not None and cu[-1] > total:
        raise ValueError("cu_seqlens ends past the token count")
    return lengths


def _bias_view(bias, shape):
    """The bias as a float64 array broadcast to ``shape`` (stride-0 views of a
    smaller bias, as PyTorch broadcasts ``attn_mask``), or None."""
    if bias is None:
        return None
    return np.broadcast_to(np.asarray(bias, dtype=np.float64), shape)


def sdpa_dense(q, k, v, scale, causal, heads=None, bias=None):
    """Dense BHSD forward.  q: (B,H,Sq,D), k/v: (B,H,Sk,D), bias (optional)
    broadcastable to (B,H,Sq,Sk).

    Returns ``(O, LSE)`` shaped (B,H,Sq,Dv) and (B,H,Sq).  ``heads``
    optionally restricts the work to a list of (b, h) pairs; the other
    entries are left as NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, h_, sq, _ = q.shape
    bias = _bias_view(bias, (b_, h_, sq, k.shape[2]))
    out = np.full(q.shape[:3] + (v.shape[3],), np.nan)
    lse = np.full((b_, h_, sq), np.nan)
    pairs = [(b, h) for b in range(b_) for h in range(h_)] if heads is None else heads
    for b, h in pairs:
        out[b, h], lse[b, h] = attention_head(q[b, h], k[b, h], v[b, h], scale, causal,
                                              bias=None if bias is None else bias[b, h])
    return out, lse


def sdpa_compact_varlen(q, k, v, cu_q, cu_k, scale, causal, bias=None):
    """Compact variable-length forward over packed THD tokens.

    q: (Tq, H, D), k/v: (Tk, H, D).  Sequence z owns query tokens
    ``[cu_q[z], cu_q[z+1])`` and key tokens ``[cu_k[z], cu_k[z+1])``; the mask
    uses indices local to the sequence.  ``bias`` (optional) is broadcastable
    to (1, H, Tq, Tk); sequence z reads its block of it.  Returns ``(O, LSE)``
    shaped (Tq, H, Dv) and (H, Tq); tokens past ``cu_q[-1]`` stay NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    tq, h_, _ = q.shape
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    lengths_from_cu(cu_q, tq)
    lengths_from_cu(cu_k, k.shape[0])
    if cu_q.size != cu_k.size:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same sequence count")
    bias = _bias_view(bias, (1, h_, tq, k.shape[0]))
    out = np.full((tq, h_, v.shape[2]), np.nan)
    lse = np.full((h_, tq), np.nan)
    for z in range(cu_q.size - 1):
        qs, qe = cu_q[z], cu_q[z + 1]
        ks, ke = cu_k[z], cu_k[z + 1]
        for h in range(h_):
            o_zh, lse_zh = attention_head(q[qs:qe, h], k[ks:ke, h], v[ks:ke, h], scale, causal,
                                          bias=None if bias is None else bias[0, h, qs:qe, ks:ke])
            out[qs:qe, h] = o_zh
            lse[h, qs:qe] = lse_zh
    return out, lse


def sdpa_padded_varlen(q, k, v, cu_q, cu_k, scale, causal, bias=None):
    """Padded variable-length forward over rank-4 BHSD slabs.

    q: (B,H,Sq_max,D), k/v: (B,H,Sk_max,D), bias (optional) broadcastable to
    (B,H,Sq_max,Sk_max).  Batch b uses rows ``0 .. cu_q[b+1]-cu_q[b]-1`` and
    keys ``0 .. cu_k[b+1]-cu_k[b]-1``.  Rows past a batch's true length are
    not defined and stay NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, h_, sq, _ = q.shape
    lq = lengths_from_cu(cu_q)
    lk = lengths_from_cu(cu_k)
    if lq.size != b_ or lk.size != b_:
        raise ValueError("padded varlen needs B+1 cu_seqlens entries")
    if (lq > sq).any() or (lk > k.shape[2]).any():
        raise ValueError("a true length exceeds the padded length")
    bias = _bias_view(bias, (b_, h_, sq, k.shape[2]))
    out = np.full(q.shape[:3] + (v.shape[3],), np.nan)
    lse = np.full((b_, h_, sq), np.nan)
    for b in range(b_):
        for h in range(h_):
            o_bh, lse_bh = attention_head(
                q[b, h, : lq[b]], k[b, h, : lk[b]], v[b, h, : lk[b]], scale, causal,
                bias=None if bias is None else bias[b, h, : lq[b], : lk[b]],
            )
            out[b, h, : lq[b]] = o_bh
            lse[b, h, : lq[b]] = lse_bh
    return out, lse


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------
# The nvFuser issue #2278 (Priya2698's meeting summary) needs an SdpaOpBwd node
# next to the forward one, and AOTriton PR #31 (opening comment) pairs every
# varlen forward API with a backward one.  The backward of the definition
# above, for an upstream gradient dO of O (the loss is sum(dO * O)), is the
# plain chain rule through O = P V, the row softmax P = softmax(S) over the
# allowed keys, and S = scale * Q K^T:
#
#     dV      = P^T dO
#     dP      = dO V^T
#     delta_i = sum_j P_ij dP_ij  (= sum_d dO_id O_id)
#     dS      = P * (dP - delta[:, None])        (0 where not allowed)
#     dQ      = scale * dS K
#     dK      = scale * dS^T Q
#
# A row with no allowed key has P = 0 and contributes nothing.

__all__ += [
    "attention_head_bwd",
    "sdpa_dense_bwd",
    "sdpa_compact_varlen_bwd",
    "sdpa_padded_varlen_bwd",
]


def attention_head_bwd(q, k, v, do, scale, causal):
    """Gradients of one (sequence, head) in float64.

    q: (Lq, D), k: (Lk, D), v: (Lk, Dv), do: (Lq, Dv).  Returns
    ``(dQ, dK, dV)`` shaped like q, k and v.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if lq == 0 or lk == 0:
        return dq, dk, dv
    # The forward's normalised weights P, step by step as in attention_head.
    s = float(scale) * (q @ k.T)
    allowed = np.ones((lq, lk), dtype=bool)
    if causal:
        allowed = np.arange(lk)[None, :] <= np.arange(lq)[:, None]
    has_key = allowed.any(axis=1)
    s_masked = np.where(allowed, s, -np.inf)
    m = np.where(has_key, s_masked.max(axis=1), 0.0)
    p = np.where(allowed, np.exp(s_masked - m[:, None]), 0.0)
    l = np.where(has_key, p.sum(axis=1), 1.0)
    p = p / l[:, None]
    # Chain rule, one library matmul per product.
    dv = p.T @ do
    dp = do @ v.T
    delta = (p * dp).sum(axis=1)
    ds = p * (dp - delta[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def sdpa_dense_bwd(q, k, v, do, scale, causal, heads=None):
    """Dense BHSD backward: returns (dQ, dK, dV) shaped like q, k, v.

    ``heads`` optionally restricts the work to a list of (b, h) pairs; the
    other entries are left as NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    b_, h_ = q.shape[:2]
    pairs = [(b, h) for b in range(b_) for h in range(h_)] if heads is None else heads
    for b, h in pairs:
        dq[b, h], dk[b, h], dv[b, h] = attention_head_bwd(q[b, h], k[b, h], v[b, h], do[b, h],
                                                          scale, causal)
    return dq, dk, dv


def sdpa_compact_varlen_bwd(q, k, v, do, cu_q, cu_k, scale, causal):
    """Compact varlen backward over packed THD tokens (q, do: (Tq,H,D); k, v:
    (Tk,H,D)).  Tokens outside every sequence get zero gradients."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    lengths_from_cu(cu_q, q.shape[0])
    lengths_from_cu(cu_k, k.shape[0])
    if cu_q.size != cu_k.size:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same sequence count")
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for z in range(cu_q.size - 1):
        qs, qe = cu_q[z], cu_q[z + 1]
        ks, ke = cu_k[z], cu_k[z + 1]
        for h in range(q.shape[1]):
            g = attention_head_bwd(q[qs:qe, h], k[ks:ke, h], v[ks:ke, h], do[qs:qe, h], scale,
                                   causal)
            dq[qs:qe, h], dk[ks:ke, h], dv[ks:ke, h] = g
    return dq, dk, dv


def sdpa_padded_varlen_bwd(q, k, v, do, cu_q, cu_k, scale, causal):
    """Padded varlen backward over rank-4 slabs; rows and keys past a batch's
    true length get zero gradients (they do not affect any output)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lq = lengths_from_cu(cu_q)
    lk = lengths_from_cu(cu_k)
    b_, h_ = q.shape[:2]
    if lq.size != b_ or lk.size != b_:
        raise ValueError("padded varlen needs B+1 cu_seqlens entries")
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(b_):
        for h in range(h_):
            g = attention_head_bwd(q[b, h, : lq[b]], k[b, h, : lk[b]], v[b, h, : lk[b]],
                                   do[b, h, : lq[b]], scale, causal)
            dq[b, h, : lq[b]], dk[b, h, : lk[b]], dv[b, h, : lk[b]] = g
    return dq, dk, dv
