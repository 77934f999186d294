"""GPU parity of every entry of the compiled-in dispatch table.

The table keys the kernel shape on (dtype, head_dim, sequence-length
bucket, mask and layout).  For every class and every bucket, a dense problem
whose lengths fall in that bucket runs through attn_fwd (both masks: the
dense variants), a compact and a padded problem whose longest sequence has
those lengths run through the varlen calls (both masks: the variable-length
variants), and in the long buckets the forward with a bias and the split
forward (which take the single-group shapes) run too; sampled rows are
compared with the float64 oracle, so each compiled kernel of the committed
library is parity-checked, not only those the small parity shapes happen to
reach.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import attention_head
from parity import check, sample_rows, to64
from scaled_dot_product_03_amd import binding, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (query length, key length) per bucket: query extent <= 128, <= 512,
# <= 4096, longer; key extent <= 512, longer.
BUCKET_SHAPES = [(100, 300), (128, 700), (300, 512), (257, 1500), (1000, 200), (2048, 900),
                 (4200, 64), (4500, 4500)]


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


def _sampled_check(x, o, lse, causal, dt, label, bias=None, heads=((0, 0), (0, 1))):
    rng = np.random.default_rng(7)
    go, gl, ro, rl = [], [], [], []
    for b, h in heads:
        rows = sample_rows(x.q.shape[2], rng, extra=6)
        r_o, r_l = attention_head(to64(x.q[b, h]), to64(x.k[b, h]), to64(x.v[b, h]), x.scale,
                                  causal, rows=rows,
                                  bias=None if bias is None else to64(bias[b, h]))
        go.append(to64(o[b, h, rows]))
        gl.append(to64(lse[b, h, rows]))
        ro.append(r_o)
        rl.append(r_l)
    check(np.concatenate(go), np.concatenate(gl), np.concatenate(ro), np.concatenate(rl), dt,
          label=label)


CLASSES = [("bf16", 128), ("fp16", 128), ("bf16", 64), ("fp16", 64), ("fp32", 64), ("fp32", 128)]


@pytest.mark.parametrize("dt,D", CLASSES)
@pytest.mark.parametrize("bucket", range(len(BUCKET_SHAPES)))
def test_every_table_entry(dt, D, bucket):
    sq, sk = BUCKET_SHAPES[bucket]
    x = inputs.dense_inputs(1, 2, sq, sk, D, dt, seed=500 + bucket)
    q, k, v = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV)
    for causal in (False, True):
        bm, bn, w = binding.kernel_config(inputs.DTYPES[dt], D, sq, sk, causal=causal)
        _log(f"dispatch {dt} D{D} bucket {bucket} Sq{sq} Sk{sk} causal={causal}: block_m {bm} "
             f"block_n {bn} waves {w}")
        o, lse = binding.attn_fwd(q, k, v, scale=x.scale, causal=causal)
        torch.cuda.synchronize()
        _sampled_check(x, o, lse, causal, dt, f"{dt} D{D} bucket {bucket} causal={causal}")


@pytest.mark.parametrize("dt,D", [c for c in CLASSES if c[0] != "fp32"])
@pytest.mark.parametrize("bucket", range(len(BUCKET_SHAPES)))
def test_unmasked_16bit_entries_on_grids_past_one_workgroup_per_cu(dt, D, bucket):
    """A 16-bit launch without the mask runs a four-wave entry as two key
    groups while it has at most 256 workgroups (the small shapes above all
    do); with enough heads to pass that, the entry's own single-group kernel
    runs, and is checked here on two sampled heads."""
    sq, sk = BUCKET_SHAPES[bucket]
    bm, bn, w = binding.kernel_config(inputs.DTYPES[dt], D, sq, sk, causal=False)
    m_tiles = -(-sq // bm)
    H = 256 // m_tiles + 1
    _log(f"dispatch grid > 256 {dt} D{D} bucket {bucket} Sq{sq} Sk{sk}: block_m {bm} waves {w} "
         f"H {H} ({m_tiles * H} workgroups)")
    assert m_tiles * H > 256
    x = inputs.dense_inputs(1, H, sq, sk, D, dt, seed=800 + bucket, causal_modes=(False,))
    q, k, v = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV)
    o, lse = binding.attn_fwd(q, k, v, scale=x.scale, causal=False)
    torch.cuda.synchronize()
    _sampled_check(x, o, lse, False, dt, f"grid>256 {dt} D{D} bucket {bucket}",
                   heads=((0, 0), (0, H - 1)))


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("fp16", 64)])
@pytest.mark.parametrize("bucket", [5, 7])
def test_single_group_entries_with_bias_and_split(dt, D, bucket):
    sq, sk = BUCKET_SHAPES[bucket]
    _log(f"dispatch single-group {dt} D{D} bucket {bucket}")
    x = inputs.dense_inputs(1, 2, sq, sk, D, dt, seed=600 + bucket)
    q, k, v = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV)
    bias = inputs.bias_tensor((1, 2, sq, sk), dt, seed=601)
    pad = (sk + 7) // 8 * 8
    bd = torch.empty((1, 2, sq, pad), dtype=q.dtype, device=DEV)[..., :sk]
    bd.copy_(bias)
    o, lse = binding.attn_fwd(q, k, v, scale=x.scale, causal=True, bias=bd)
    torch.cuda.synchronize()
    _sampled_check(x, o, lse, True, dt, f"bias {dt} D{D} bucket {bucket}", bias=bias)
    o, lse = binding.attn_fwd_splitk(q, k, v, scale=x.scale, causal=False)
    torch.cuda.synchronize()
    _sampled_check(x, o, lse, False, dt, f"split {dt} D{D} bucket {bucket}")


@pytest.mark.parametrize("dt,D", CLASSES)
@pytest.mark.parametrize("bucket", range(len(BUCKET_SHAPES)))
def test_every_table_entry_varlen(dt, D, bucket):
    """The compact and padded kernels of every entry: two sequences whose
    longest has the bucket's lengths (the dispatch key of the varlen layouts
    is the longest sequence), the other shorter and ragged."""
    sq, sk = BUCKET_SHAPES[bucket]
    lq, lk = [sq, max(1, sq // 3 + 5)], [sk, max(1, sk // 2 + 3)]
    H = 2
    rng = np.random.default_rng(7)
    for causal in (False, True):
        _log(f"dispatch varlen {dt} D{D} bucket {bucket} causal={causal}")
        x = inputs.compact_inputs(2, H, D, dt, seed=700 + bucket, len_lo=1, len_hi=2,
                                  lengths_q=lq, lengths_k=lk)
        q, k, v = x.q.to(DEV), x.k.to(DEV), x.v.to(DEV)
        o, lse = binding.attn_fwd_compact_varlen(q, k, v, x.cu_seqlens_q, x.cu_seqlens_k,
                                                 scale=x.scale, causal=causal)
        torch.cuda.synchronize()
        go, gl, ro, rl = [], [], [], []
        for z in range(2):
            qs, qe = int(x.cu_seqlens_q[z]), int(x.cu_seqlens_q[z + 1])
            ks, ke = int(x.cu_seqlens_k[z]), int(x.cu_seqlens_k[z + 1])
            rows = sample_rows(qe - qs, rng, extra=4)
            for h in range(H):
                r_o, r_l = attention_head(to64(x.q[qs:qe, h]), to64(x.k[ks:ke, h]),
                                          to64(x.v[ks:ke, h]), x.scale, causal, rows=rows)
                go.append(to64(o[qs + rows, h]))
                gl.append(to64(lse[0, h, qs + rows]))
                ro.append(r_o)
                rl.append(r_l)
        check(np.concatenate(go), np.concatenate(gl), np.concatenate(ro), np.concatenate(rl), dt,
              label=f"compact {dt} D{D} bucket {bucket} causal={causal}")
        # the same two sequences as padded batches of the longest lengths
        xp = inputs.padded_inputs(2, H, sq, sk, D, dt, seed=710 + bucket, len_lo=1, len_hi=2,
                                  lengths_q=lq, lengths_k=lk)
        o, lse = binding.attn_fwd_padded_varlen(xp.q.to(DEV), xp.k.to(DEV), xp.v.to(DEV),
                                                xp.cu_seqlens_q, xp.cu_seqlens_k, scale=xp.scale,
                                                causal=causal)
        torch.cuda.synchronize()
        go, gl, ro, rl = [], [], [], []
        for b in range(2):
            rows = sample_rows(lq[b], rng, extra=4)
            for h in range(H):
                r_o, r_l = attention_head(to64(xp.q[b, h, :lq[b]]), to64(xp.k[b, h, :lk[b]]),
                                          to64(xp.v[b, h, :lk[b]]), xp.scale, causal, rows=rows)
                go.append(to64(o[b, h, rows]))
                gl.append(to64(lse[b, h, rows]))
                ro.append(r_o)
                rl.append(r_l)
        check(np.concatenate(go), np.concatenate(gl), np.concatenate(ro), np.concatenate(rl), dt,
              label=f"padded {dt} D{D} bucket {bucket} causal={causal}")
