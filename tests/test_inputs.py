"""The seeded input generator: reproducible draws and the workload sizes."""

import json
import os

import numpy as np
import torch

from scaled_dot_product_03_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_varlen_lengths_match_golden():
    with open(os.path.join(GOLDEN, "varlen_lengths.json")) as f:
        g = json.load(f)
    rng = np.random.default_rng(4)
    assert rng.integers(1, 4096, size=16, endpoint=True).tolist() == g["thd_seed4"]
    rng = np.random.default_rng(5)
    lengths = rng.integers(2048, 8192, size=8, endpoint=True)
    assert lengths.tolist() == g["padded_seed5"]
    assert inputs.cu_from_lengths(lengths).tolist() == g["padded_seed5_cu"]
    assert sum(g["thd_seed4"]) == g["thd_seed4_total"]


def test_small_compact_inputs_follow_recipe():
    x = inputs.compact_inputs(n_seqs=5, H=2, D=8, dtype="bf16", seed=4, len_lo=1, len_hi=40)
    rng = np.random.default_rng(4)
    lengths = rng.integers(1, 40, size=5, endpoint=True)
    assert x.meta["lengths_q"] == lengths.tolist()
    assert x.cu_seqlens_q.dtype == np.int32
    assert x.cu_seqlens_q.tolist() == [0] + np.cumsum(lengths).tolist()
    t = int(lengths.sum())
    q = torch.from_numpy(rng.standard_normal((t, 2, 8), dtype=np.float32)).to(torch.bfloat16)
    assert torch.equal(x.q, q)
    assert x.q.shape == (t, 2, 8) and x.q.dtype == torch.bfloat16


def test_same_seed_same_tensors_and_rne_rounding():
    a = inputs.dense_inputs(1, 2, 8, 9, 16, "fp16", seed=3)
    b = inputs.dense_inputs(1, 2, 8, 9, 16, "fp16", seed=3)
    assert torch.equal(a.q, b.q) and torch.equal(a.v, b.v)
    rng = np.random.default_rng(3)
    q32 = rng.standard_normal((1, 2, 8, 16), dtype=np.float32)
    # round-to-nearest-even to fp16, as numpy does it independently
    assert np.array_equal(a.q.numpy(), q32.astype(np.float16))
    assert a.scale == float(np.float32(0.25))


def test_workload_table_shapes():
    names = list(inputs.WORKLOADS)
    assert len(names) == 5
    kw = inputs.WORKLOADS["dense_bf16_b4h16s2048d128"][1]
    assert (kw["B"], kw["H"], kw["Sq"], kw["Sk"], kw["D"], kw["dtype"]) == (4, 16, 2048, 2048, 128, "bf16")
    kw = inputs.WORKLOADS["dense_fp16_b2h32sq512sk8192d64"][1]
    assert (kw["Sq"], kw["Sk"], kw["D"], kw["dtype"]) == (512, 8192, 64, "fp16")
    tiny = inputs.workload("tiny_dense_fp32_b1h2s128d64")
    assert tiny.q.shape == (1, 2, 128, 64) and tiny.q.dtype == torch.float32
    assert tiny.scale == 0.125 and tiny.causal_modes == (False, True)
