#!/usr/bin/env python3
"""Benchmark of the flash-attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

One step is one pass of the whole forward path over the dense bf16 BHSD
workload B=4, H=16, Sq=Sk=2048, D=128 with scale 1/sqrt(128): the
non-causal forward followed by the causal forward (both masks of that
workload), inputs resident in HBM.  FLOPs are 4*Sq*Sk*D*H*B per forward,
halved for causal.  The line also carries the compact varlen THD workload
(16 sequences, lengths U{1..4096} from seed 4, H=16, D=128, bf16, causal), the
padded varlen workload (B=8, H=32, 8192-row slabs, true lengths U{2048..8192}
from seed 5, D=128, bf16, causal; FLOPs over the true lengths)
and the fp16 B=2, H=32, Sq=512, Sk=8192, D=64 workload (through attn_fwd
and through the key-parallel attn_fwd_splitk), the dense workload with a full
(B, H, Sq, Sk) additive bias, and the backward of the dense workload timed
the same way, a roofline record for the dominant kernel (the
non-causal forward, timed with HIP events on the stream it runs on around the
block of its back-to-back launches) and the float64 CPU oracle timed on a bounded sample of the same
workload.

Prints ONE JSON line on stdout.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s & % MFMA peak (bf16 BHSD S=2048 D=128; varlen THD)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0

from scaled_dot_product_03_amd.rocprof import (  # noqa: E402
    clock_from_profiles, kernel_source_hash, traffic_from_profiles)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dense_flops(B, H, Sq, Sk, D, causal):
    f = 4.0 * Sq * Sk * D * H * B
    return f / 2 if causal else f


def varlen_flops(lengths, H, D, causal):
    f = sum(4.0 * L * L * D * H for L in lengths)
    return f / 2 if causal else f


SETTLE_S = 0.25  # untimed sustained load before each timed block
COLD_MIB = 512  # written between cold launches: twice the 256 MB MALL


def settle(call, torch, seconds=SETTLE_S):
    """Runs `call` back to back, untimed, for `seconds` of wall time.  The GPU
    raises its clocks only under sustained load (a 5-step warmup after the
    host spent seconds generating inputs times the clock ramp, not the
    kernel: 0.163 ms against 0.134 ms for the dense non-causal forward), so
    every timed block starts from steady clocks."""
    t_end = time.perf_counter() + seconds
    n = 0
    while n == 0 or time.perf_counter() < t_end:
        call()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()  # keep the host within a few launches of the GPU
    torch.cuda.synchronize()


def launch_stats(call, torch, stream, n, cold_buf=None):
    """Median and minimum duration (ms) of n launches of `call`, each between
    its own pair of HIP events on the launch stream, after 10 untimed ones.
    The events add their own processing to every sample, so these sit a few
    microseconds above the block averages.  With `cold_buf`, the buffer is
    overwritten before every launch (outside its events), so neither the
    L2 caches nor the MALL hold any of the inputs when the launch starts."""
    for _ in range(10):
        call()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        if cold_buf is not None:
            cold_buf.fill_(i & 0xFF)
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    return {"launches": n, "median_ms": float(np.median(t)), "min_ms": t[0], "max_ms": t[-1]}


def cpu_baseline(x, budget_s=12.0):
    """The float64 oracle, as it is, on a bounded sample of the workload's
    heads (both masks), on this host's cores."""
    from oracle import attention_head
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default
        threads = os.cpu_count() or 1
    B, H, Sq, D = x.q.shape
    Sk = x.k.shape[2]
    pairs = [(b, h) for b in range(B) for h in range(H)]
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    for b, h in pairs:
        q = x.q[b, h].double().numpy()
        k = x.k[b, h].double().numpy()
        v = x.v[b, h].double().numpy()
        for causal in x.causal_modes:
            attention_head(q, k, v, x.scale, causal)
            flops += dense_flops(1, 1, Sq, Sk, D, causal)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{done} of {len(pairs)} (batch, head) pairs of B{B} H{H} S{Sq} D{D} bf16 "
                  f"(inputs widened to fp64), non-causal + causal, {dt:.1f} s wall",
        "cpu_model": _cpu_model(), "host_cpu_count": os.cpu_count(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-padded", action="store_true",
                    help="skip the padded varlen workload (B8 H32 Smax 8192 D128)")
    ap.add_argument("--no-splitk", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-bias", action="store_true")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of untimed back-to-back calls before each timed block")
    ap.add_argument("--launch-stats", type=int, default=50,
                    help="launches per mask for the per-launch median/min (warm and cold MALL) "
                         "of the headline kernels; 0 skips them")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB (a kernel of "
                         "known HBM traffic, for scaling counter readings)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the kernels are single-GPU; --gpus {args.gpus} "
              "is not supported)", file=sys.stderr)
        sys.exit(2)

    import torch
    from scaled_dot_product_03_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    binding.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    wl = "dense_bf16_b4h16s2048d128"
    x = inputs.workload(wl)
    B, H, Sq, D = x.q.shape
    Sk = x.k.shape[2]
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    f_nc = dense_flops(B, H, Sq, Sk, D, False)
    f_c = dense_flops(B, H, Sq, Sk, D, True)

    def fwd_noncausal():
        binding.attn_fwd(q, k, v, scale=x.scale, causal=False, out=o, lse=lse)

    def fwd_causal():
        binding.attn_fwd(q, k, v, scale=x.scale, causal=True, out=o, lse=lse)

    def step():
        fwd_noncausal()
        fwd_causal()

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read + {n} bytes written per launch, 3 launches")
        del src, dst

    log(f"warmup {args.warmup} steps on {wl}, then {args.settle_s} s of untimed steps")
    for _ in range(args.warmup):
        step()
    settle(step, torch, args.settle_s)

    # The timed region runs the K steps' non-causal forwards back to back, then
    # their causal forwards, with HIP events on the launch stream only at the
    # three block boundaries: per-launch events would add each launch's
    # dispatch latency to the kernel average.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(args.steps):
        fwd_noncausal()
    ev[1].record(stream)
    for _ in range(args.steps):
        fwd_causal()
    ev[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps: {wall * 1e3 / args.steps:.3f} ms/step")

    ms_per_step = wall * 1e3 / args.steps
    value = (f_nc + f_c) / (ms_per_step * 1e-3) / 1e12
    nc_avg = ev[0].elapsed_time(ev[1]) / args.steps
    c_avg = ev[1].elapsed_time(ev[2]) / args.steps
    achieved = f_nc / (nc_avg * 1e-3) / 1e12
    traffic = traffic_from_profiles()
    clock = clock_from_profiles()

    breakdown = {
        "noncausal": {"flops": f_nc, "avg_ms": nc_avg, "tflops": achieved,
                      "pct_mfma_peak": 100 * achieved / PEAK_BF16_TFLOPS},
        "causal": {"flops": f_c, "avg_ms": c_avg, "tflops": f_c / (c_avg * 1e-3) / 1e12,
                   "pct_mfma_peak": 100 * f_c / (c_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
    }

    def block_ms(call, n=None):
        """Average ms of `call` over n (default args.steps) back-to-back calls
        (after warmup and a clock-settling phase), from two HIP events on the
        launch stream."""
        n = n or args.steps
        for _ in range(args.warmup):
            call()
        settle(call, torch, args.settle_s)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        e[0].record(stream)
        for _ in range(n):
            call()
        e[1].record(stream)
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]) / n

    if args.launch_stats > 0:
        # Per-launch statistics of the headline kernels: warm (inputs resident
        # in the caches as far as they fit, as in the timed steps) and cold.
        cold = torch.empty(COLD_MIB << 20, dtype=torch.uint8, device=dev)
        for name, call in (("noncausal", fwd_noncausal), ("causal", fwd_causal)):
            settle(call, torch, args.settle_s)
            warm = launch_stats(call, torch, stream, args.launch_stats)
            cold_s = launch_stats(call, torch, stream, args.launch_stats, cold_buf=cold)
            breakdown[name]["per_launch"] = {"warm": warm, f"cold_after_{COLD_MIB}MiB_write": cold_s}
        del cold

    if not args.no_varlen:
        vx = inputs.workload("thd_bf16_16seq_len1to4096_h16d128_causal")
        vq, vk, vv = vx.q.to(dev), vx.k.to(dev), vx.v.to(dev)
        cu = torch.from_numpy(vx.cu_seqlens_q).to(dev)
        lengths = vx.meta["lengths_q"]
        maxlen = int(max(lengths))
        vo = torch.empty_like(vq)
        vlse = torch.empty((1, vq.shape[1], vq.shape[0]), dtype=torch.float32, device=dev)
        v_avg = block_ms(lambda: binding.attn_fwd_compact_varlen(
            vq, vk, vv, cu, cu, maxlen, maxlen, scale=vx.scale, causal=True, out=vo, lse=vlse))
        vf = varlen_flops(lengths, vq.shape[1], vq.shape[2], True)
        breakdown["varlen_thd_causal"] = {
            "workload": "thd_bf16_16seq_len1to4096_h16d128_causal (seed 4, T=%d)" % vq.shape[0],
            "flops": vf, "avg_ms": v_avg, "tflops": vf / (v_avg * 1e-3) / 1e12,
            "pct_mfma_peak": 100 * vf / (v_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        del vq, vk, vv, vo, vlse

    if not args.no_padded:
        px = inputs.workload("padded_bf16_b8h32smax8192d128_len2048to8192_causal")
        pq, pk, pv = px.q.to(dev), px.k.to(dev), px.v.to(dev)
        pcu = torch.from_numpy(px.cu_seqlens_q).to(dev)
        plen, pscale = px.meta["lengths_q"], px.scale
        del px
        po = torch.empty_like(pq)
        plse = torch.empty(pq.shape[:3], dtype=torch.float32, device=dev)
        p_avg = block_ms(lambda: binding.attn_fwd_padded_varlen(
            pq, pk, pv, pcu, pcu, scale=pscale, causal=True, out=po, lse=plse),
            min(args.steps, 10))
        pf = varlen_flops(plen, pq.shape[1], pq.shape[3], True)
        breakdown["padded_varlen_causal"] = {
            "workload": "padded_bf16_b8h32smax8192d128_len2048to8192_causal (seed 5, true "
                        "lengths %s)" % list(int(v) for v in plen),
            "flops": pf, "avg_ms": p_avg, "tflops": pf / (p_avg * 1e-3) / 1e12,
            "pct_mfma_peak": 100 * pf / (p_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        del pq, pk, pv, po, plse

    if not args.no_splitk:
        sx = inputs.workload("dense_fp16_b2h32sq512sk8192d64")
        sq, sk, sv = sx.q.to(dev), sx.k.to(dev), sx.v.to(dev)
        sB, sH, sSq, sD = sq.shape
        sSk = sk.shape[2]
        splits, nbytes = binding.splitk_plan(sq.dtype, sB, sH, sSq, sSk, sD)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        so = torch.empty_like(sq)
        slse = torch.empty((sB, sH, sSq), dtype=torch.float32, device=dev)
        calls = {
            "attn_fwd": lambda: binding.attn_fwd(sq, sk, sv, scale=sx.scale, out=so, lse=slse),
            "attn_fwd_splitk": lambda: binding.attn_fwd_splitk(sq, sk, sv, scale=sx.scale, out=so,
                                                               lse=slse, workspace=ws),
        }
        sf = dense_flops(sB, sH, sSq, sSk, sD, False)
        entry = {"workload": "dense_fp16_b2h32sq512sk8192d64 (seed 3), non-causal",
                 "flops": sf, "splits": splits}
        for name, call in calls.items():
            s_avg = block_ms(call)
            entry[name] = {"avg_ms": s_avg, "tflops": sf / (s_avg * 1e-3) / 1e12,
                           "pct_mfma_peak": 100 * sf / (s_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        breakdown["dense_fp16_sq512_sk8192"] = entry
        del sq, sk, sv, so, slse, ws

    if not args.no_bias:
        # The same workload with a full (B, H, Sq, Sk) bf16 additive bias
        # (seeded standard normal, rows padded to 8 elements in memory).  The
        # bias is read once per allowed (row, key) tile, which makes the
        # kernel HBM-bound: algorithmic bytes are Q, K, V, O and LSE plus the
        # bias entries of the loaded key tiles (all of them non-causal; the
        # tiles up to each query tile's diagonal causal).
        bias = inputs.bias_tensor((B, H, Sq, Sk), "bf16", seed=402)
        bpad = (Sk + 7) // 8 * 8
        bd = torch.empty((B, H, Sq, bpad), dtype=q.dtype, device=dev)[..., :Sk]
        bd.copy_(bias)
        del bias
        io_bytes = B * H * (2 * Sq * D * 2 + 2 * Sk * D * 2 + Sq * 4)
        entry = {"workload": "dense_bf16_b4h16s2048d128 (seed 2) + bias (B,H,Sq,Sk) bf16 seed 402"}
        for causal in (False, True):
            b_avg = block_ms(lambda: binding.attn_fwd(q, k, v, scale=x.scale, causal=causal,
                                                      out=o, lse=lse, bias=bd))
            if causal:
                # query tile m reads key tiles 0 .. (m+1)*bm/bn - 1, bm rows each
                bm_ = binding.kernel_config(torch.bfloat16, D, Sq, Sk, causal=True,
                                            single_group=True)[0]
                keys = sum(min(Sk, (m + 1) * bm_) for m in range((Sq + bm_ - 1) // bm_))
                bias_bytes = B * H * bm_ * keys * 2
            else:
                bias_bytes = B * H * Sq * Sk * 2
            hbm = io_bytes + bias_bytes
            bf = dense_flops(B, H, Sq, Sk, D, causal)
            entry["causal" if causal else "noncausal"] = {
                "flops": bf, "avg_ms": b_avg, "tflops": bf / (b_avg * 1e-3) / 1e12,
                "pct_mfma_peak": 100 * bf / (b_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "roofline": {"bound": "hbm", "algorithmic_bytes": hbm,
                             "achieved_gbs": hbm / (b_avg * 1e-3) / 1e9,
                             "frac": hbm / (b_avg * 1e-3) / 1e9 / HBM_PEAK_GBS}}
        breakdown["dense_bf16_s2048_bias"] = entry
        del bd

    if not args.no_bwd:
        # Backward of the same workload: gradients for an upstream dO drawn
        # from the same seeded generator.  FLOPs are the five products of the
        # method (S, dP, dV, dK, dQ: 2.5x the forward's), halved for causal;
        # the kernels recompute S and dP once more than that.
        rng = np.random.default_rng(2 + 1000)
        dout = torch.from_numpy(rng.standard_normal(tuple(x.q.shape), dtype=np.float32)).to(
            x.q.dtype).to(dev)
        ws = torch.empty(binding.bwd_workspace_bytes(B, H, Sq), dtype=torch.uint8, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bwd = {"workload": "dense_bf16_b4h16s2048d128 (seed 2), dO seed 1002"}
        for causal in (False, True):
            bo, blse = binding.attn_fwd(q, k, v, scale=x.scale, causal=causal)
            b_avg = block_ms(lambda: binding.attn_bwd(q, k, v, bo, dout, blse, scale=x.scale,
                                                      causal=causal, dq=dq, dk=dk, dv=dv,
                                                      workspace=ws))
            bf = 2.5 * dense_flops(B, H, Sq, Sk, D, causal)
            bwd["causal" if causal else "noncausal"] = {
                "flops": bf, "avg_ms": b_avg, "tflops": bf / (b_avg * 1e-3) / 1e12,
                "pct_mfma_peak": 100 * bf / (b_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        breakdown["backward_dense_bf16_s2048"] = bwd
        del dout, ws, dq, dk, dv, bo, blse

    bm, bn, waves = binding.kernel_config(torch.bfloat16, D, Sq, Sk)
    record = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense_bf16_b4h16s2048d128: BHSD B=4 H=16 Sq=Sk=2048 D=128 bf16, "
                               "scale 1/sqrt(128), one non-causal + one causal forward per step",
                   "global_batch": B, "seq_len": Sq, "heads": H, "head_dim": D,
                   "parallelism": "single GPU",
                   "kernel": {"block_m": bm, "block_n": bn, "waves": waves}},
        "pct_mfma_peak": 100 * value / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "shader_clock_ghz": clock,
                     "frac_at_shader_clock": (achieved / (PEAK_BF16_TFLOPS * clock / 2.4)
                                              if clock else None),
                     "clock_source": "GRBM_GUI_ACTIVE per XCD over the dispatch duration in the "
                                     "committed rocprofv3 counter pass of these kernel sources "
                                     "(null when the sources changed since)",
                     "kernel": "attn_fwd_kernel<bf16, D=128, dense, non-causal>",
                     "flops_per_launch": f_nc, "avg_launch_ms": nc_avg},
        "breakdown": breakdown,
        "settle_s_before_each_block": args.settle_s,
        "kernel_source_sha": kernel_source_hash(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the float64 CPU oracle on a bounded sample")
        record["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
