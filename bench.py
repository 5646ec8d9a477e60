#!/usr/bin/env python3
"""Forward-pass benchmark of the exact attention library on one MI355X.

Metric: attention forward TFLOP/s for bf16, causal, head dim 128, N = 8192
(B = 2, H = 16), counting 4*B*H*N^2*d FLOPs halved for causal, and the fraction of
the dense bf16 MFMA peak. One step is one forward pass of the whole path (workgroup
order, Q/K/V loads, both MFMA contractions, masking, online softmax, epilogue) over
one batch of seeded synthetic inputs that are already resident in HBM.

Prints ONE JSON line. Also reported, outside ``value``: the backward pass of the same
bf16 workload (dQ, dK, dV from a seeded dO; 2.5 times the forward FLOPs), the fp8 path
on the fp8 workload (B = 2, H = 16, N = 8192, d = 128, causal: quantiser and attention
timed separately), one split-KV decoding step (B = 16, H = 16, 1 query row against
8192 keys; HBM-bound, reported in GB/s), and the CPU oracle timed on a bounded sample
of the bf16 workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X published dense bf16 MFMA peak
PEAK_FP8_TFLOPS = 5000.0      # MI355X published dense fp8 MFMA peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_H_counters.txt")
KERNEL_SOURCES = ["exact_attention_78_amd/csrc/attn_fwd.hip", "exact_attention_78_amd/csrc/device_common.h"]


def kernel_source_hash() -> str:
    """sha256 of the bf16 kernel's sources with comments and blank space removed, so that a
    comment-only edit does not invalidate the counter summary while any code change does."""
    import re

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = re.sub(r"//[^\n]*", "", f.read())
        h.update("\n".join(line.strip() for line in text.splitlines() if line.strip()).encode())
    return h.hexdigest()


def read_counters(key="hbm_bytes_per_launch"):
    """A figure of the committed rocprofv3 counter summary of the bf16 kernel (HBM bytes per
    launch by default), or None when the summary is missing or was taken on different
    kernel sources."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    for line in open(COUNTERS_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv[key].split()[0])
    except (KeyError, ValueError):
        return None


def counted_flops(B, H, N, d, causal):
    """4*B*H*N^2*d (two N x N x d contractions), halved for causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def timed(fn, steps, warmup, torch):
    """Average time of fn() in ms over `steps` calls on the current stream (HIP events)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def cpu_baseline(q, k, v, causal, scale, budget_s):
    """Time the oracle (as it stands) on whole heads of the workload until the budget is used."""
    from threadpoolctl import threadpool_info

    from oracle.attention import attention_forward

    B, H, N, d = q.shape
    heads = [(b, h) for b in range(B) for h in range(H)]
    done, t0 = 0, time.perf_counter()
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        attention_forward(q[sl], k[sl], v[sl], causal, scale)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = counted_flops(1, done, N, d, causal)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {B * H} heads (all {N} query rows each, causal) of the bf16 B2 H16 N8192 d128 "
                      f"workload, fp64 NumPy, {dt:.1f} s"}


def backward_leg(torch, ea, inputs, w, tensors, o, lse, steps, warmup):
    """The backward pass of the forward call just timed (same inputs, its O and LSE)."""
    gq, gk, gv = tensors
    g = inputs.to_torch(inputs.draw_dout(w.wid, w.B, w.H, w.N, w.d), "bf16").cuda()
    ea.attn_fwd_bf16(gq, gk, gv, causal=True, scale=w.scale, out=o, lse=lse)
    dq, dk, dv = (torch.empty_like(gq) for _ in range(3))
    ws = torch.empty((2, w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    ms = timed(lambda: ea.attn_bwd_bf16(gq, gk, gv, o, lse, g, causal=True, scale=w.scale, dq=dq, dk=dk, dv=dv,
                                        workspace=ws), steps, warmup, torch)
    flops = 2.5 * counted_flops(w.B, w.H, w.N, w.d, True)
    assert all(bool(torch.isfinite(t.float()).all()) for t in (dq, dk, dv))
    return {"workload": "bf16 causal attention backward (dQ, dK, dV), B=2 H=16 N=8192 d=128",
            "us": ms * 1e3, "tflops": flops / (ms * 1e-3) / 1e12,
            "frac_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "flop_convention": "2.5 x forward (five N x N x d contractions), halved for causal"}


def decode_leg(torch, ea, inputs, steps, warmup):
    """One decoding step (split-KV): 1 query row per head against an 8192-key bf16 cache."""
    B, H, Nq, Nk, d = 16, 16, 1, 8192, 128
    q = inputs.to_torch(inputs.normal_f32(7, inputs.Q_ID, (B, H, Nq, d)), "bf16").cuda()
    k = inputs.to_torch(inputs.normal_f32(7, inputs.K_ID, (B, H, Nk, d)), "bf16").cuda()
    v = inputs.to_torch(inputs.normal_f32(7, inputs.V_ID, (B, H, Nk, d)), "bf16").cuda()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(ea.library().attn_decode_workspace_floats(B, H, Nq, Nk, d), dtype=torch.float32, device="cuda")
    ms = timed(lambda: ea.attn_decode_bf16(q, k, v, out=o, lse=lse, workspace=ws), steps, warmup, torch)
    nbytes = 2 * B * H * Nk * d * 2 + 2 * B * H * Nq * d * 2 + B * H * Nq * 4   # K, V, Q read; O, LSE written
    assert bool(torch.isfinite(o.float()).all())
    return {"workload": "bf16 decoding step, B=16 H=16 Nq=1 Nk=8192 d=128, no mask (split-KV)",
            "us": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def fp8_leg(torch, ea, inputs, steps, warmup):
    import numpy as np

    w = inputs.WORKLOADS["C5"]
    q, k, v, signs = inputs.draw_fp8_workload(w.wid, w.B, w.H, w.N, w.d)
    tq, tk, tv = (inputs.to_torch(x, "bf16").cuda() for x in (q, k, v))
    sg = torch.from_numpy(signs).cuda()
    q8, sq = ea.attn_quant_fp8(tq, sg)
    k8, sk = ea.attn_quant_fp8(tk, sg)
    v8, sv = ea.attn_quant_fp8(tv, None)
    o, lse = ea.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=True)

    def quant_all():
        ea.attn_quant_fp8(tq, sg, out=q8, scales=sq)
        ea.attn_quant_fp8(tk, sg, out=k8, scales=sk)
        ea.attn_quant_fp8(tv, None, out=v8, scales=sv)

    ms_q = timed(quant_all, steps, warmup, torch)
    ms_a = timed(lambda: ea.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=True, out=o, lse=lse), steps, warmup, torch)
    flops = counted_flops(w.B, w.H, w.N, w.d, True)
    n = w.B * w.H * w.N * w.d
    nblk = (w.N + 127) // 128
    qbytes = 3 * (2 * n + n + 4 * w.B * w.H * nblk)      # read bf16, write codes + scales
    assert bool(torch.isfinite(o.float()).all())
    return {
        "workload": "fp8 e4m3, causal, B=2 H=16 N=8192 d=128, Hadamard-rotated Q/K with shared outlier channels",
        "attn_us": ms_a * 1e3, "attn_tflops": flops / (ms_a * 1e-3) / 1e12,
        "attn_frac_fp8_peak": flops / (ms_a * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
        "quant_qkv_us": ms_q * 1e3, "quant_gbs": qbytes / (ms_q * 1e-3) / 1e9,
        "quant_frac_hbm": qbytes / (ms_q * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The GPU needs a few tens of milliseconds of sustained load to reach its steady clock;
    # 100 untimed steps (~60 ms here) get there before the timed region starts.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--no-extra", action="store_true", help="skip the backward, fp8 and decode legs")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of 1 GiB x 4 (HBM counter calibration) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one MI355X only: --gpus {args.gpus} (WORLD_SIZE {world}) is not supported; "
              f"run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_78_amd as ea
    from exact_attention_78_amd import inputs

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": 2 * (1 << 30), "launches": 4}))
        return

    w = inputs.WORKLOADS["H"]
    q, k, v = inputs.draw_qkv(w.wid, w.B, w.H, w.N, w.d)
    cpu = tuple(inputs.to_torch(x, "bf16") for x in (q, k, v))
    gq, gk, gv = (t.cuda() for t in cpu)
    o = torch.empty_like(gq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    scale = w.scale

    def step():
        ea.attn_fwd_bf16(gq, gk, gv, causal=True, scale=scale, out=o, lse=lse)

    ms = timed(step, args.steps, args.warmup, torch)
    sclk = read_counters("sclk_ghz_estimate")
    flops = counted_flops(w.B, w.H, w.N, w.d, True)
    tflops = flops / (ms * 1e-3) / 1e12

    out = {
        "metric": "attention fwd TFLOP/s (bf16, causal, d=128, N=8k) and % of MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16",
        "config": {"workload": "bf16 causal attention forward, B=2 H=16 N=8192 d=128", "B": w.B, "H": w.H,
                   "N": w.N, "d": w.d, "causal": True, "flop_per_step": flops},
        "pct_of_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        # the engine clock under this load (counter run) and the peak scaled to it
        "sclk_ghz": sclk,
        "pct_of_peak_at_measured_clock": None if sclk is None else 100.0 * tflops / (PEAK_BF16_TFLOPS * sclk / 2.4),
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS, "traffic": read_counters()},
    }
    if not args.no_extra:
        # each leg gets untimed calls of its own first (its kernels' first launches, and
        # ~20 ms of load so the clock is at its steady state for that kernel mix)
        legw = min(args.warmup, 10)
        out["backward"] = backward_leg(torch, ea, inputs, w, (gq, gk, gv), o, lse, max(3, args.steps // 2), legw)
        out["fp8"] = fp8_leg(torch, ea, inputs, max(3, args.steps // 2), 4 * legw)
        out["decode"] = decode_leg(torch, ea, inputs, max(3, args.steps), 10 * legw)
    if not args.no_cpu_baseline:
        qf, kf, vf = (t.float().numpy() for t in cpu)     # the bf16 values, upcast exactly
        out["cpu_baseline"] = cpu_baseline(qf, kf, vf, True, scale, args.cpu_budget)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
