#!/usr/bin/env python3
"""Forward-pass benchmark of the exact attention library on one MI355X.

Metric: attention forward TFLOP/s for bf16, causal, head dim 128, N = 8192
(B = 2, H = 16), counting 4*B*H*N^2*d FLOPs halved for causal, and the fraction of
the dense bf16 MFMA peak. One step is one forward call of the whole path (workgroup
order, Q/K/V loads, both MFMA contractions, masking, online softmax, epilogue) over
one batch of seeded synthetic inputs that are already resident in HBM.

Prints ONE JSON line. Besides the headline it reports, from the same run:
  calibration  what a dense MFMA loop and a dense exp2 loop sustain at the loaded clock,
               MFMA loops with the kernels' VALU/LDS work between MFMAs, a large bf16
               GEMM through torch (hipBLASLt), and a streaming-read loop over 1 GiB
  forward      the headline call's per-launch statistics (median, min, std over the
               timed launches), the exact (running-max) pass alone on the same inputs,
               the same call on inputs whose query tiles all need the exact pass, the
               tile schedules and persistent grids, configurations C1-C4 (C2 also with
               a cold cache), and the exponentials/s secondary bound
  backward     dQ, dK, dV of the headline call (2.5x the forward FLOPs)
  fp8          quantiser and fp8 attention on the fp8 workload (B2 H16 N8192 d128 causal)
  decode       one split-KV decoding step (B16 H16, 1 query row, 8192 keys; GB/s)
  cpu_baseline the CPU oracle on whole heads of the headline workload, on every core of
               this process's affinity set
The extra legs run before the headline's warm-up and timed steps, so the headline is
timed at the clock the chip holds under sustained load.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_attention_78_amd.flops import counted_flops, counted_flops_backward  # noqa: E402

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


def sample_sclk(torch, fn, seconds=1.5, settle=0.5):
    """Mean GFX clock of this process's GPU while fn() keeps it busy: amd-smi (a child
    process) reads the clock of every GFX partition of the device whose PCI address
    matches torch's device 0, repeatedly for `seconds`, after `settle` seconds of load
    (the firmware's metrics refresh every few hundred milliseconds, so earlier readings
    can still show the idle clock), while this thread enqueues fn() in synchronised
    batches of 64 calls. Returns {"mhz": mean over samples and partitions, "min_mhz",
    "max_mhz", "samples": n} or {"mhz": None, "why": ...}."""
    import shutil
    import subprocess
    import threading

    if any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", ""):
        # a profiler's preloaded library would initialise the GPU in the child before amd-smi starts
        return {"mhz": None, "why": "not sampled under rocprofv3"}
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe):
        return {"mhz": None, "why": "amd-smi not found"}
    try:
        p = torch.cuda.get_device_properties(0)
        bdf = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}"
        lst = json.loads(subprocess.run([exe, "list", "--json"], capture_output=True, text=True, timeout=60).stdout)
        lst = lst if isinstance(lst, list) else lst.get("gpu_data", lst.get("gpus", []))
        idx = [g["gpu"] for g in lst if str(g.get("bdf", "")).lower().startswith(bdf)]
    except Exception as e:  # noqa: BLE001 - reported, not raised: the clock is context, not the metric
        return {"mhz": None, "why": f"device lookup failed: {e!r}"}
    if len(idx) != 1:
        return {"mhz": None, "why": f"no unique amd-smi device with PCI address {bdf}"}
    samples, errs = [], []

    def sampler():
        time.sleep(settle)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            try:
                r = subprocess.run([exe, "metric", "-g", str(idx[0]), "--clock", "--json"], capture_output=True,
                                   text=True, timeout=60)
                d = json.loads(r.stdout)
                g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
                vals = [float(v["clk"]["value"]) for k, v in g["clock"].items()
                        if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
                if vals:
                    samples.append(vals)
            except Exception as e:  # noqa: BLE001
                errs.append(repr(e))
                return

    th = threading.Thread(target=sampler)
    th.start()
    while th.is_alive():
        for _ in range(64):
            fn()
        torch.cuda.synchronize()
    th.join()
    if not samples:
        return {"mhz": None, "why": errs[0] if errs else "no clock sample"}
    flat = [x for v in samples for x in v]
    return {"mhz": sum(flat) / len(flat), "min_mhz": min(flat), "max_mhz": max(flat), "samples": len(samples),
            "amd_smi_gpu": idx[0]}


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


def time_launches(torch, fn, steps, warmup, reps=1, between=None, warm_s=0.3):
    """Run fn() `warmup` times untimed, and then on for at least `warm_s` seconds (in
    synchronised batches of 8 calls, so that the launch queue stays short), so that the
    clock has settled under this kernel's load; then time `steps` launches (each a group of
    `reps` back-to-back calls) with HIP events on the current stream (the stream the library
    launches on). `between`, if given, runs untimed before each timed launch (e.g. a cache
    flush; every launch then has its own event pair). Returns per-call milliseconds: the
    mean over the timed calls, and median / min / std over the launches."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    if between is None:
        # the mean from one event pair around all calls (an event recorded between two
        # calls adds a gap of a few microseconds); then the same number of launches again,
        # one pair each, for the spread
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps * reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        total = e0.elapsed_time(e1) / (steps * reps)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            for _ in range(reps):
                fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) / reps for i in range(steps)]
    else:
        per = []
        for _ in range(steps):
            between()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / reps)
        total = sum(per) / steps
    return {"mean_ms": total, "median_ms": statistics.median(per), "min_ms": min(per),
            "std_ms": statistics.pstdev(per) if len(per) > 1 else 0.0, "launches": steps, "calls_per_launch": reps}


def us(t):
    """The timing dict in microseconds (keys *_ms -> *_us)."""
    return {(k[:-3] + "_us" if k.endswith("_ms") else k): (v * 1e3 if k.endswith("_ms") else v) for k, v in t.items()}


def rate(work, t, scale=1e12):
    return work / (t["mean_ms"] * 1e-3) / scale


# ----------------------------------------------------------------------------- legs


def calibration_leg(torch, ea):
    """Dense MFMA and exp2 loops (one 8-wave workgroup per CU, the attention kernels'
    launch shape), an 8192^3 bf16 GEMM through torch.matmul (hipBLASLt), and a streaming
    read loop over 1 GiB."""
    res = {}
    wg = torch.cuda.get_device_properties(0).multi_processor_count
    for kind, iters, unit, scale in (("mfma", 4000, "TFLOP/s", 1e12), ("exp", 8000, "Gexp/s", 1e9)):
        out, ops = ea.attn_calibrate(kind, wg, iters)
        t = time_launches(torch, lambda: ea.attn_calibrate(kind, wg, iters, out=out), 5, 3)
        res[f"{kind}_loop"] = {"value": rate(ops, t, scale), "unit": unit, "us": t["mean_ms"] * 1e3,
                               "workgroups": wg}
    res["mfma_loop"]["frac_of_published_peak"] = res["mfma_loop"]["value"] / PEAK_BF16_TFLOPS
    # MFMA loops with the attention kernels' work between MFMAs (one fma, exp and add each)
    mixes = {}
    for kind, what in (("mix_nolds_2w", "no LDS read, 2 waves/SIMD"),
                       ("mix_lds1_2w", "one 16-byte LDS read per MFMA, 2 waves/SIMD"),
                       ("mix_lds0.5_2w", "one LDS read per 2 MFMAs, 2 waves/SIMD"),
                       ("mix_lds0.5_1w", "one LDS read per 2 MFMAs, 1 wave/SIMD")):
        out, ops = ea.attn_calibrate(kind, wg, 400)
        t = time_launches(torch, lambda: ea.attn_calibrate(kind, wg, 400, out=out), 5, 2)
        mixes[kind] = {"tflops": rate(ops, t), "what": what}
    res["mfma_mix_loops"] = mixes
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    t = time_launches(torch, lambda: torch.matmul(a, b, out=c), 10, 5)
    res["gemm_bf16_8192"] = {"value": rate(2.0 * n ** 3, t), "unit": "TFLOP/s", "us": t["mean_ms"] * 1e3,
                             "frac_of_published_peak": rate(2.0 * n ** 3, t) / PEAK_BF16_TFLOPS,
                             "library": "torch.matmul (hipBLASLt)"}
    del a, b, c
    # what streaming reads attain (the HBM-bound kernels' attainable rate beside the
    # published 8 TB/s): the read loop sweeping 1 GiB once, 2048 workgroups of 256 threads
    wgr, itr = 2048, 128
    buf = torch.zeros(wgr * 256 * itr * 4, dtype=torch.int32, device="cuda")
    out, nbytes = ea.attn_calibrate("read", wgr, itr, seed=buf)
    t = time_launches(torch, lambda: ea.attn_calibrate("read", wgr, itr, seed=buf, out=out), 10, 5)
    res["read_loop"] = {"value": rate(nbytes, t, 1e9), "unit": "GB/s", "us": t["mean_ms"] * 1e3, "bytes": nbytes,
                        "frac_of_published_hbm": rate(nbytes, t, 1e9) / PEAK_HBM_GBS}
    del buf, out
    # LDS read rate, one workgroup of 8 waves per CU: 16-byte reads and the 8-byte transpose
    # reads that feed the attention kernels' V^T (and backward Q^T, dO^T) operands
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for kind, what in (("lds_b128", "ds_read_b128, 16 bytes per lane"),
                       ("lds_tr_b64", "ds_read_b64_tr_b16, 8 bytes per lane")):
        out, nb = ea.attn_calibrate(kind, cus, 2000)
        t = time_launches(torch, lambda: ea.attn_calibrate(kind, cus, 2000, out=out), 5, 3)
        res[f"{kind}_loop"] = {"value": rate(nb, t, 1e9), "unit": "GB/s", "bytes_per_cu_per_ns": rate(nb, t, 1e9) / cus,
                               "what": what}
    return res


def schedules(torch, ea, flops, rounds, calls, call):
    """Every tile schedule of the forward pass on one workload, timed in interleaved rounds
    (each round times `calls` back-to-back calls of every schedule in turn), so that all
    schedules see the same clock; per schedule the median over rounds."""
    names = list(ea._binding.SCHEDULES)
    for s in names:
        call(s)
    torch.cuda.synchronize()
    per = {s: [] for s in names}
    for _ in range(rounds):
        for s in names:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(calls):
                call(s)
            e1.record()
            torch.cuda.synchronize()
            per[s].append(e0.elapsed_time(e1) / calls)
    out = {}
    for s in names:
        ms = statistics.median(per[s])
        out[s] = {"us": ms * 1e3, "tflops": flops / (ms * 1e-3) / 1e12}
    return out


def forward_legs(torch, ea, inputs, w, gq, gk, gv, o, lse, steps, warmup, calib):
    """Exact pass alone, all tiles needing the exact pass, schedules, C1-C4, C2 cold, exps/s."""
    res = {}
    flops = counted_flops(w.B, w.H, w.N, w.d, True)

    def leg(fn, work=flops, n=steps, wu=warmup, **kw):
        t = time_launches(torch, fn, n, wu, **kw)
        return {"us": us(t), "tflops": rate(work, t), "frac_bf16_peak": rate(work, t) / PEAK_BF16_TFLOPS}

    cfg = {}
    for name, causal in (("C1", False), ("C1", True), ("C2", True), ("C3", True), ("C3", False), ("C4", True)):
        c = inputs.WORKLOADS[name]
        dt = "f32" if name == "C1" else "bf16"
        q, k, v = (inputs.to_torch(x, dt).cuda() for x in inputs.draw_qkv(c.wid, c.B, c.H, c.N, c.d))
        f = counted_flops(c.B, c.H, c.N, c.d, causal)
        call = lambda: ea.fwd(q, k, v, causal=causal, scale=c.scale)   # noqa: E731
        small = name in ("C1", "C2")
        r = leg(call, work=f, n=10 if small else max(5, steps // 2), wu=10 if small else 3, reps=50 if small else 1)
        key = f"{name}_{'causal' if causal else 'noncausal'}"
        cfg[key] = {"workload": f"{dt} B{c.B} H{c.H} N{c.N} d{c.d} {'causal' if causal else 'non-causal'}",
                    "us": r["us"], "tflops": r["tflops"], "frac_bf16_peak": r["frac_bf16_peak"] if dt == "bf16" else None}
        if name == "C2":
            scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
            rc = leg(call, work=f, n=10, wu=2, between=lambda: scratch.fill_(1))
            cfg[key + "_cold"] = {"workload": cfg[key]["workload"] + ", L2/MALL flushed by a 512 MiB write before "
                                  "each launch", "us": rc["us"], "tflops": rc["tflops"]}
            del scratch
        del q, k, v
    res["configs"] = cfg

    res["exact_pass_only"] = leg(lambda: ea.attn_fwd_variant(gq, gk, gv, causal=True, scale=w.scale, passes="exact",
                                                             out=o, lse=lse))
    res["exact_pass_only"]["what"] = ("the running-max online softmax alone on every tile (per-tile row max, lazy "
                                      "rescale), same inputs as the headline")
    # keys from 300 on scaled x30: every query tile past row 300 outgrows the first tile's max
    import numpy as np

    k_marked = inputs.normal_f32(w.wid, inputs.K_ID, (w.B, w.H, w.N, w.d))
    k_marked[:, :, 300:] *= np.float32(30.0)
    gkm = inputs.to_torch(k_marked, "bf16").cuda()
    del k_marked
    res["all_tiles_marked"] = leg(lambda: ea.attn_fwd_bf16(gq, gkm, gv, causal=True, scale=w.scale, out=o, lse=lse))
    res["all_tiles_marked"]["what"] = ("the headline call on inputs whose keys from 300 on are scaled x30: the first "
                                       "pass marks every query tile that sees them and stops, the exact pass redoes them")
    del gkm

    queue = ea.queue_workspace()
    for name in ("C3", "C4", "H"):
        c = inputs.WORKLOADS[name]
        if name == "H":
            q, k, v, oc, lc = gq, gk, gv, o, lse
        else:
            q, k, v = (inputs.to_torch(x, "bf16").cuda() for x in inputs.draw_qkv(c.wid, c.B, c.H, c.N, c.d))
            oc, lc = torch.empty_like(q), torch.empty((c.B, c.H, c.N), device="cuda", dtype=torch.float32)
        res[f"schedules_{name}_causal"] = schedules(
            torch, ea, counted_flops(c.B, c.H, c.N, c.d, True), rounds=4, calls=max(3, steps // 4),
            call=lambda s, q=q, k=k, v=v, oc=oc, lc=lc, sc=c.scale: ea.attn_fwd_variant(
                q, k, v, causal=True, scale=sc, sched=s, queue=queue, out=oc, lse=lc))
        del q, k, v, oc, lc

    return res


def backward_leg(torch, ea, inputs, w, tensors, o, lse, steps, warmup):
    """The backward pass of the forward call timed (same inputs, its O and LSE)."""
    gq, gk, gv = tensors
    g = inputs.to_torch(inputs.draw_dout(w.wid, w.B, w.H, w.N, w.d), "bf16").cuda()
    ea.attn_fwd_bf16(gq, gk, gv, causal=True, scale=w.scale, out=o, lse=lse)
    dq, dk, dv = (torch.empty_like(gq) for _ in range(3))
    ws = torch.empty((2, w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    t = time_launches(torch, lambda: ea.attn_bwd_bf16(gq, gk, gv, o, lse, g, causal=True, scale=w.scale, dq=dq, dk=dk,
                                                      dv=dv, workspace=ws), steps, warmup)
    flops = counted_flops_backward(w.B, w.H, w.N, w.d, True)
    assert all(bool(torch.isfinite(x.float()).all()) for x in (dq, dk, dv))
    return {"workload": "bf16 causal attention backward (dQ, dK, dV), B=2 H=16 N=8192 d=128",
            "us": us(t), "tflops": rate(flops, t), "frac_bf16_peak": rate(flops, t) / PEAK_BF16_TFLOPS,
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
    t = time_launches(torch, lambda: ea.attn_decode_bf16(q, k, v, out=o, lse=lse, workspace=ws), steps, warmup)
    nbytes = 2 * B * H * Nk * d * 2 + 2 * B * H * Nq * d * 2 + B * H * Nq * 4   # K, V, Q read; O, LSE written
    assert bool(torch.isfinite(o.float()).all())
    return {"workload": "bf16 decoding step, B=16 H=16 Nq=1 Nk=8192 d=128, no mask (split-KV)",
            "us": us(t), "gbs": rate(nbytes, t, 1e9), "frac_hbm": rate(nbytes, t, 1e9) / PEAK_HBM_GBS}


def fp8_leg(torch, ea, inputs, steps, warmup):
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

    tqnt = time_launches(torch, quant_all, steps, warmup)
    # the same three tensors in one launch
    tq1 = time_launches(torch, lambda: ea.attn_quant_fp8_qkv(tq, tk, tv, sg, q8=q8, k8=k8, v8=v8, q_scale=sq,
                                                             k_scale=sk, v_scale=sv), steps, warmup)
    tatt = time_launches(torch, lambda: ea.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=True, out=o, lse=lse), steps,
                         warmup)
    # the two-launch path: K and V quantised in one launch, Q prepared inside the attention kernel
    tkv = time_launches(torch, lambda: ea.attn_quant_fp8_kv(tk, tv, sg, k8=k8, v8=v8, k_scale=sk, v_scale=sv), steps,
                        warmup)
    trq = time_launches(torch, lambda: ea.attn_fwd_fp8_rotq(tq, sg, k8, v8, sk, sv, causal=True, out=o, lse=lse),
                        steps, warmup)
    flops = counted_flops(w.B, w.H, w.N, w.d, True)
    n = w.B * w.H * w.N * w.d
    nblk = (w.N + 127) // 128
    qbytes = 3 * (2 * n + n + 4 * w.B * w.H * nblk)      # read bf16, write codes + scales
    assert bool(torch.isfinite(o.float()).all())
    return {
        "workload": "fp8 e4m3, causal, B=2 H=16 N=8192 d=128, Hadamard-rotated Q/K with shared outlier channels",
        "attn_us": us(tatt), "attn_tflops": rate(flops, tatt), "attn_frac_fp8_peak": rate(flops, tatt) / PEAK_FP8_TFLOPS,
        "quant_qkv_us": us(tqnt), "quant_gbs": rate(qbytes, tqnt, 1e9),
        "quant_frac_hbm": rate(qbytes, tqnt, 1e9) / PEAK_HBM_GBS,
        "path_three_quant_launches_plus_attention_us": (tqnt["mean_ms"] + tatt["mean_ms"]) * 1e3,
        "quant_qkv_one_launch_us": us(tq1), "quant_one_launch_gbs": rate(qbytes, tq1, 1e9),
        "quant_one_launch_frac_hbm": rate(qbytes, tq1, 1e9) / PEAK_HBM_GBS,
        "path_one_quant_launch_plus_attention_us": (tq1["mean_ms"] + tatt["mean_ms"]) * 1e3,
        "fused_q": {
            "what": "K and V quantised in one launch (attn_quant_fp8_kv), Q rotated and quantised inside the "
                    "attention kernel (attn_fwd_fp8_rotq)",
            "quant_kv_us": us(tkv), "quant_kv_gbs": rate(2 * qbytes / 3, tkv, 1e9),
            "attn_rotq_us": us(trq), "attn_rotq_tflops": rate(flops, trq),
            "path_us": (tkv["mean_ms"] + trq["mean_ms"]) * 1e3},
    }


def cpu_baseline(q, k, v, causal, scale, budget_s):
    """Time the oracle (as it stands) on whole heads of the workload, every core of this
    process's affinity set working on (head, 1024-row chunk) units, until the budget is used."""
    from oracle.pool import forward_pooled, host_cores

    B, H, N, d = q.shape
    cores = host_cores()
    heads = [(b, h) for b in range(B) for h in range(H)]
    done, t0 = 0, time.perf_counter()
    while done < len(heads) and time.perf_counter() - t0 < budget_s:
        batch = heads[done:done + max(1, cores // 4)]
        forward_pooled(q, k, v, causal, scale, heads=batch, workers=cores)
        done += len(batch)
    dt = time.perf_counter() - t0
    flops = counted_flops(1, done, N, d, causal)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {B * H} heads (all {N} query rows each, causal) of the bf16 B2 H16 N8192 d128 "
                      f"workload, fp64 NumPy on {cores} worker threads (one BLAS thread each), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--no-extra", action="store_true", help="headline only: skip every other leg")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--only", choices=["calibration", "fp8", "backward", "decode"],
                    help="run only this leg (for profiler runs) and print its JSON")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of 1 GiB x 4 (HBM counter calibration) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one MI355X only: --gpus {args.gpus} (WORLD_SIZE {world}) is not supported; "
              f"nothing here uses a second GPU. Run with --gpus 1.", file=sys.stderr)
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

    if args.only == "calibration":
        print(json.dumps({"calibration": calibration_leg(torch, ea)}))
        return
    if args.only in ("fp8", "decode"):
        fn = fp8_leg if args.only == "fp8" else decode_leg
        print(json.dumps({args.only: fn(torch, ea, inputs, args.steps, args.warmup)}))
        return

    w = inputs.WORKLOADS["H"]
    q, k, v = inputs.draw_qkv(w.wid, w.B, w.H, w.N, w.d)
    cpu = tuple(inputs.to_torch(x, "bf16") for x in (q, k, v))
    del q, k, v
    gq, gk, gv = (t.cuda() for t in cpu)
    o = torch.empty_like(gq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    flops = counted_flops(w.B, w.H, w.N, w.d, True)

    def step():
        ea.attn_fwd_bf16(gq, gk, gv, causal=True, scale=w.scale, out=o, lse=lse)

    if args.only == "backward":
        print(json.dumps({"backward": backward_leg(torch, ea, inputs, w, (gq, gk, gv), o, lse, args.steps,
                                                   args.warmup)}))
        return

    extra = {}
    if not args.no_extra:
        legs_steps, legs_warm = max(5, min(args.steps, 20)), max(3, min(args.warmup, 10))
        # the forward legs come last: the headline then starts with the chip already at the
        # clock it holds under this kernel's load
        extra["calibration"] = calibration_leg(torch, ea)
        extra["backward"] = backward_leg(torch, ea, inputs, w, (gq, gk, gv), o, lse, legs_steps, legs_warm)
        extra["fp8"] = fp8_leg(torch, ea, inputs, legs_steps, legs_warm)
        extra["decode"] = decode_leg(torch, ea, inputs, legs_steps, 4 * legs_warm)
        extra["decode"]["frac_of_read_loop"] = extra["decode"]["gbs"] / extra["calibration"]["read_loop"]["value"]
        extra["forward"] = forward_legs(torch, ea, inputs, w, gq, gk, gv, o, lse, legs_steps, legs_warm,
                                        extra["calibration"])

    # the headline: W untimed steps, then exactly K timed steps between one pair of HIP
    # events (events recorded between the calls would add a gap of several microseconds
    # to each); then K more calls, each between its own pair of events, for the per-call
    # median, min and std
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    t = time_launches(torch, step, args.steps, 0, warm_s=0.0)
    t["mean_ms"] = ms
    # the clock the chip holds under this call, sampled after the timed region while the
    # same call keeps running (outside the timed region: it does not enter `value`)
    clk = sample_sclk(torch, step)

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
        # the published peak is at 2.4 GHz; at the sampled clock the matrix cores can do
        # peak * sclk / 2.4 GHz
        "sclk": {**clk, "source": "amd-smi metric --clock of this GPU, mean over its GFX partitions and over "
                                  "1.5 s of samples taken after the timed region while the same call kept "
                                  "running (after 0.5 s of it)",
                 "pct_of_peak_at_measured_clock": (100.0 * tflops / (PEAK_BF16_TFLOPS * clk["mhz"] / 2400.0)
                                                   if clk.get("mhz") else None)},
        "launch_us": {**us(t), "what": "mean: the K timed calls (one event pair around them); median, min, std: "
                                        "K more calls, one event pair each (the pairs add a few microseconds per call)"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS, "traffic": read_counters()},
    }
    if extra:
        cal = extra["calibration"]
        out["pct_of_attainable_mfma_loop"] = 100.0 * tflops / cal["mfma_loop"]["value"]
        # secondary bound: one exponential per unmasked score (causal: N(N+1)/2 per head)
        exps = w.B * w.H * w.N * (w.N + 1) / 2
        extra["forward"]["exp_bound"] = {
            "exps_per_call": exps, "exps_per_s": exps / (ms * 1e-3),
            "frac_of_exp_loop": exps / (ms * 1e-3) / (cal["exp_loop"]["value"] * 1e9)}
        out.update(extra)
    if not args.no_cpu_baseline:
        qf, kf, vf = (x.double().numpy() for x in cpu)    # the bf16 values, upcast exactly
        out["cpu_baseline"] = cpu_baseline(qf, kf, vf, True, w.scale, args.cpu_budget)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
