#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

One step = one flash_attn_fwd call (the whole forward: scores, online softmax,
P V, O and LSE) on the LLaMA-7B-shaped causal workload B=2, H=32, N=4096,
d=128, bf16, inputs resident in HBM. Prints one JSON line:

* value: TFLOP/s with the metric's count 4*B*H*N^2*d / 2 (causal), over the
  K timed steps bracketed by synchronisations;
* roofline: the kernel's average launch time from HIP events recorded on the
  stream it runs on, its algorithmic FLOPs per launch, and the fraction of the
  MI355X dense bf16 MFMA peak (2.5 PFLOP/s); `traffic` is the HBM bytes per
  launch measured by rocprofv3 counters for this exact kernel source, or null;
* cpu_baseline: the float64 CPU oracle timed on a bounded sample of the same
  workload (a few complete (batch, head) slices) on this host's cores.

Options --workload and --all select other workloads (diagnostics; the JSON line
keeps the headline workload by default). --bwd times the backward pass instead
(one step = one flash_attn_bwd call: D, dQ, dK and dV from Q, K, V, O, LSE and
dO), counted as 2.5x the forward's FLOPs (five N x N x d products instead of
two), with the float64 backward oracle as its CPU baseline. --splitkv times the
forward with and without the key split (flash_attn_fwd_splitkv, split count
planned for this GPU) on the shapes that underfill it. --strided times
flash_attn_fwd_strided at the headline shape with head dimensions 80, 96, 192 and
256 (the last two on the 256-wide instance, one launch per 128 columns of V and O)
and with q, k, v taken from one packed [B, N, 3, H, d] tensor (FLOPs counted with
the real d). --fp8 times the FP8 path at the headline shape: flash_attn_fwd_fp8 alone
(the attention on quantized inputs, E4M3 and E5M2; FLOPs as the metric counts them,
against the 5 PFLOP/s dense FP8 peak) and the three quantization calls. --table prints one
line per workload and mask: launch-time median, p10 and p90, TFLOP/s, % of peak,
the recorded HBM bytes, and the oracle's time and parity metrics (max and mean abs
error of O, excess over half an ulp, LSE error) on whole (batch, head) slices.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA, vendor figure
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 MFMA, vendor figure
# the two forward kernels flash_attn_fwd can launch (flash_attn_fwd_kernel names the
# one a shape runs): kernel symbol and the sources it is built from
FWD_KERNELS = {
    "pipelined": ("fwd_sp", ["exact_attention_flash_amd/csrc/fwd_sp.hip", "exact_attention_flash_amd/csrc/fwd_kernel.h",
                             "exact_attention_flash_amd/csrc/gfx950_ops.h"]),
    "pingpong": ("fwd_pingpong", ["exact_attention_flash_amd/csrc/fwd_kernel.hip",
                                  "exact_attention_flash_amd/csrc/fwd_kernel.h",
                                  "exact_attention_flash_amd/csrc/gfx950_ops.h"]),
}
# (batch, head) slices the oracle runs per workload in --table (all rows of each)
TABLE_SLICES = {"single_head_n256_d64": 1, "mha_b4_h16_n1024_d64": 64, "llama7b_b2_h32_n4096_d128_causal": 8,
                "longctx_b1_h32_n16384_d128_causal": 1, "stress_b3_h8_n4099_d128_sigma8": 6}
BWD_FLOP_FACTOR = 2.5       # backward: S, dP, dV, dQ, dK products versus the forward's S and PV
TRAFFIC_FILE = "profiles/fwd_hbm_traffic.txt"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def fwd_kernel_of(w, causal: bool) -> str:
    """"pipelined" or "pingpong": the forward kernel flash_attn_fwd runs for workload w."""
    import exact_attention_flash_amd as fa

    return fa.flash_attn_fwd_kernel(w.N, w.d, causal)


def kernel_symbol(kernel: str) -> str:
    return FWD_KERNELS[kernel][0]


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for p in FWD_KERNELS[kernel][1]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, causal: bool, kernel: str):
    """HBM bytes per launch recorded for this kernel and its source, or None if stale/absent."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    want = kernel_source_hash(kernel)
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fields = dict(kv.split("=", 1) for kv in line.split())
            if (fields.get("workload") == workload and fields.get("causal") == str(int(causal))
                    and fields.get("kernel") == kernel_symbol(kernel)
                    and fields.get("source_sha256_16") == want):
                return float(fields["hbm_bytes_per_launch"])
    return None


def time_gpu(w, causal, steps, warmup, bwd=False, splits=None):
    import torch

    import exact_attention_flash_amd as fa
    from exact_attention_flash_amd import inputs

    dev = torch.device("cuda:0")
    qb, kb, vb = inputs.workload_qkv(w)
    q, k, v = (inputs.to_torch(x, w.dtype, dev) for x in (qb, kb, vb))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    scale = inputs.default_scale(w.d)
    stream = torch.cuda.current_stream(dev)

    if splits is not None:
        nbytes = fa.splitkv_workspace_size(w.B, w.H, w.N, w.d, causal, splits)
        ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=dev) if nbytes else None

        def step():
            fa.flash_attn_fwd_splitkv(q, k, v, o, lse, ws, causal=causal, scale=scale, num_splits=splits,
                                      stream=stream)
    elif bwd:
        # gradient of the output drawn like the inputs (unit variance), O and LSE
        # from the forward pass; dQ, dK, dV and the D workspace preallocated
        dob, _, _ = inputs.workload_qkv(w, seed_offset=7)
        do = inputs.to_torch(dob, w.dtype, dev)
        fa.flash_attn_fwd(q, k, v, o, lse, causal=causal, scale=scale, stream=stream)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        delta = torch.empty_like(lse)

        def step():
            fa.flash_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, delta, causal=causal, scale=scale, stream=stream)
    else:
        def step():
            fa.flash_attn_fwd(q, k, v, o, lse, causal=causal, scale=scale, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)

    # per-launch HIP events on the kernel's stream: the distribution
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per_launch = sorted(a.elapsed_time(b) for a, b in evs)

    # the timed region of the contract: K back-to-back steps between synchronisations
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1) / steps
    extra = torch.cuda.max_memory_allocated(dev) - mem0
    gpu_out = None
    if not bwd and splits is None:
        gpu_out = (inputs.from_torch_bits(o), lse.double().cpu().numpy())
    return {
        "wall_s": wall, "ms_per_step": wall * 1e3 / steps, "event_ms_per_launch": ev_ms,
        "launch_ms_median": statistics.median(per_launch),
        "launch_ms_p10": per_launch[int(0.1 * (len(per_launch) - 1))],
        "launch_ms_p90": per_launch[int(0.9 * (len(per_launch) - 1))],
        "extra_alloc_bytes": int(extra),
        "device": torch.cuda.get_device_name(dev),
        "gpu_out": gpu_out,
    }, (qb, kb, vb)


def _half_ulp(x, dtype):
    """Half the spacing of the 16-bit output type at |x| (subnormal spacing near 0)."""
    import numpy as np

    mant, min_exp = (7, -126) if dtype == "bf16" else (10, -14)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(ax))
    e = np.maximum(np.where(np.isfinite(e), e, min_exp), min_exp)
    return np.ldexp(0.5, (e - mant).astype(np.int64))


def cpu_baseline(w, causal, qkv_bits, slices, gpu_out=None):
    """Time the float64 oracle on `slices` complete (batch, head) slices of the workload;
    with the GPU's o (16-bit bits) and lse, also compare them on those slices."""
    import numpy as np

    from exact_attention_flash_amd import inputs
    from oracle.dense import attention

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
                           default=1)
    except Exception:  # noqa: BLE001 - reporting only
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    qb, kb, vb = (x.reshape(-1, w.N, w.d)[:slices] for x in qkv_bits)
    q, k, v = (inputs.bits_to_f64(x, w.dtype) for x in (qb, kb, vb))
    t0 = time.perf_counter()
    ro, rl = attention(q, k, v, inputs.default_scale(w.d), causal=causal)
    dt = time.perf_counter() - t0
    flops = 4.0 * slices * w.N * w.N * w.d / (2.0 if causal else 1.0)
    out = {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads or cores, "kind": "oracle",
        "sample": f"{slices} of {w.B * w.H} (batch, head) slices of the same workload, all {w.N} rows, "
                  f"float64 numpy (BLAS matmuls, {blas_threads} BLAS threads on {cores} host cores); "
                  f"{dt:.1f} s, scaled with the same FLOP formula",
        "seconds": dt,
    }
    if gpu_out is not None:
        ob, lse = gpu_out
        o64 = inputs.bits_to_f64(ob.reshape(-1, w.N, w.d)[:slices], w.dtype)
        l64 = lse.reshape(-1, w.N)[:slices]
        err = np.abs(o64 - ro)
        out["parity"] = {
            "slices": slices,
            "o_max_abs": float(err.max()),
            "o_max_excess_over_half_ulp": float(np.maximum(err - _half_ulp(ro, w.dtype), 0.0).max()),
            "o_mean_abs": float(err.mean()),
            "lse_max_abs": float(np.abs(l64 - rl).max()),
        }
    return out


def cpu_baseline_bwd(w, causal, qkv_bits, slices):
    """Time the float64 backward oracle on `slices` complete (batch, head) slices."""
    from exact_attention_flash_amd import inputs
    from oracle.backward import attention_backward

    cores = len(os.sched_getaffinity(0))
    dob, _, _ = inputs.workload_qkv(w, seed_offset=7)
    qb, kb, vb, db = (x.reshape(-1, w.N, w.d)[:slices] for x in (*qkv_bits, dob))
    q, k, v, do = (inputs.bits_to_f64(x, w.dtype) for x in (qb, kb, vb, db))
    t0 = time.perf_counter()
    attention_backward(q, k, v, do, inputs.default_scale(w.d), causal=causal)
    dt = time.perf_counter() - t0
    flops = BWD_FLOP_FACTOR * 4.0 * slices * w.N * w.N * w.d / (2.0 if causal else 1.0)
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": f"{slices} of {w.B * w.H} (batch, head) slices of the same workload, all {w.N} rows, "
                  f"float64 numpy backward oracle on {cores} host cores; {dt:.1f} s, scaled with the same "
                  "FLOP formula",
        "seconds": dt,
    }


def copy_calibration(mib, reps):
    """A plain copy kernel of known size: reads and writes MIB MiB per launch."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_mib": mib, "bytes_read": n * 4, "bytes_written": n * 4, "ms_per_copy": ms,
                      "GB_per_s": 2 * n * 4 / (ms * 1e-3) / 1e9}), flush=True)


def run_bwd(args, workload_name, causal):
    """Diagnostic line for the backward pass (not the forward's contract line)."""
    from exact_attention_flash_amd import inputs

    w = inputs.WORKLOADS[workload_name]
    flops = BWD_FLOP_FACTOR * w.flops(causal)
    g, qkv = time_gpu(w, causal, args.steps, args.warmup, bwd=True)
    tflops = flops / (g["ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (g["event_ms_per_launch"] * 1e-3) / 1e12
    line = {
        "metric": "attention bwd TFLOP/s (2.5x forward FLOPs) and % of bf16 MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOP/s",
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(g["ms_per_step"], 5),
        "higher_is_better": True, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": causal,
                   "dtype": w.dtype, "pass": "backward"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "kernel": "bwd_dq + bwd_dkdv (flash_attn_bwd)", "flop_per_launch": flops,
                     "launch_ms": round(g["event_ms_per_launch"], 5),
                     "launch_ms_median": round(g["launch_ms_median"], 5)},
        "extra_alloc_bytes": g["extra_alloc_bytes"], "device": g["device"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_bwd(w, causal, qkv, args.cpu_bwd_slices)
    return line


def run_splitkv(args):
    """Diagnostic lines: forward with and without the key split on underfilled shapes."""
    import torch

    import exact_attention_flash_amd as fa
    from exact_attention_flash_amd import inputs

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    names = list(inputs.SPLIT_WORKLOADS) + ["single_head_n256_d64", "mha_b4_h16_n1024_d64"]
    for name in names:
        w = inputs.SPLIT_WORKLOADS.get(name) or inputs.WORKLOADS[name]
        causal = w.causal[0]
        flops = w.flops(causal)
        splits = fa.splitkv_plan(w.B, w.H, w.N, w.d, causal, cus)
        plain, _ = time_gpu(w, causal, args.steps, args.warmup)
        split, _ = time_gpu(w, causal, args.steps, args.warmup, splits=splits)
        items = w.B * w.H * -(-w.N // 256)
        line = {
            "metric": "attention fwd TFLOP/s, key split versus plain (diagnostic)",
            "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": causal,
                       "dtype": w.dtype, "work_items": items, "compute_units": cus, "splits": splits},
            "plain": {"launch_ms": round(plain["event_ms_per_launch"], 5),
                      "tflops": round(flops / (plain["event_ms_per_launch"] * 1e-3) / 1e12, 2)},
            "splitkv": {"launch_ms": round(split["event_ms_per_launch"], 5),
                        "tflops": round(flops / (split["event_ms_per_launch"] * 1e-3) / 1e12, 2),
                        "note": "split kernel + merge kernel, one call"},
            "speedup": round(plain["event_ms_per_launch"] / split["event_ms_per_launch"], 3),
            "unit": "TFLOP/s", "steps": args.steps, "warmup": args.warmup,
        }
        print(json.dumps(line), flush=True)


def run_strided(args):
    """Diagnostic lines: the strided entry at the headline shape (B2 H32 N4096 causal bf16)."""
    import torch

    import exact_attention_flash_amd as fa
    from exact_attention_flash_amd import inputs

    dev = torch.device("cuda:0")
    B, H, N = 2, 32, 4096
    cases = [("contiguous d=128 (plain entry)", 128, False), ("contiguous d=80", 80, False),
             ("contiguous d=96", 96, False), ("packed qkv [B,N,3,H,d] d=128, o [B,N,H,d]", 128, True),
             ("contiguous d=256 (plain entry, two launches)", 256, False), ("contiguous d=192", 192, False)]
    for label, d, packed in cases:
        qb, kb, vb = inputs.draw_qkv((B, H, N, d), inputs.BF16, 1.0, 3)
        q0, k0, v0 = (inputs.to_torch(x, inputs.BF16, dev) for x in (qb, kb, vb))
        if packed:
            pk = torch.stack([t.permute(0, 2, 1, 3) for t in (q0, k0, v0)], dim=2).contiguous()
            q, k, v = (pk[:, :, i].permute(0, 2, 1, 3) for i in range(3))
            o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3)
        else:
            q, k, v = q0, k0, v0
            o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        scale = inputs.default_scale(d)
        stream = torch.cuda.current_stream(dev)
        if d in (128, 256) and not packed:
            step = lambda: fa.flash_attn_fwd(q, k, v, o, lse, causal=True, scale=scale, stream=stream)
        else:
            step = lambda: fa.flash_attn_fwd_strided(q, k, v, o, lse, causal=True, scale=scale, stream=stream)
        # same protocol as time_gpu: warm-up, one pass of per-launch events (this also
        # brings the clocks back up after the idle time of drawing the inputs), then
        # the timed back-to-back launches
        for _ in range(args.warmup):
            step()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a_, b_ in evs:
            a_.record(stream)
            step()
            b_.record(stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        flops = 4.0 * B * H * N * N * d / 2
        print(json.dumps({"metric": "attention fwd TFLOP/s, strided entry (diagnostic)", "case": label,
                          "config": {"B": B, "H": H, "N": N, "d": d, "causal": True, "dtype": "bf16"},
                          "launch_ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                          "pct_of_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                          "steps": args.steps, "warmup": args.warmup}), flush=True)


def _time_calls(step, steps, warmup, stream):
    """time_gpu's protocol for an arbitrary step: warm-up, per-launch events, timed run."""
    import torch

    for _ in range(warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a_, b_ in evs:
        a_.record(stream)
        step()
        b_.record(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, statistics.median(a_.elapsed_time(b_) for a_, b_ in evs)


def run_fp8(args):
    """Diagnostic lines: the FP8 forward at the headline shape (B2 H32 N4096 d128 causal)
    and at the same shape with d = 64, E4M3 and E5M2."""
    import torch

    import exact_attention_flash_amd as fa
    from exact_attention_flash_amd import inputs

    head = inputs.WORKLOADS[inputs.HEADLINE]
    d64 = inputs.Workload("llama7b_shape_b2_h32_n4096_d64_causal", head.B, head.H, head.N, 64, head.dtype,
                          head.sigma, (True,), head.seed)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for w in (head, d64):
        qb, kb, vb = inputs.workload_qkv(w)
        q, k, v = (inputs.to_torch(x, w.dtype, dev) for x in (qb, kb, vb))
        scale = inputs.default_scale(w.d)
        for fmt in ("e4m3", "e5m2"):
            q8, qs = fa.quantize_fp8(q, fmt=fmt)
            k8, ks = fa.quantize_fp8(k, fmt=fmt)
            v8, vs = fa.quantize_fp8(v, keys_transposed=True, fmt=fmt)
            o = torch.empty_like(q)
            lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

            def attn():
                fa.flash_attn_fwd_fp8(q8, k8, v8, qs, ks, vs, o, lse, causal=True, scale=scale, stream=stream,
                                      fmt=fmt)

            def quant():
                fa.quantize_fp8(q, stream=stream, fmt=fmt)
                fa.quantize_fp8(k, stream=stream, fmt=fmt)
                fa.quantize_fp8(v, keys_transposed=True, stream=stream, fmt=fmt)

            ms, med = _time_calls(attn, args.steps, args.warmup, stream)
            qms, _ = _time_calls(quant, max(10, args.steps // 4), args.warmup, stream)
            flops = w.flops(True)
            tf = flops / (ms * 1e-3) / 1e12
            in_bytes = 3 * w.B * w.H * w.N * w.d * 2
            print(json.dumps({
                "metric": "attention fwd TFLOP/s on FP8 inputs (diagnostic)",
                "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": True,
                           "inputs": f"{fmt.upper()}, power-of-two scale per 64 rows", "out_dtype": w.dtype},
                "value": round(tf, 2), "unit": "TFLOP/s", "launch_ms": round(ms, 5),
                "launch_ms_median": round(med, 5),
                "pct_of_fp8_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2),
                "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                "quantize_q_k_v_ms": round(qms, 5),
                "quantize_GB_per_s": round((in_bytes + in_bytes / 2) / (qms * 1e-3) / 1e9, 1),
                "steps": args.steps, "warmup": args.warmup}), flush=True)


def run(args, workload_name, causal):
    from exact_attention_flash_amd import inputs

    w = inputs.WORKLOADS[workload_name]
    flops = w.flops(causal)
    g, qkv = time_gpu(w, causal, args.steps, args.warmup)
    tflops = flops / (g["ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (g["event_ms_per_launch"] * 1e-3) / 1e12
    kernel = fwd_kernel_of(w, causal)
    traffic = measured_traffic(workload_name, causal, kernel)
    line = {
        "metric": "attention fwd TFLOP/s and % of bf16 MFMA peak, N=4096 d=128 causal",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": causal,
                   "dtype": w.dtype, "sigma": w.sigma, "seed": w.seed, "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": kernel_symbol(kernel),
            "flop_per_launch": flops,
            "launch_ms": round(g["event_ms_per_launch"], 5),
            "launch_ms_median": round(g["launch_ms_median"], 5),
            "launch_ms_p10": round(g["launch_ms_p10"], 5),
            "launch_ms_p90": round(g["launch_ms_p90"], 5),
            "compulsory_hbm_bytes": w.compulsory_bytes(),
        },
        "extra_alloc_bytes": g["extra_alloc_bytes"],
        "device": g["device"],
        "kernel_source_sha256_16": kernel_source_hash(kernel),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, causal, qkv, args.cpu_slices, g["gpu_out"])
    return line


def run_table(args):
    """One line per workload and mask: launch-time distribution, TFLOP/s, % of peak,
    recorded HBM bytes, and the oracle's time and parity metrics on whole slices."""
    from exact_attention_flash_amd import inputs

    for name, w in inputs.WORKLOADS.items():
        for causal in w.causal:
            g, qkv = time_gpu(w, causal, args.steps, args.warmup)
            flops = w.flops(causal)
            med = g["launch_ms_median"]
            cb = cpu_baseline(w, causal, qkv, TABLE_SLICES[name], g["gpu_out"])
            kernel = fwd_kernel_of(w, causal)
            print(json.dumps({
                "workload": name, "dtype": w.dtype, "causal": causal, "kernel": kernel_symbol(kernel),
                "launch_ms_median": round(med, 5), "launch_ms_p10": round(g["launch_ms_p10"], 5),
                "launch_ms_p90": round(g["launch_ms_p90"], 5),
                "tflops_at_median": round(flops / (med * 1e-3) / 1e12, 2),
                "pct_of_bf16_peak": round(100.0 * flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                "hbm_bytes_per_launch": measured_traffic(name, causal, kernel),
                "compulsory_hbm_bytes": w.compulsory_bytes(),
                "parity": cb["parity"], "oracle_seconds": round(cb["seconds"], 2), "oracle_cores": cb["cores"],
                "kernel_source_sha256_16": kernel_source_hash(kernel), "device": g["device"],
                "steps": args.steps, "warmup": args.warmup}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: the LLaMA-7B causal one)")
    ap.add_argument("--causal", type=int, default=None, help="override the mask for --workload (0/1)")
    ap.add_argument("--all", action="store_true", help="one line per workload and mask (diagnostics)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-slices", type=int, default=64, help="(batch, head) slices the oracle times")
    ap.add_argument("--bwd", action="store_true", help="time the backward pass instead (diagnostic line)")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 forward and the quantization at the headline shape (diagnostic)")
    ap.add_argument("--strided", action="store_true",
                    help="time the strided entry (head dims 80/96, packed qkv) at the headline shape (diagnostic)")
    ap.add_argument("--splitkv", action="store_true",
                    help="time the key-split forward against the plain one on underfilled shapes (diagnostic)")
    ap.add_argument("--cpu-bwd-slices", type=int, default=16,
                    help="(batch, head) slices the backward oracle times with --bwd")
    ap.add_argument("--table", action="store_true",
                    help="one line per workload and mask with timing distribution, recorded HBM bytes and "
                         "oracle parity on whole slices (diagnostic)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run plain device-to-device copies of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the forward pass shards over (batch, head) with no communication; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") != "1":
        print("bench.py: launched with WORLD_SIZE > 1; only one GPU is supported", file=sys.stderr)
        sys.exit(2)

    if args.copy_calib:
        copy_calibration(args.copy_calib, args.steps)
        return

    from exact_attention_flash_amd import inputs

    if args.table:
        run_table(args)
        return
    if args.splitkv:
        run_splitkv(args)
        return
    if args.strided:
        run_strided(args)
        return
    if args.fp8:
        run_fp8(args)
        return
    runner = run_bwd if args.bwd else run
    if args.all:
        for name, w in inputs.WORKLOADS.items():
            for c in w.causal:
                args2 = argparse.Namespace(**vars(args))
                args2.no_cpu_baseline = True
                print(json.dumps(runner(args2, name, c)), flush=True)
        return
    name = args.workload or inputs.HEADLINE
    causal = inputs.WORKLOADS[name].causal[0] if args.causal is None else bool(args.causal)
    print(json.dumps(runner(args, name, causal)), flush=True)


if __name__ == "__main__":
    main()
