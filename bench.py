#!/usr/bin/env python3
"""Benchmark of the NVFP4 data path on one MI355X.

Default workload (one "step"): one KV-cache chunk of 8 latent frames x 880
tokens = 7040 tokens, 24 heads x 128, K and V in bf16 -- K-smoothing
statistics, NVFP4 4/6 quantization of K_s and V into a ring slot
(kv_store_chunk), then dequantization of the chunk back to bf16
(gather_window of the next step, window of one chunk, no sinks).  Inputs are
resident in HBM before the timed region; four buffer sets are rotated so
consecutive steps do not hit the 256 MB last-level cache with the previous
step's data.

Prints one JSON line.  `value` is algorithmic GB/s of the whole step (one read
of every input, one write of every output), from the mean of the timed steps;
`median_ms_per_step` is the median of the steps' own event-timed durations.
`roofline` is the dominant kernel: algorithmic bytes per launch / its mean
launch time from HIP events recorded around each launch on the launch's own
stream, against 8 TB/s, with what it reads cold and what may come from the
last-level cache.  `cpu_baseline` times the CPU oracle (test infrastructure)
on the whole chunk on all the host's usable cores, and on one thread.
`secondary` carries, each as a step of its own: the store alone and with the
producer's value amax, the gather at a steady-state ring step (33,440
tokens), the activation quantize (all cold, rotated sets), the W4A4 GEMM
(7040x3072x3072, TFLOP/s vs the 2.5 PFLOP/s dense fp16/bf16 MFMA peak), the
MXFP4 comparison, the FFN chain (labelled warm), the 64 s ring, the small
configuration, the weight-gradient RHT and LoRA lines and the fused
attention.

Other workloads (--workload): kv_store, kv_store_vamax, gather_steady, gemm_attn, ffn,
ring64s, quant_act, wgrad, lora, attn.
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

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
MFMA_FP4_PEAK_TFLOPS = 10100.0
METRIC = "NVFP4 quant/dequant GB/s (% HBM peak); W4A4 GEMM TFLOP/s (% bf16 MFMA peak)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="kv_chunk",
                    choices=["kv_chunk", "kv_store", "kv_store_vamax", "gather_steady",
                             "gemm_attn", "ffn", "ring64s", "quant_act", "wgrad", "lora", "attn"])
    ap.add_argument("--sets", type=int, default=4, help="rotated input/output buffer sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain device copy of 256 MiB first (for scaling HBM counters)")
    return ap.parse_args()


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def bf16_from_bits(bits, device):
    import numpy as np
    import torch

    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)


WARMUP_MIN_S = 0.25  # every timing warms up for at least this long (clocks settle)


def time_steps(step_fn, steps, warmup, per_step=False, warm_s=WARMUP_MIN_S):
    """Mean ms per step over `steps` steps bracketed by synchronisations (and
    the wall-clock mean), after `warmup` untimed steps and at least `warm_s`
    seconds of untimed steps (the shader clock takes about a tenth of a
    second of sustained work to settle: back-to-back W4A4 GEMMs went 136 ->
    124 -> 118 us a call over the first runs).  Nothing but the steps runs
    between the two synchronisations.  With per_step, a second pass of
    `steps` steps records an event after every step and gives the median of
    the steps' own durations (each such event adds ~2.5 us to a step on this
    GPU, so the mean is taken from the first pass)."""
    import torch

    i = 0
    t0 = time.perf_counter()
    while i < warmup or time.perf_counter() - t0 < warm_s:
        step_fn(i)
        i += 1
        if i >= warmup and i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    w0 = time.perf_counter()
    ev[0].record(s)
    for k in range(steps):
        step_fn(i + k)
    ev[1].record(s)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - w0) * 1e3
    mean = ev[0].elapsed_time(ev[1]) / steps
    if not per_step:
        return mean, wall / steps
    i += steps
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    pe[0].record(s)
    for k in range(steps):
        step_fn(i + k)
        pe[k + 1].record(s)
    torch.cuda.synchronize()
    med = statistics.median(pe[k].elapsed_time(pe[k + 1]) for k in range(steps))
    return mean, wall / steps, med


def kernel_times(nv, step_fn, steps, base):
    """Per-kernel mean launch time (ms) from the library's event timing."""
    import torch

    torch.cuda.synchronize()
    nv.profile_collect()
    nv.profile_enable(True)
    for i in range(steps):
        step_fn(base + i)
    torch.cuda.synchronize()
    nv.profile_enable(False)
    rec = nv.profile_collect()
    return {k: (n, ms / n) for k, (n, ms) in rec.items() if n}


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, alg_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get("kernels", {}).get(kernel)
    if not ent or ent.get("source_hash") != source_hash(data.get("sources", [])):
        return None
    return ent.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

KV_T, KV_H, KV_D = 7040, 24, 128


def kv_bytes_per_chunk(T=KV_T, H=KV_H, D=KV_D):
    """Algorithmic bytes of storing (or dequantizing) one chunk: bf16 K and V
    (2 B/element) on one side, packed NVFP4 ((9/8) B per K+V element pair,
    i.e. 0.5625 B/element) plus the key mean (fp32 [H*D]) and two fp32 tensor
    scales on the other."""
    elems = 2 * T * H * D
    return elems * 2 + elems * 9 // 16 + H * D * 4 + 8


def setup_kv_chunk(nv, args, dev):
    import numpy as np
    import torch

    import synth

    kb, vb = synth.kv_chunk(1002, 0, KV_T, KV_H, KV_D)
    K0, V0 = bf16_from_bits(kb, dev), bf16_from_bits(vb, dev)
    Ks = [K0.clone() for _ in range(args.sets)]
    Vs = [V0.clone() for _ in range(args.sets)]
    Ko = [torch.empty_like(K0) for _ in range(args.sets)]
    Vo = [torch.empty_like(V0) for _ in range(args.sets)]
    cfg = nv.KVConfig(sink_frames_global=0, sink_frames_shot=0, window_chunks=1)
    ring = nv.KVRing(cfg)
    state = {"t": 0}

    def step(i):
        j = i % args.sets
        t = state["t"]
        ring.store_chunk(t, Ks[j], Vs[j])
        ring.gather_window(t + 1, Ko[j], Vo[j])
        state["t"] = t + 1

    return step, {"K": kb, "V": vb}


def host_info():
    """nproc and the CPU model of this host (lscpu), for the CPU baseline."""
    import subprocess

    info = {"nproc": os.cpu_count()}
    try:
        info["nproc"] = int(subprocess.run(["nproc"], capture_output=True, text=True,
                                           timeout=10).stdout.strip())
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    return info


def cpu_baseline_kv(sample_tokens=KV_T, reps=3):
    """The oracle on the whole chunk (7040 x 24 x 128 K and V): K-smoothing,
    4/6 quantization of K_s and V, then dequantization of both back to bf16,
    in GB/s of the same algorithmic bytes.  Timed as it stands on all the
    host's usable cores (the oracle's row-range driver: one C call per row
    range on a thread pool; the statistics pass is single-threaded), `reps`
    times, and once on one thread."""
    import numpy as np

    import oracle
    import synth

    threads = synth.host_threads()
    kb, vb = synth.kv_chunk(1002, 0, sample_tokens, KV_H, KV_D, threads=threads)
    K = synth.bf16_bits_to_f32(kb).reshape(sample_tokens, -1)
    V = synth.bf16_bits_to_f32(vb).reshape(sample_tokens, -1)
    oracle.lib()

    def one(n):
        ch = oracle.kv_encode_chunk(K, V, threads=n)
        oracle.kv_dequant_rows(ch, key=True, threads=n)
        oracle.kv_dequant_rows(ch, key=False, threads=n)

    one(threads)  # warm-up
    t0 = time.perf_counter()
    for _ in range(reps):
        one(threads)
    dt = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    one(1)
    dt1 = time.perf_counter() - t0
    alg = 2 * kv_bytes_per_chunk(T=sample_tokens)
    out = {"value": round(alg / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"the whole chunk ({sample_tokens}x{KV_H}x{KV_D} K and V): store + "
                     f"dequantize, {reps} runs on {threads} threads ({dt:.2f} s each) and one "
                     f"on 1 thread ({dt1:.2f} s)",
           "one_thread_GB/s": round(alg / dt1 / 1e9, 4), "seconds_per_chunk": round(dt, 3),
           "seconds_per_chunk_1_thread": round(dt1, 3)}
    out.update(host_info())
    return out


def run_kv_store(nv, args, dev, producer_vamax=False):
    """The store alone (K-smoothing statistics, finalize, 4/6 quantization of
    K_s and V into a ring slot) of one 7040 x 24 x 128 chunk per step, over
    `sets` rotated input sets (4 x 86.5 MB, past the 256 MB last-level
    cache: cold).  With producer_vamax the value amax comes from the
    producer (max|V| of each set, computed before the timed region, as the
    V projection's amax_out would give it) and the statistics pass reads the
    keys only.  GB/s of the store's algorithmic bytes (K and V read once,
    packed codes, scales, mu and decode scales written once)."""
    import torch

    import synth

    kb, vb = synth.kv_chunk(1002, 0, KV_T, KV_H, KV_D, threads=synth.host_threads())
    K0, V0 = bf16_from_bits(kb, dev), bf16_from_bits(vb, dev)
    Ks = [K0.clone() for _ in range(args.sets)]
    Vs = [V0.clone() for _ in range(args.sets)]
    vmax = [V.float().abs().max().reshape(1) for V in Vs]
    ring = nv.KVRing(nv.KVConfig(sink_frames_global=0, sink_frames_shot=0, window_chunks=1))
    state = {"t": 0}

    def step(i):
        j = i % args.sets
        ring.store_chunk(state["t"], Ks[j], Vs[j], v_amax=vmax[j] if producer_vamax else None)
        state["t"] += 1

    ms, wall, med = time_steps(step, args.steps, args.warmup, per_step=True)
    kt = kernel_times(nv, step, args.steps, args.warmup + args.steps)
    alg = kv_bytes_per_chunk()
    return {"GB/s": round(alg / ms / 1e6, 1), "frac_hbm_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4),
            "us": round(ms * 1e3, 2), "median_us": round(med * 1e3, 2), "alg_bytes": alg,
            "kernels_us": {k: round(v[1] * 1e3, 2) for k, v in kt.items()},
            "cache": f"cold: {args.sets} rotated input sets"}


def run_gather_steady(nv, args, dev):
    """The gather at a steady-state step of the 64 s ring (step 15: 2640 +
    2640 sink tokens and 4 window chunks, 33,440 tokens x 24 x 128 K and V to
    bf16).  `sets` rings, each filled with the schedule's first 15 chunks,
    and as many output sets, rotate (4 x ~115 MB packed in, 4 x 411 MB out:
    cold).  GB/s of the gather's algorithmic bytes (packed K and V read
    once, bf16 written once)."""
    import torch

    import synth

    cfg = nv.KVConfig()
    kb, vb = synth.kv_chunk(1005, 0, KV_T, KV_H, KV_D, threads=synth.host_threads())
    K, V = bf16_from_bits(kb, dev), bf16_from_bits(vb, dev)
    rings = []
    for _ in range(args.sets):
        r = nv.KVRing(cfg)
        for t in range(15):
            if t % 10 == 0:
                r.begin_shot(t)
            r.store_chunk(t, K, V)
        rings.append(r)
    n = rings[0].effective_tokens(15)
    outs = [(torch.empty((n, KV_H, KV_D), dtype=torch.bfloat16, device=dev),
             torch.empty((n, KV_H, KV_D), dtype=torch.bfloat16, device=dev)) for _ in rings]

    def step(i):
        j = i % len(rings)
        rings[j].gather_window(15, *outs[j])

    ms, wall, med = time_steps(step, args.steps, args.warmup, per_step=True)
    kt = kernel_times(nv, step, args.steps, args.warmup + args.steps)
    alg = int(n * KV_H * KV_D * 2 * (2 + 0.5625))
    k_us = kt["kv_gather"][1] * 1e3
    return {"tokens": n, "GB/s": round(alg / ms / 1e6, 1),
            "frac_hbm_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4), "us": round(ms * 1e3, 2),
            "median_us": round(med * 1e3, 2), "kernel_us": round(k_us, 2),
            "kernel_GB/s": round(alg / k_us / 1e3, 1), "alg_bytes": alg,
            "cache": f"cold: {args.sets} rings and output sets rotated"}


def setup_gemm(nv, dev, M=7040, N=3072, K=3072, seed=1003):
    import torch

    import synth

    X = torch.from_numpy(synth.activations(seed, 0, M, K, 0.005, 30.0)).to(dev).to(torch.bfloat16)
    W = torch.from_numpy(synth.weights(seed, 1, N, K)).to(dev).to(torch.bfloat16)
    qa = nv.quantize(X)
    qw = nv.quantize(W, layout=nv.LAYOUT_2D)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    return X, qa, qw, Y


def run_gemm_attn(nv, args, dev):
    M, N, K = 7040, 3072, 3072
    X, qa, qw, Y = setup_gemm(nv, dev, M, N, K)

    def step(i):
        nv.gemm_w4a4(qa, qw, out=Y)

    ms, wall, med = time_steps(step, args.steps, args.warmup, per_step=True)
    kt = kernel_times(nv, step, max(5, args.steps // 5), 0)
    flops = 2.0 * M * N * K
    kms = kt["gemm_w4a4"][1]
    out = {"ms": ms, "wall_ms": wall, "median_ms": med, "tflops": flops / ms / 1e9, "kernel_ms": kms,
           "kernel_tflops": flops / kms / 1e9, "flops": flops, "kernels": kt,
           "dense_bf16_tflops": dense_bf16_tflops(dev, M, N, K)}
    out.update(mx_comparison(nv, args, dev, X, Y, M, N, K))
    return out


def mx_comparison(nv, args, dev, X, Y, M, N, K, nrows=64):
    """The MXFP4 speed reference on the same bf16 operands (E8M0 scale per
    32, native scaled FP4 MFMA), and the relative Frobenius error of both
    formats against the fp64 product of the unquantized operands on `nrows`
    sampled rows (first and last included)."""
    import numpy as np
    import torch

    import synth

    W = torch.from_numpy(synth.weights(1003, 1, N, K)).to(dev).to(torch.bfloat16)
    qa, qw = nv.mx_quantize(X), nv.mx_quantize(W)
    Ym = torch.empty_like(Y)

    def step(i):
        nv.gemm_mx(qa, qw, out=Ym)

    ms, _ = time_steps(step, args.steps, args.warmup)
    kt = kernel_times(nv, step, max(5, args.steps // 5), 0)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(5).integers(0, M, nrows - 2)]))
    x = X.float().cpu().numpy().astype(np.float64)[rows]
    w = W.float().cpu().numpy().astype(np.float64)
    ref = x @ w.T
    nrm = np.linalg.norm(ref)
    err_nv = np.linalg.norm(Y.float().cpu().numpy().astype(np.float64)[rows] - ref) / nrm
    err_mx = np.linalg.norm(Ym.float().cpu().numpy().astype(np.float64)[rows] - ref) / nrm
    return {"mx_ms": ms, "mx_kernel_ms": kt["gemm_mx"][1],
            "mx_kernel_tflops": 2.0 * M * N * K / kt["gemm_mx"][1] / 1e9,
            "rel_err_nvfp4": float(err_nv), "rel_err_mxfp4": float(err_mx)}


def dense_bf16_tflops(dev, M, N, K, reps=20):
    """Context only: the vendor library's dense bf16 GEMM (torch.matmul ->
    hipBLASLt) on the same shape and random operands, TFLOP/s."""
    import torch

    a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
    b = torch.randn(K, N, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    del c
    return 2.0 * M * N * K / (e0.elapsed_time(e1) / reps) / 1e9


def copy_gbs(dev, nbytes=256 << 20, reps=10):
    """Context only: a plain device-to-device copy (torch), GB/s counting the
    read and the write."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = [torch.empty_like(src) for _ in range(2)]
    dst[0].copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        dst[i & 1].copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * nbytes / (e0.elapsed_time(e1) / reps) / 1e6


def run_quant_act(nv, args, dev, M=7040, K=3072):
    import torch

    import synth

    X = torch.from_numpy(synth.activations(1003, 0, M, K, 0.005, 30.0)).to(dev).to(torch.bfloat16)
    Xs = [X.clone() for _ in range(args.sets)]
    outs = [nv.NVFP4Tensor.empty(M, K) for _ in range(args.sets)]
    ws = torch.empty(nv.quantize_workspace_bytes(M, K), dtype=torch.uint8, device=dev)

    def step(i):
        j = i % args.sets
        nv.quantize(Xs[j], out=outs[j], workspace=ws)

    ms, wall, med = time_steps(step, args.steps, args.warmup, per_step=True)
    kt = kernel_times(nv, step, max(5, args.steps // 5), 0)
    alg = M * K * 2 + M * K // 2 + M * K // 16 + 4
    # the same with the tensor amax from a producer (a GEMM's amax_out): the
    # encode pass alone
    amax = X.float().abs().max().reshape(1).contiguous()

    def pstep(i):
        j = i % args.sets
        nv.quantize(Xs[j], out=outs[j], workspace=ws, amax_in=amax)

    pms, _, pmed = time_steps(pstep, args.steps, args.warmup, per_step=True)
    # and back: dequantize each set to bf16 (rotated outputs)
    Ys = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(args.sets)]

    def dstep(i):
        j = i % args.sets
        nv.dequantize(outs[j], out=Ys[j])

    dms, _, dmed = time_steps(dstep, args.steps, args.warmup, per_step=True)
    dkt = kernel_times(nv, dstep, max(5, args.steps // 5), 0)
    return {"ms": ms, "wall_ms": wall, "median_ms": med, "gbs": alg / ms / 1e6, "alg_bytes": alg,
            "kernels": kt, "producer_amax_ms": pms, "producer_amax_median_ms": pmed,
            "dequant_ms": dms, "dequant_median_ms": dmed,
            "dequant_gbs": alg / dms / 1e6, "dequant_kernel_ms": dkt["dequant"][1]}


def run_ffn(nv, args, dev):
    import torch

    import synth

    M, K, F = 7040, 3072, 14336
    X = torch.from_numpy(synth.activations(1004, 0, M, K, 0.005, 30.0)).to(dev).to(torch.bfloat16)
    Wu = torch.from_numpy(synth.weights(1004, 1, F, K)).to(dev).to(torch.bfloat16)
    Wd = torch.from_numpy(synth.weights(1004, 2, K, F)).to(dev).to(torch.bfloat16)
    qx = nv.quantize(X)
    qu = nv.quantize(Wu, layout=nv.LAYOUT_2D)
    qd = nv.quantize(Wd, layout=nv.LAYOUT_2D)
    H = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    qh = nv.NVFP4Tensor.empty(M, F)
    ws = torch.empty(nv.quantize_workspace_bytes(M, F), dtype=torch.uint8, device=dev)
    Y = torch.empty((M, K), dtype=torch.bfloat16, device=dev)

    amax = torch.zeros(1, dtype=torch.float32, device=dev)

    def step(i):
        # the up projection's epilogue emits max|H|, so the requantize of H
        # skips its amax pass
        amax.zero_()
        nv.gemm_w4a4(qx, qu, out=H, amax_out=amax)
        nv.quantize(H, out=qh, workspace=ws, amax_in=amax)
        nv.gemm_w4a4(qh, qd, out=Y)

    ms, wall = time_steps(step, args.steps, args.warmup)
    kt = kernel_times(nv, step, max(3, args.steps // 5), 0)
    flops = 2.0 * 2 * M * K * F

    # producer-fused requantize: the up projection's epilogue writes H as
    # NVFP4 with the amax of the previous step (delayed scaling; the input
    # is the same every step, so it is the exact amax and H's codes equal
    # the two-call path's), and raises a fresh amax for the next step
    amax_buf = [amax.clone(), torch.zeros_like(amax)]

    def step_fused(i):
        a_in, a_out = amax_buf[i % 2], amax_buf[(i + 1) % 2]
        a_out.zero_()
        nv.gemm_w4a4_quant(qx, qu, a_in, out=qh, amax_out=a_out)
        nv.gemm_w4a4(qh, qd, out=Y)

    fms, _ = time_steps(step_fused, args.steps, args.warmup)
    fkt = kernel_times(nv, step_fused, max(3, args.steps // 5), 0)
    return {"ms": ms, "wall_ms": wall, "tflops": flops / ms / 1e9, "flops": flops, "kernels": kt,
            "fused_ms": fms, "fused_tflops": flops / fms / 1e9, "fused_kernels": fkt}


def run_lora(nv, args, dev, M=7040, N=3072, K=3072, r=32, alpha=32.0):
    """W4A4 layer with a LoRA adapter on the frozen backbone: lora_down
    (XA = bf16(X A^T)) plus the GEMM with the adapter in its epilogue, timed
    against the plain W4A4 GEMM on the same operands."""
    import torch

    import synth

    X, qa, qw, Y = setup_gemm(nv, dev, M, N, K)
    A = torch.from_numpy(synth.weights(1041, 2, r, K, 0.05)).to(dev).to(torch.bfloat16)
    B = torch.from_numpy(synth.weights(1041, 3, N, r, 0.05)).to(dev).to(torch.bfloat16)
    XA = torch.empty((M, r), dtype=torch.bfloat16, device=dev)

    def step(i):
        nv.lora_down(X, A, out=XA)
        nv.gemm_w4a4_lora(qa, qw, XA, B, alpha / r, out=Y)

    ms, _ = time_steps(step, args.steps, args.warmup)
    kt = kernel_times(nv, step, max(5, args.steps // 5), 0)
    base, _ = time_steps(lambda i: nv.gemm_w4a4(qa, qw, out=Y), args.steps, args.warmup)
    flops = 2.0 * M * N * K
    return {"rank": r, "ms": ms, "plain_gemm_ms": base,
            "overhead_vs_plain": ms / base - 1.0,
            "lora_down_us": kt["lora_down"][1] * 1e3, "gemm_lora_us": kt["gemm_w4a4_lora"][1] * 1e3,
            "tflops_backbone": flops / ms / 1e9}


def run_wgrad(nv, args, dev, T=7040, D=3072, signs=0xB7E1, nrows=64):
    """Weight-gradient GEMM dW = dY^T X (both operands 1-D along the token
    dimension) with and without the random Hadamard transform: quantize
    rates, GEMM TFLOP/s, and the relative Frobenius error of dW against the
    fp64 product of the unquantized operands on `nrows` sampled rows.  The
    token dimension is padded with zeros to a multiple of 256 (the GEMM's
    LDS path), which leaves the product unchanged; flops count T."""
    import numpy as np
    import torch

    import synth

    X = torch.from_numpy(synth.activations(1021, 0, T, D, 0.005, 30.0)).to(dev).to(torch.bfloat16)
    dY = torch.from_numpy(synth.activations(1021, 1, T, D, 0.005, 30.0)).to(dev).to(torch.bfloat16)
    Tp = (T + 255) // 256 * 256
    Xt = torch.zeros((D, Tp), dtype=torch.bfloat16, device=dev)
    dYt = torch.zeros_like(Xt)
    Xt[:, :T] = X.t()
    dYt[:, :T] = dY.t()
    ws = torch.empty(nv.quantize_workspace_bytes(D, Tp), dtype=torch.uint8, device=dev)
    qa = [nv.NVFP4Tensor.empty(D, Tp) for _ in range(2)]
    qw = [nv.NVFP4Tensor.empty(D, Tp) for _ in range(2)]
    Y = torch.empty((D, D), dtype=torch.float32, device=dev)
    out = {}
    for k, rht in enumerate((False, True)):
        def quant(i):
            if rht:
                nv.quantize_rht(dYt, signs, out=qa[k], workspace=ws)
                nv.quantize_rht(Xt, signs, out=qw[k], workspace=ws)
            else:
                nv.quantize(dYt, out=qa[k], workspace=ws)
                nv.quantize(Xt, out=qw[k], workspace=ws)

        qms, _ = time_steps(quant, args.steps, args.warmup)
        gms, _ = time_steps(lambda i: nv.gemm_w4a4(qa[k], qw[k], out=Y), args.steps, args.warmup)
        rows = np.unique(np.concatenate([[0, D - 1], np.random.default_rng(6).integers(0, D, nrows - 2)]))
        ref = dY.float().cpu().numpy().astype(np.float64).T[rows] @ X.float().cpu().numpy().astype(np.float64)
        err = np.linalg.norm(Y.cpu().numpy().astype(np.float64)[rows] - ref) / np.linalg.norm(ref)
        alg = 2 * (D * T * 2 + D * Tp * 9 // 16 + 4)
        tag = "rht" if rht else "plain"
        out[tag] = {"quantize_GB/s": round(alg / qms / 1e6, 1), "quantize_us": round(qms * 1e3, 2),
                    "gemm_TFLOP/s": round(2.0 * D * D * T / gms / 1e9, 1),
                    "gemm_us": round(gms * 1e3, 2), "rel_err_vs_fp64_unquantized": round(float(err), 5)}
    return out


def run_ring64s(nv, args, dev):
    """40 chunks; cuts every 10 chunks; per step: gather K_eff(t), store chunk t."""
    import torch

    import synth

    cfg = nv.KVConfig()
    ring = nv.KVRing(cfg)
    kb, vb = synth.kv_chunk(1005, 0, KV_T, KV_H, KV_D)
    Ks = [bf16_from_bits(kb, dev) for _ in range(args.sets)]
    Vs = [bf16_from_bits(vb, dev) for _ in range(args.sets)]
    cap = 4 * KV_T + 2 * 3 * 880
    Ko = torch.empty((cap, KV_H, KV_D), dtype=torch.bfloat16, device=dev)
    Vo = torch.empty_like(Ko)
    gathered = []

    def one_pass():
        nonlocal ring
        ring = nv.KVRing(cfg)
        n_tot = 0
        for t in range(40):
            if t % 10 == 0:
                ring.begin_shot(t)
            k, _ = ring.gather_window(t, Ko, Vo)
            n_tot += k.shape[0]
            ring.store_chunk(t, Ks[t % args.sets], Vs[t % args.sets])
        return n_tot

    n_tok = one_pass()
    torch.cuda.synchronize()
    steps = max(1, args.steps // 10)
    ms, wall = time_steps(lambda i: one_pass(), steps, 1)
    per_tok = KV_H * KV_D * 2 * (2 + 0.5625)
    alg = n_tok * per_tok + 40 * kv_bytes_per_chunk()
    return {"ms": ms, "wall_ms": wall, "gbs": alg / ms / 1e6, "tokens_gathered": n_tok,
            "alg_bytes": alg}


def run_cfg1(nv, dev, reps=50):
    """The small configuration (launch-latency bound, reported in us): 1-D 4/6
    quantize of fp32 4096x128 (amax + encode), dequantize back to fp32, and
    the W4A4 GEMM 256x256x512."""
    import torch

    import synth

    x = torch.from_numpy(synth.activations(1001, 0, 4096, 128, 0.01, 20.0)).to(dev)
    q = nv.NVFP4Tensor.empty(4096, 128)
    ws = torch.empty(nv.quantize_workspace_bytes(4096, 128), dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    A = torch.from_numpy(synth.activations(1001, 1, 256, 512, 0.01, 20.0)).to(dev)
    W = torch.from_numpy(synth.weights(1001, 2, 256, 512)).to(dev)
    qa, qw = nv.quantize(A), nv.quantize(W, layout=nv.LAYOUT_2D)
    Y = torch.empty((256, 256), dtype=torch.float32, device=dev)
    qms, _ = time_steps(lambda i: nv.quantize(x, out=q, workspace=ws), reps, 10)
    dms, _ = time_steps(lambda i: nv.dequantize(q, out=y), reps, 10)
    gms, _ = time_steps(lambda i: nv.gemm_w4a4(qa, qw, out=Y), reps, 10)
    return {"quantize_us": round(qms * 1e3, 2), "dequantize_us": round(dms * 1e3, 2),
            "gemm_256x256x512_us": round(gms * 1e3, 2),
            "note": "launch-latency bound; a parity configuration, not a roofline one"}


def attention_context(nv, dev, reps=5):
    """Context for fusing the dequantization into attention: one steady-state
    step of the 64 s ring (7040 queries against the 33,440-token effective
    set, 24 heads of 128) timed as the gather alone and as torch's flash
    attention on the gathered bf16 K/V.  Only the flash kernel is allowed (no
    fallback to the math path); None if it is unavailable."""
    import torch

    import synth

    cfg = nv.KVConfig()
    ring = nv.KVRing(cfg)
    kb, vb = synth.kv_chunk(1006, 0, KV_T, KV_H, KV_D)
    K, V = bf16_from_bits(kb, dev), bf16_from_bits(vb, dev)
    for t in range(15):  # steps 15..19 gather 33,440 tokens
        if t % 10 == 0:
            ring.begin_shot(t)
        ring.store_chunk(t, K, V)
    n = ring.effective_tokens(15)
    Ko = torch.empty((n, KV_H, KV_D), dtype=torch.bfloat16, device=dev)
    Vo = torch.empty_like(Ko)
    gms, _ = time_steps(lambda i: ring.gather_window(15, Ko, Vo), 10, 3)
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel

        q = torch.randn((1, KV_H, KV_T, KV_D), dtype=torch.bfloat16, device=dev)
        k = Ko.permute(1, 0, 2).contiguous().unsqueeze(0)
        v = Vo.permute(1, 0, 2).contiguous().unsqueeze(0)
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            torch.nn.functional.scaled_dot_product_attention(q, k, v)
    except (RuntimeError, ImportError) as e:
        return {"gather_us": round(gms * 1e3, 2), "tokens": n, "flash_attention": None,
                "note": f"flash attention unavailable: {type(e).__name__}"}
    flops = 4.0 * KV_T * n * KV_D * KV_H
    # the same attention with the dequantization fused in, straight from the ring
    qt = q[0].permute(1, 0, 2).contiguous()
    ot = torch.empty_like(qt)
    splits, wsb = ring.attention_plan(15, KV_T)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    # launches of either kernel move by ~5% with the chip's clock and
    # temperature: the two paths alternate, three rounds, medians reported
    a_ms, f_ms = [], []
    for _ in range(3):
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            a_ms.append(time_steps(
                lambda i: torch.nn.functional.scaled_dot_product_attention(q, k, v), reps, 1)[0])
        f_ms.append(time_steps(lambda i: ring.attention(15, qt, out=ot, workspace=ws), reps, 1)[0])
    ams, fms = statistics.median(a_ms), statistics.median(f_ms)
    kt = kernel_times(nv, lambda i: ring.attention(15, qt, out=ot, workspace=ws), reps, 0)
    merge = kt.get("attn_merge", (0, 0.0))[1]
    return {"tokens": n, "gather_us": round(gms * 1e3, 2), "flash_attention_ms": round(ams, 3),
            "flash_attention_TFLOP/s": round(flops / ams / 1e9, 1),
            "gather_share_of_gather_plus_attention": round(gms / (gms + ams), 4),
            "fused_dequant_attention_ms": round(fms, 3),
            "fused_dequant_attention_key_splits": splits,
            "fused_dequant_attention_kernel_ms": round(kt["attn_window"][1], 3),
            "fused_dequant_attention_merge_ms": round(merge, 3),
            "fused_dequant_attention_TFLOP/s": round(flops / fms / 1e9, 1),
            "rounds_ms": {"flash": [round(x, 3) for x in a_ms], "fused": [round(x, 3) for x in f_ms]},
            "fused_vs_gather_plus_flash": round((gms + ams) / fms, 3)}


def sustained_sclk_mhz(nv, dev, seconds=0.6):
    """Shader clock (MHz) reported by rocm-smi while W4A4 GEMMs run back to
    back; None if rocm-smi is unavailable."""
    import re
    import subprocess
    import threading

    import torch

    _, qa, qw, Y = setup_gemm(nv, dev)
    stop = threading.Event()

    def loop():
        while not stop.is_set():
            for _ in range(10):
                nv.gemm_w4a4(qa, qw, out=Y)
            torch.cuda.synchronize()

    t = threading.Thread(target=loop)
    t.start()
    try:
        time.sleep(seconds)
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=30)
        m = re.search(r'"sclk clock speed:": "\((\d+)Mhz\)"', r.stdout)
        return int(m.group(1)) if m else None
    except (OSError, subprocess.SubprocessError):
        return None
    finally:
        stop.set()
        t.join()


# --------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)
    import torch

    import nvfp4_bit_quantization_amd as nv

    nv.lib()
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # a plain copy of known size: 256 MiB read + 256 MiB written
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.workload != "kv_chunk":
        fn = {"kv_store": run_kv_store,
              "kv_store_vamax": lambda nv, args, dev: run_kv_store(nv, args, dev, True),
              "gather_steady": run_gather_steady,
              "gemm_attn": run_gemm_attn, "ffn": run_ffn, "ring64s": run_ring64s,
              "quant_act": run_quant_act, "wgrad": run_wgrad, "lora": run_lora,
              "attn": lambda nv, args, dev: attention_context(nv, dev, max(5, args.steps // 10))
              }[args.workload]
        r = fn(nv, args, dev)
        for key in ("kernels", "fused_kernels"):
            if key in r:
                r[key] = {k: {"launches": v[0], "mean_ms": v[1]} for k, v in r[key].items()}
        print(json.dumps({"workload": args.workload, **r}))
        return

    step, _ = setup_kv_chunk(nv, args, dev)
    ms, wall, med = time_steps(step, args.steps, args.warmup, per_step=True)
    alg_step = 2 * kv_bytes_per_chunk()
    gbs = alg_step / ms / 1e6
    kt = kernel_times(nv, step, args.steps, args.warmup + args.steps)
    dom = max(kt, key=lambda k: kt[k][0] * kt[k][1])
    per_launch = {"kv_encode": kv_bytes_per_chunk(), "kv_gather": kv_bytes_per_chunk(),
                  "kv_stats": 2 * KV_T * KV_H * KV_D * 2}
    k_ms = kt[dom][1]
    achieved = per_launch[dom] / k_ms / 1e6
    cache = {"kv_stats": "cold: reads the step's chunk from HBM (4 rotated input sets) while "
                         "the previous step's gather output is written back",
             "kv_encode": "re-reads the chunk kv_stats has just read: part of it may come from "
                          "the 256 MB last-level cache",
             "kv_gather": "reads the slot the store has just written (from the last-level "
                          "cache); writes cold output sets"}
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(dom, per_launch[dom]),
            "alg_bytes_per_launch": per_launch[dom], "mean_launch_us": round(k_ms * 1e3, 2),
            "cache": cache.get(dom, "")}

    out = {"metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "warmup_min_s": WARMUP_MIN_S,
           "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": "kv_chunk_quant_dequant", "tokens": KV_T, "heads": KV_H,
                      "head_dim": KV_D, "input_dtype": "bf16", "search": "4/6",
                      "buffer_sets": args.sets, "alg_bytes_per_step": alg_step},
           "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "median_ms_per_step": round(med, 5),
           "wall_ms_per_step": round(wall, 5),
           "kernels_us": {k: round(v[1] * 1e3, 2) for k, v in kt.items()},
           "roofline": roof}

    if not args.no_secondary:
        sec = {}
        # the store and the steady-state gather, each as a step of its own, cold
        ns = argparse.Namespace(steps=max(50, args.steps), warmup=10, sets=max(4, args.sets))
        sec["kv_store_step_7040x24x128_cold"] = run_kv_store(nv, ns, dev)
        sec["kv_store_step_7040x24x128_producer_value_amax_cold"] = run_kv_store(nv, ns, dev, True)
        sec["kv_gather_ring_step_15_33440_tokens_cold"] = run_gather_steady(nv, ns, dev)
        g = run_gemm_attn(nv, argparse.Namespace(steps=50, warmup=10, sets=args.sets), dev)
        sec["gemm_w4a4_7040x3072x3072_bf16"] = {
            "TFLOP/s": round(g["tflops"], 1), "frac_mfma_peak": round(g["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
            "kernel_TFLOP/s": round(g["kernel_tflops"], 1), "ms": round(g["ms"], 4),
            "median_TFLOP/s": round(2.0 * 7040 * 3072 * 3072 / g["median_ms"] / 1e9, 1),
            "peak_TFLOP/s": MFMA_F16_PEAK_TFLOPS,
            "context_dense_bf16_hipblaslt_TFLOP/s": round(g["dense_bf16_tflops"], 1),
            "rel_err_vs_fp64_unquantized": round(g["rel_err_nvfp4"], 5)}
        sec["mxfp4_reference_gemm_7040x3072x3072_bf16"] = {
            "kernel_TFLOP/s": round(g["mx_kernel_tflops"], 1),
            "peak_TFLOP/s": MFMA_FP4_PEAK_TFLOPS,
            "frac_fp4_mfma_peak": round(g["mx_kernel_tflops"] / MFMA_FP4_PEAK_TFLOPS, 4),
            "rel_err_vs_fp64_unquantized": round(g["rel_err_mxfp4"], 5),
            "note": "E8M0 scale per 32 elements: a different quantization, not NVFP4"}
        q = run_quant_act(nv, argparse.Namespace(steps=max(50, args.steps), warmup=10,
                                                 sets=max(4, args.sets)), dev)
        sec["quantize_act_7040x3072_bf16_cold"] = {
            "GB/s": round(q["gbs"], 1), "frac_hbm_peak": round(q["gbs"] / HBM_PEAK_GBS, 4),
            "us": round(q["ms"] * 1e3, 2), "median_us": round(q["median_ms"] * 1e3, 2),
            "alg_bytes": q["alg_bytes"],
            "kernels_us": {k: round(v[1] * 1e3, 2) for k, v in q["kernels"].items()},
            "cache": f"cold: {max(4, args.sets)} rotated input and output sets (4 x 43 MB bf16 in)"}
        sec["quantize_act_7040x3072_bf16_producer_amax_cold"] = {
            "GB/s": round(q["alg_bytes"] / q["producer_amax_ms"] / 1e6, 1),
            "frac_hbm_peak": round(q["alg_bytes"] / q["producer_amax_ms"] / 1e6 / HBM_PEAK_GBS, 4),
            "us": round(q["producer_amax_ms"] * 1e3, 2),
            "median_us": round(q["producer_amax_median_ms"] * 1e3, 2), "alg_bytes": q["alg_bytes"],
            "cache": f"cold: {max(4, args.sets)} rotated input and output sets; the tensor amax "
                     "given (as a producer's epilogue has it), so the encode pass alone"}
        sec["dequantize_act_7040x3072_to_bf16_cold"] = {
            "GB/s": round(q["dequant_gbs"], 1), "frac_hbm_peak": round(q["dequant_gbs"] / HBM_PEAK_GBS, 4),
            "us": round(q["dequant_ms"] * 1e3, 2), "median_us": round(q["dequant_median_ms"] * 1e3, 2),
            "kernel_us": round(q["dequant_kernel_ms"] * 1e3, 2), "alg_bytes": q["alg_bytes"],
            "cache": f"cold: {max(4, args.sets)} rotated sets"}
        w = run_wgrad(nv, argparse.Namespace(steps=10, warmup=3, sets=args.sets), dev)
        sec["wgrad_3072x3072x7040_1d_operands"] = w
        lo = run_lora(nv, argparse.Namespace(steps=20, warmup=5, sets=args.sets), dev)
        sec["lora_r32_7040x3072x3072"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                          for k, v in lo.items()}
        # the same KV step with one buffer set: the chunk's 86.5 MB stay in the
        # 256 MB last-level cache between steps (labelled warm)
        wstep, _ = setup_kv_chunk(nv, argparse.Namespace(sets=1), dev)
        wms, _ = time_steps(wstep, args.steps, args.warmup)
        sec["kv_chunk_warm_cache_1_buffer_set"] = {"GB/s": round(alg_step / wms / 1e6, 1),
                                                   "ms_per_step": round(wms, 5)}
        sec["cfg1_4096x128_fp32_and_gemm_256x256x512"] = run_cfg1(nv, dev)
        f = run_ffn(nv, argparse.Namespace(steps=5, warmup=2, sets=1), dev)
        warm = ("warm: one set of operands (packed X 12 MB, weights 2 x 24 MB, intermediate) "
                "fits the 256 MB last-level cache; the GEMMs are MFMA-bound, the requantize "
                "reads a 202 MB intermediate just written")
        sec["ffn_7040x3072x14336_up_requantize_down"] = {
            "cache": warm, "TFLOP/s": round(f["tflops"], 1), "ms": round(f["ms"], 4),
            "frac_mfma_peak": round(f["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
            "kernels_us": {k: round(v[1] * 1e3, 2) for k, v in f["kernels"].items()}}
        sec["ffn_7040x3072x14336_up_with_fused_requantize_down"] = {
            "cache": warm, "TFLOP/s": round(f["fused_tflops"], 1), "ms": round(f["fused_ms"], 4),
            "frac_mfma_peak": round(f["fused_tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
            "kernels_us": {k: round(v[1] * 1e3, 2) for k, v in f["fused_kernels"].items()}}
        r = run_ring64s(nv, argparse.Namespace(steps=10, warmup=1, sets=args.sets), dev)
        sec["ring64s_40_chunks_gather_and_store"] = {
            "GB/s": round(r["gbs"], 1), "ms_per_40_chunks": round(r["ms"], 3),
            "tokens_gathered": r["tokens_gathered"], "alg_bytes": r["alg_bytes"]}
        sec["attention_context_ring_step_33440_tokens"] = attention_context(nv, dev)
        out["secondary"] = sec
        out["context_copy_GB/s"] = round(copy_gbs(dev), 1)
        out["sclk_MHz_during_gemm"] = sustained_sclk_mhz(nv, dev)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_kv()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
