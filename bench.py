#!/usr/bin/env python3
"""Benchmark of the packed ARCHead LM-head forward on one MI355X.

Prints ONE JSON line.  ``value`` is the decode throughput (GB/s of packed head
bytes per forward, whole call: pre-projection + decode kernel) on the
Qwen3-8B-shaped decode workload (V=151936, D=4096, N=1, r_c=r_r=32, g=128);
``secondary`` carries the other half of the metric, prefill TFLOP/s on
V=151936, D=4096, N=4096, r_c=r_r=64, g=128 with bf16 logits.

Inputs are seeded synthetic tensors already resident in HBM.  Two device
copies of the packed head alternate between steps so the 256 MB last-level
cache cannot serve a head that was just read.  ``roofline`` times the dominant
kernel with HIP events that the library records on the launch stream.
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed-head logits: decode HBM GB/s and prefill TFLOP/s (% of roofline), V=151936"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
# sources that decide each main kernel's code (a counter summary is only
# reported while these are unchanged)
KERNEL_SOURCES = {
    "decode_kernel": ["decode.hip", "device_common.h", "internal.h"],
    "small_decode_kernel": ["decode_small.hip", "device_common.h", "internal.h"],
    "batch_kernel": ["batch.hip", "batch_kernel.h", "device_common.h", "internal.h"],
    "tile32_kernel": ["tile.hip", "tile32.h", "rowstat.h", "device_common.h", "internal.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg, L, N):
    """Algorithmic bytes and flops of one forward.

    Bytes: per vocabulary row D/2 + D/g + 2 + r + 2*nA bytes of the packed
    head plus N logits written; per call the B factors (r*D + 2*r*D/g bytes)
    and the bf16 hidden states (2*N*D).  That is payload_bytes + H + Y.  On the
    decode path a small pre-projection kernel reads B and H first and the
    streaming kernel reads the rest; the streaming kernel's figure counts the
    whole call's bytes (B is under 0.1% of them at the decode workloads).
    Flops: the main contraction does 2*(D + r) per logit (the tile kernel's
    unit); the pre-projection 2*N*D*r.
    """
    V, D, g, r_c, r_r = cfg["V"], cfg["D"], cfg["g"], cfg["r_c"], cfg["r_r"]
    r = r_c + r_r
    nA = (r_c > 0) + (r_r > 0)
    ysz = 2 if cfg["y_dtype"] == "bf16" else 4
    per_row = D // 2 + D // g + 2 + r + 2 * nA
    main_bytes = L["payload_bytes"] + 2 * N * D + N * V * ysz
    main_flops = 2 * N * V * (D + r)
    total_flops = main_flops + 2 * N * D * r
    return dict(per_row_bytes=per_row, main_bytes=main_bytes, main_flops=main_flops,
                total_flops=total_flops, payload=L["payload_bytes"],
                step_bytes=L["payload_bytes"] + 2 * N * D + N * V * ysz)


def kernel_hash(kernel=None):
    h = hashlib.sha256()
    names = KERNEL_SOURCES.get(kernel) or sorted({f for v in KERNEL_SOURCES.values() for f in v})
    for s in names:
        with open(os.path.join(ROOT, "compressed_output_head_amd", "csrc", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current sources of that kernel; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except (OSError, ValueError):
        return None
    if t.get("kernel") != kernel or t.get("kernel_hash") != kernel_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


COPY_CAL_BYTES = 256 << 20  # device-to-device copy used to calibrate the HBM byte counters
COPY_CAL_REPS = 4


def copy_calibration():
    """COPY_CAL_REPS device-to-device copies of COPY_CAL_BYTES, issued as the
    process's first GPU work so a counter run can find them as its first
    copy dispatches."""
    import torch
    src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(COPY_CAL_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _pmc_per_dispatch(path, counter):
    import csv
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows]


def pmc_summary(workload, kernel, fetch_csv, write_csv, commands):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    of ``bench.py --copy-calibration`` into HBM bytes per launch of ``kernel``,
    scaled by what the counters read for the calibration copies."""
    out = {"workload": workload, "kernel": kernel, "kernel_hash": kernel_hash(kernel),
           "copy_calibration_bytes": COPY_CAL_BYTES, "commands": commands}
    total = 0.0
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        d = _pmc_per_dispatch(path, name)
        cal = [v for k, v in d if "copyBuffer" in k][:COPY_CAL_REPS]
        ker = [v for k, v in d if kernel in k]
        if len(cal) < COPY_CAL_REPS or not ker:
            raise SystemExit(f"{path}: {len(cal)} calibration copies, {len(ker)} dispatches of {kernel}")
        factor = COPY_CAL_BYTES / (float(np.mean(cal)) * 1024.0)
        per_launch = float(np.mean(ker)) * 1024.0 * factor
        out[name] = {"kib_per_dispatch_mean": float(np.mean(ker)), "dispatches": len(ker),
                     "copy_kib_mean": float(np.mean(cal)), "scale": round(factor, 4),
                     "bytes_per_launch": round(per_launch)}
        total += per_launch
    out["hbm_bytes_per_launch"] = round(total)
    return out


def dominant_kernel(cfg, n_rows=None, path=0):
    """Name of the main kernel the library launches for a call of n_rows
    (default: all N) tokens of a workload on `path`."""
    import compressed_output_head_amd as ah
    return ah.archead_main_kernel(cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"],
                                  cfg["N"] if n_rows is None else n_rows, path)


# workloads whose logits are written in row chunks, one call per chunk into
# one reused buffer (the prefill workload: 512-row chunks of bf16 logits)
CHUNK_ROWS = {"prefill": 512}


def run_workload(name, steps, warmup, path=0, n_tokens=None, chunk=None):
    """K timed steps of one workload.  A step is one forward of all N tokens:
    one call, or with ``chunk`` rows one call per chunk into one reused
    [chunk x V] output buffer."""
    import torch
    import synth
    import compressed_output_head_amd as ah

    cfg = synth.config(name)
    if n_tokens is not None:
        cfg["N"] = n_tokens
    t0 = time.time()
    inp = synth.make(name, N=cfg["N"])
    packed = ah.archead_pack(inp.head)
    L = ah.archead_pack_layout(cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"])
    heads = [ah.PackedHead(cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"], packed)]
    heads.append(ah.PackedHead(cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"], heads[0].buffer.clone()))
    N = cfg["N"]
    H = torch.from_numpy(inp.H_bits.view(np.int16)).view(torch.bfloat16).cuda()
    ydt = torch.bfloat16 if cfg["y_dtype"] == "bf16" else torch.float32
    rows = min(chunk or N, N)
    Y = torch.empty((rows, cfg["V"]), dtype=ydt, device="cuda")
    parts = [H[i:i + rows] for i in range(0, N, rows)]
    for h in heads:
        h.ensure_workspace(rows)
    del inp
    log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s "
        f"(packed head {L['payload_bytes'] / 1e6:.1f} MB payload, x2 copies)")

    stream = torch.cuda.current_stream()

    def step(i):
        for Hp in parts:
            ah.archead_logits_path(Hp, heads[i % 2], Y[:Hp.shape[0]], path)

    # main-kernel events of every timed call: the library's launch of the main
    # kernel records the first at the kernel's start and the second at the end
    # of the forward's last kernel (the dispatches' own timestamps: nothing
    # else goes on the stream)
    nev = steps * len(parts)
    evb = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    eve = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    for e in evb + eve:
        e.record(stream)  # creates the underlying hipEvent

    def step_ev(i):
        for j, Hp in enumerate(parts):
            k = i * len(parts) + j
            ah.archead_logits_events(Hp, heads[i % 2], Y[:Hp.shape[0]], path, evb[k], eve[k])

    for i in range(warmup):
        step(i)
    # timed region: K whole forward steps, nothing else on the stream
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # dominant-kernel duration: the same K steps again, back to back, with the
    # launches recording their events (a launch that records events costs a
    # few microseconds of dispatch, so the timed loop above runs without them);
    # a chunked step's kernel time is the sum over its chunks
    for i in range(steps):
        step_ev(i)
    torch.cuda.synchronize()
    kms = [sum(evb[i * len(parts) + j].elapsed_time(eve[i * len(parts) + j]) for j in range(len(parts)))
           for i in range(steps)]
    A = algorithmic(cfg, L, N)
    return dict(cfg=cfg, L=L, A=A, ms=ms, kernel=dominant_kernel(cfg, rows, path), kernel_ms=float(np.mean(kms)),
                chunk_rows=rows if rows < N else None, calls_per_step=len(parts),
                kernel_ms_min=float(np.min(kms)), kernel_ms_max=float(np.max(kms)),
                kernel_ms_pct=[round(float(np.percentile(kms, q)), 5) for q in (10, 50, 90)])


def run_stats(name, steps, warmup):
    """archead_logits_stats (row max, argmax, log-sum-exp, cross-entropy; no
    logits written) on one workload, K timed calls."""
    import torch
    import synth
    import compressed_output_head_amd as ah

    cfg = synth.config(name)
    inp = synth.make(name)
    packed = ah.archead_pack(inp.head)
    heads = [ah.PackedHead(cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"], packed)]
    heads.append(ah.PackedHead(cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"], heads[0].buffer.clone()))
    N = cfg["N"]
    H = torch.from_numpy(inp.H_bits.view(np.int16)).view(torch.bfloat16).cuda()
    targets = torch.as_tensor(np.random.default_rng(0).integers(0, cfg["V"], size=N).astype(np.int32), device="cuda")
    del inp
    for i in range(warmup):
        ah.archead_logits_stats(H, heads[i % 2], targets)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        ah.archead_logits_stats(H, heads[i % 2], targets)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    flops = 2 * N * cfg["V"] * (cfg["D"] + cfg["r_c"] + cfg["r_r"]) + 2 * N * cfg["D"] * (cfg["r_c"] + cfg["r_r"])
    return {"workload": name, "ms_per_call": round(ms, 4), "steps": steps,
            "what": "row max, argmax, log-sum-exp and cross-entropy of given targets; the logits are never written",
            "tflops": round(flops / (ms / 1e3) / 1e12, 2)}


FP64_PEAK_TFLOPS = 78.6  # MI355X vector fp64

ALT_NAMES = {1: "group_int4", 2: "row_int8"}


def run_alt(name, fmt, steps, warmup, archead_ms=None):
    """archead_logits on a storage-matched comparison head (fmt 1: group INT4
    with fp16 group scales; fmt 2: row INT8) of one workload's shape (V, D, g,
    N): K timed whole calls, two copies of the head rotated as in the main
    workload, and the main kernel's time from the library's events (with more
    than 32 tokens, the events span every launch of the call and the later
    launches' conversions)."""
    import torch
    import synth
    import compressed_output_head_amd as ah

    cfg = synth.config(name)
    V, D, g, N = cfg["V"], cfg["D"], cfg["g"], cfg["N"]
    H_bits, h = synth.make_alt(fmt, 11 + fmt, V, D, N, g)
    packed = ah.archead_pack(h)
    L = ah.archead_pack_layout(V, D, 0, 0, g, fmt)
    heads = [ah.PackedHead(V, D, 0, 0, g, packed, fmt=fmt)]
    heads.append(ah.PackedHead(V, D, 0, 0, g, heads[0].buffer.clone(), fmt=fmt))
    H = torch.from_numpy(H_bits.view(np.int16)).view(torch.bfloat16).cuda()
    Y = torch.empty((N, V), dtype=torch.bfloat16 if cfg["y_dtype"] == "bf16" else torch.float32, device="cuda")
    for hd in heads:
        hd.ensure_workspace(N)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        ah.archead_logits(H, heads[i % 2], Y)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        ah.archead_logits(H, heads[i % 2], Y)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # main-kernel spans of back-to-back calls (recorded by the launches themselves)
    ebs = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ees = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for e in ebs + ees:
        e.record(stream)  # creates the underlying hipEvents
    torch.cuda.synchronize()
    for i in range(steps):
        ah.archead_logits_events(H, heads[i % 2], Y, 0, ebs[i], ees[i])
    torch.cuda.synchronize()
    kernel_ms = float(np.mean([ebs[i].elapsed_time(ees[i]) for i in range(steps)]))
    payload = L["payload_bytes"]
    out = {"workload": name, "format": ALT_NAMES[fmt], "N": N, "ms_per_call": round(ms, 5),
           "kernel_ms": round(kernel_ms, 5), "launches": (N + 31) // 32, "payload_bytes": payload,
           "head_gbps": round(payload / (kernel_ms / 1e3) / 1e9, 1) if N <= 32 else None}
    if archead_ms:
        out["ms_vs_archead"] = round(ms / archead_ms, 3)
    return out


def run_topk(name, steps, warmup, k=10):
    """archead_logits_topk (top-k logits and indices per row; the forward
    writes fp32 logits of 256-token chunks into the workspace and the
    selection kernel reads them back) on one workload, K timed calls."""
    import torch
    import synth
    import compressed_output_head_amd as ah

    cfg = synth.config(name)
    inp = synth.make(name)
    head = ah.PackedHead.from_components(inp.head)
    H = torch.from_numpy(inp.H_bits.view(np.int16)).view(torch.bfloat16).cuda()
    del inp
    for _ in range(warmup):
        ah.archead_logits_topk(H, head, k)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        ah.archead_logits_topk(H, head, k)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    return {"workload": name, "k": k, "ms_per_call": round(ms, 4), "steps": steps,
            "what": "k largest logits and their indices per row; fp32 logits of 256-token chunks pass "
                    "through the workspace once"}


def run_quantize(name, steps, warmup):
    """archead_quantize (the packing step) on one workload's head shape: dense
    bf16 W and fp32 factors resident in HBM, K timed calls of the whole step
    (zero fill, header, four INT8 passes, the residual/SC4 kernel), without
    the optional error output.  The residual kernel is fp64-bound: 2 V D r_c
    flops of core products; the HBM bytes are W read once plus the packed
    buffer written once."""
    import torch
    import synth
    import compressed_output_head_amd as ah

    cfg = synth.config(name)
    V, D, r_c, r_r, g = cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"]
    dense = synth.draw_dense(np.random.default_rng(2024), V, D, r_c, r_r, "bf16")
    W = torch.from_numpy(dense.W.view(np.int16)).view(torch.bfloat16).cuda()
    F = [torch.from_numpy(x).cuda() for x in (dense.A_c, dense.B_c, dense.A_w, dense.B_w)]
    del dense
    for _ in range(warmup):
        ah.archead_quantize(W, *F, g)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        ah.archead_quantize(W, *F, g)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    flops = 2 * V * D * r_c
    nbytes = 2 * V * D + ah.archead_pack_layout(V, D, r_c, r_r, g)["total_bytes"]
    tf = flops / (ms / 1e3) / 1e12
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": name, "V": V, "D": D, "r_c": r_c, "r_r": r_r, "g": g, "W": "bf16",
            "ms_per_call": round(ms, 4), "steps": steps, "timed": "whole call",
            "fp64_tflops": round(tf, 2), "fp64_frac": round(tf / FP64_PEAK_TFLOPS, 4),
            "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic": {"fp64_flops": flops, "bytes": nbytes},
            "roofline": {"bound": "alu", "achieved": round(tf, 2), "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / FP64_PEAK_TFLOPS, 4), "traffic": None,
                         "timed": "whole call; the fp64 core products of the residual kernel"}}


FP32_PEAK_TFLOPS = 157.3  # MI355X fp32


def run_fit(name, steps, n_calib=4096, oversample=8, power_iters=2, p=0.75, lam=0.01):
    """archead_fit (the whole construction) on one workload's head shape: bf16
    W, n_calib bf16 calibration tokens and the test matrices resident in HBM;
    K timed calls (each waits for its stream).  Work: the products the call
    performs: the passes of the two randomized SVDs over W and E (the
    correction applies T_p to each thin panel instead of forming E T_p), the
    Cholesky-QR panels and Gram matrices, the covariance, the two metric
    transforms and the map-back; the eigendecomposition of the covariance is
    not counted."""
    import torch
    import synth
    import compressed_output_head_amd as ah

    cfg = synth.config(name)
    V, D, r_c, r_r, g = cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"]
    fi = synth.draw_fit(np.random.default_rng(77), V, D, r_c, r_r, n_calib, oversample=oversample)
    dev = lambda x: torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()
    W, H = dev(fi.W).view(torch.bfloat16), dev(fi.H).view(torch.bfloat16)
    oc, orr = dev(fi.omega_c), dev(fi.omega_r)
    del fi
    ah.archead_fit(W, H, oc, orr, r_c, r_r, g, p=p, lam=lam, oversample=oversample, power_iters=power_iters)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ah.archead_fit(W, H, oc, orr, r_c, r_r, g, p=p, lam=lam, oversample=oversample, power_iters=power_iters)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    kc, kr = r_c + oversample, r_r + oversample
    passes = 2 * power_iters + 2  # M Omega, q times (M^T Y, M Z), Q^T M
    flops = 0
    for k, r, metric in ((kc, r_c, False), (kr, r_r, True)):
        if r == 0:
            continue
        flops += 2 * V * D * k * passes + 2 * V * k * r + 2 * D * k * r     # passes over M, the factors
        flops += (power_iters + 1) * 2 * 4 * V * k * k + power_iters * 2 * 4 * D * k * k  # CholeskyQR2 panels
        flops += 2 * D * k * k                                               # Gram matrix of the sketch
        if metric:
            flops += passes * 2 * D * D * k                                   # T_p applied to thin panels
    if r_r:
        flops += 2 * n_calib * D * D + 2 * 2 * D ** 3 + 2 * D * D * r_r      # covariance, T_p, T_p^-1, map-back
    tf = flops / (ms / 1e3) / 1e12
    return {"workload": name, "V": V, "D": D, "r_c": r_c, "r_r": r_r, "g": g, "calibration_tokens": n_calib,
            "p": p, "lambda": lam, "oversample": oversample, "power_iters": power_iters,
            "ms_per_call": round(ms, 2), "steps": steps, "timed": "whole call, host clock (the call waits)",
            "fp32_tflops": round(tf, 2), "fp32_frac": round(tf / FP32_PEAK_TFLOPS, 4), "fp32_flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / FP32_PEAK_TFLOPS, 4), "traffic": None,
                         "timed": "whole call; the products it performs (the covariance eigensolver, "
                                  "latency-bound, overlaps the core on a second stream and is not counted)"}}


def dense_context(name, steps=10):
    """Measured ceilings for context (not the target): a dense bf16
    torch.matmul of the workload's shapes (H [N x D] times a dense [D x V]
    head, what the packed format avoids storing), and a device-to-device copy
    of the packed head's size (read + write)."""
    import torch
    import synth
    cfg = synth.config(name)
    N, V, D = cfg["N"], cfg["V"], cfg["D"]
    H = torch.randn(N, D, device="cuda", dtype=torch.bfloat16)
    W = torch.randn(D, V, device="cuda", dtype=torch.bfloat16)
    out = {}
    for _ in range(2):
        torch.matmul(H, W)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        torch.matmul(H, W)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    out["dense_bf16_matmul"] = {"shape": [N, D, V], "ms": round(ms, 4),
                                "tflops": round(2 * N * V * D / (ms / 1e3) / 1e12, 1),
                                "dense_head_bytes": 2 * V * D}
    del H, W
    src = torch.empty(336 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    out["device_copy"] = {"bytes": src.numel(), "ms": round(ms, 4),
                          "gbs_read_plus_write": round(2 * src.numel() / (ms / 1e3) / 1e9, 1)}
    return out


def tile_workload(N):
    """Workloads of more than 64 tokens are bound by the MFMA and reported in
    TFLOP/s against its peak; up to 64 tokens the head's bytes bound the call,
    reported in GB/s of packed head bytes against the HBM peak."""
    return N > 64


def blas_info():
    """The BLAS numpy (and so the oracle's matrix products) runs on, and its threads."""
    info = {"name": None, "version": None, "threads": None}
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        info["name"], info["version"] = b.get("name"), b.get("version")
    except Exception:
        pass
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            info["threads"] = max(p.get("num_threads", 1) for p in pools)
            info["name"] = info["name"] or pools[0].get("internal_api")
    except Exception:
        pass
    return info


def cpu_baseline(name, sample_rows, min_seconds=6.0):
    """The oracle as it stands, timed on a bounded sample of the workload:
    the first ``sample_rows`` vocabulary rows, repeated until at least
    ``min_seconds`` of host time have passed.  Reported in the workload's own
    unit: GB/s of packed bytes of those rows, or TFLOP/s of their logits.
    ``gemm_only`` times the fp64 product H W_hat^T alone on the same rows
    (W_hat rebuilt once beforehand), to show how much of the oracle is the
    unpacking and rebuilding of W_hat."""
    import synth
    import oracle
    blas = blas_info()
    cfg = synth.config(name)
    inp = synth.make(name)
    cols = np.arange(min(sample_rows, cfg["V"]))

    def timed(fn):
        reps, t0 = 0, time.time()
        while True:
            fn()
            reps += 1
            if time.time() - t0 >= min_seconds:
                return reps, time.time() - t0

    reps, dt = timed(lambda: oracle.logits(inp.H_bits, inp.head, cols=cols))
    Hf = oracle.bf16_bits_to_f64(inp.H_bits)
    Wc = oracle.w_hat(inp.head, 0, int(cols.size))  # the rows of the sample: 0 .. n-1
    reps_g, dt_g = timed(lambda: Hf @ Wc.T)
    what = (f"fp64 oracle (unpack, rebuild W_hat, H W_hat^T) on vocabulary rows 0..{cols.size - 1} "
            f"of the {name} workload (N={cfg['N']}), {reps} passes in {dt:.1f}s; ")
    common = dict(cores=int(blas["threads"] or 1), kind="oracle", blas=blas,
                  sample_rows=int(cols.size), seconds=round(dt, 2))
    if tile_workload(cfg["N"]):
        r = cfg["r_c"] + cfg["r_r"]
        per_pass = 2 * cfg["N"] * cols.size * (cfg["D"] + r)
        v, vg = per_pass * reps / dt / 1e12, 2 * cfg["N"] * cols.size * cfg["D"] * reps_g / dt_g / 1e12
        return dict(value=round(v, 6), unit="TFLOP/s", **common,
                    gemm_only=dict(value=round(vg, 6), unit="TFLOP/s of the dgemm's own flops",
                                   seconds=round(dt_g, 2), passes=reps_g),
                    sample=what + "TFLOP/s of the logits of those rows (2 N (D + r_c + r_r) per logit)")
    L = oracle.layout(cfg["V"], cfg["D"], cfg["r_c"], cfg["r_r"], cfg["g"])
    per_pass = L["payload_bytes"] * cols.size / cfg["V"]
    return dict(value=round(per_pass * reps / dt / 1e9, 4), unit="GB/s", **common,
                gemm_only=dict(value=round(per_pass * reps_g / dt_g / 1e9, 4),
                               unit="GB/s of the same packed bytes, H W_hat^T alone",
                               seconds=round(dt_g, 2), passes=reps_g),
                sample=what + "GB/s of packed bytes of those rows")


# vocabulary rows of each workload the CPU oracle is timed on (about 5-10 s each)
CPU_SAMPLE_ROWS = {"decode": 151936, "batched": 32768, "prefill": 1024, "head70b": 4096}


def roofline_decode(r):
    A = r["A"]
    achieved = A["main_bytes"] / (r["kernel_ms"] / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(r["cfg"]["name"], r["kernel"]),
            "kernel": r["kernel"], "kernel_ms": round(r["kernel_ms"], 5),
            "algorithmic_bytes_per_launch": A["main_bytes"]}


def roofline_tile(r):
    A = r["A"]
    achieved = A["main_flops"] / (r["kernel_ms"] / 1e3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic_for(r["cfg"]["name"], r["kernel"]),
            "kernel": r["kernel"], "kernel_ms": round(r["kernel_ms"], 4),
            "algorithmic_flops_per_launch": A["main_flops"]}


def summary(r):
    """(value, unit, roofline) of one workload run: whole-call throughput in
    the workload's unit, and the dominant kernel against its roofline."""
    A = r["A"]
    if tile_workload(r["cfg"]["N"]):
        return round(A["total_flops"] / (r["ms"] / 1e3) / 1e12, 2), "TFLOP/s", roofline_tile(r)
    return round(A["payload"] / (r["ms"] / 1e3) / 1e9, 1), "GB/s", roofline_decode(r)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode", help="headline workload (decode, batched, prefill, head70b)")
    ap.add_argument("--n", type=int, default=None, help="token count of the headline workload (default: its own)")
    ap.add_argument("--secondary", default="prefill,batched,head70b",
                    help="further workloads, comma-separated ('' to skip); the first is also reported as "
                         "'secondary'")
    ap.add_argument("--cpu-sample-rows", type=int, default=None,
                    help="vocabulary rows the CPU oracle is timed on (default: per workload, CPU_SAMPLE_ROWS)")
    ap.add_argument("--cpu-workloads", default="all",
                    help="workloads the CPU oracle is timed on: 'all' (the headline and --secondary) or the "
                         "headline only ('headline')")
    ap.add_argument("--stats", default="prefill",
                    help="workload timed through archead_logits_stats ('' to skip)")
    ap.add_argument("--quantize", default="decode",
                    help="head shape timed through archead_quantize, the packing step ('' to skip)")
    ap.add_argument("--topk", default="batched", help="workload timed through archead_logits_topk, k=10 ('' to skip)")
    ap.add_argument("--fit", default="decode",
                    help="head shape timed through archead_fit, the whole construction ('' to skip)")
    ap.add_argument("--compare", default="decode,batched",
                    help="workloads whose shape the two storage-matched comparison heads (group INT4, row INT8) "
                         "are timed on ('' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true", help="skip the dense-matmul and copy ceilings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run the device copies that calibrate HBM byte counters")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("WORKLOAD", "KERNEL", "FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: write profiles/traffic_WORKLOAD.json from two rocprofv3 --pmc runs")
    ap.add_argument("--pmc-commands", nargs="*", default=[], help="the commands that made the --pmc runs")
    args = ap.parse_args()

    if args.pmc_summary:
        wl, kern, fcsv, wcsv = args.pmc_summary
        t = pmc_summary(wl, kern, fcsv, wcsv, args.pmc_commands)
        with open(os.path.join(ROOT, "profiles", f"traffic_{wl}.json"), "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        copy_calibration()
    r = run_workload(args.config, args.steps, args.warmup, n_tokens=args.n)
    cfg, A = r["cfg"], r["A"]
    value, unit, roof = summary(r)
    log(f"[bench] {args.config}: {r['ms'] * 1e3:.1f} us/step, {r['kernel']} {r['kernel_ms'] * 1e3:.1f} us")
    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "V": cfg["V"], "D": cfg["D"], "N": cfg["N"], "r_c": cfg["r_c"],
                   "r_r": cfg["r_r"], "g": cfg["g"], "logits": cfg["y_dtype"],
                   "packed_payload_bytes": A["payload"], "head_copies_rotated": 2},
        "roofline": roof,
    }
    names = [w for w in args.secondary.split(",") if w]
    if names:
        out["workloads"] = {}
    for w in names:
        steps2 = max(5, args.steps // 5)
        s = run_workload(w, steps2, max(2, args.warmup // 5), chunk=CHUNK_ROWS.get(w))
        v2, u2, roof2 = summary(s)
        log(f"[bench] {w}: {s['ms']:.3f} ms/step ({s['calls_per_step']} calls), {s['kernel']} {s['kernel_ms']:.3f} ms")
        entry = {
            "workload": w, "value": v2, "unit": u2,
            "ms_per_step": round(s["ms"], 4), "steps": steps2, "calls_per_step": s["calls_per_step"],
            "config": {k: s["cfg"][k] for k in ("V", "D", "N", "r_c", "r_r", "g")} | {"logits": s["cfg"]["y_dtype"]},
            "roofline": roof2,
        }
        if s["chunk_rows"]:
            entry["chunk_rows"] = s["chunk_rows"]
            one = run_workload(w, max(3, steps2 // 2), 1)
            v1, _, roof1 = summary(one)
            entry["one_call"] = {"value": v1, "ms_per_step": round(one["ms"], 4),
                                 "kernel_ms": round(one["kernel_ms"], 4), "roofline_frac": roof1["frac"]}
            log(f"[bench] {w} in one call: {one['ms']:.3f} ms")
        out["workloads"][w] = entry
        if "secondary" not in out:
            out["secondary"] = entry
    if args.compare:
        out["comparison_heads"] = {}
        known = {args.config: r["ms"]} | {w: e["ms_per_step"] for w, e in out.get("workloads", {}).items()
                                          if "chunk_rows" not in e}
        for w in [w for w in args.compare.split(",") if w]:
            for fmt in (1, 2):
                c = run_alt(w, fmt, max(5, args.steps // 5), 2, known.get(w))
                log(f"[bench] {ALT_NAMES[fmt]} head on {w}: {c['ms_per_call'] * 1e3:.1f} us/call")
                out["comparison_heads"][f"{w}/{ALT_NAMES[fmt]}"] = c
    if args.stats:
        st = run_stats(args.stats, max(5, args.steps // 5), max(2, args.warmup // 5))
        log(f"[bench] stats on {args.stats}: {st['ms_per_call']:.3f} ms/call")
        out["stats"] = st
    if args.topk:
        tk = run_topk(args.topk, max(5, args.steps // 5), 2)
        log(f"[bench] top-k on {args.topk}: {tk['ms_per_call']:.3f} ms/call")
        out["topk"] = tk
    if args.quantize:
        q = run_quantize(args.quantize, max(3, args.steps // 10), 2)
        log(f"[bench] quantize on {args.quantize}: {q['ms_per_call']:.3f} ms/call")
        out["quantize"] = q
    if args.fit:
        ft = run_fit(args.fit, 2)
        log(f"[bench] fit on {args.fit}: {ft['ms_per_call']:.1f} ms/call")
        out["fit"] = ft
    out["roofline"]["kernel_ms_p10_p50_p90"] = r["kernel_ms_pct"]
    if not args.no_context and names:
        out["context"] = dense_context(names[0])
        log(f"[bench] context: {out['context']}")
    out["kernel_sources"] = kernel_hash()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        rows = args.cpu_sample_rows or CPU_SAMPLE_ROWS.get(args.config, 4096)
        out["cpu_baseline"] = cpu_baseline(args.config, rows)
        if args.cpu_workloads == "all":
            for w in names:
                log(f"[bench] timing the CPU oracle on {w} ...")
                out["workloads"][w]["cpu_baseline"] = cpu_baseline(w, CPU_SAMPLE_ROWS.get(w, 4096))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
