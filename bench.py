#!/usr/bin/env python3
"""Benchmark of the attention forward pass on one MI355X.

A step is one fa_fwd call over one batch of synthetic input already resident in HBM. The
default workload is the long-sequence causal prefill (B=2, H=16, N=16384, d=128, bf16); the
decode workload (B=64, H=32, Nk=8192 cache with valid lengths in [1024, 8192], d=128) is timed in
the same run and reported under "decode". Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-decode]
                  [--no-short] [--no-standard] [--no-masks] [--no-backward] [--no-fp8]
                  [--no-gemm-reference] [--no-cpu-baseline] [--cpu-seconds S] [--calibrate-copy]

"run" records the GPU, its peak engine clock, the ROCm and HIP versions, the compiler and target the
library was built with (fa_build_info) and the host CPU.
"cpu_baseline" is the fp64 oracle timed on a bounded sample of the workload on the host cores;
"parity" compares the GPU output of the last timed step with the oracle on the same rows.
"short_prefill" times the GPT-2- and BERT-shaped workloads per launch from a replayed HIP graph
(no host launch gaps) with their MFMA roofline objects.

The standard (materialising) algorithm, fa_std_fwd, is timed on the three prefill workloads and
reported under "standard_attention" with its speedup ratio against fa_fwd (the pages' headline
comparison) and the HBM roofline of the whole call on the default workload. The generalised masks
are timed on the long workload's shape and reported under "masks": a causal sliding window of
4096 keys (fa_fwd_window) and the same batch packed as variable-length sequences
(fa_fwd_varlen), with FLOPs counted over the allowed (query, key) pairs. The backward pass,
fa_bwd, is timed on the 16K causal and GPT-2 shapes and reported under "backward", its FLOPs
counted as the five products of the gradient. The e4m3 path (fa_quantize_fp8 + fa_fwd_fp8) is
timed on the 16K causal shape and reported under "fp8" with its roofline against the fp8 matrix
peak, the conversion cost, and its output's distance from the bf16 path's. "gemm_reference" is a
plain dense bf16 GEMM through torch.matmul on random operands, reported for context beside the
matrix-core fractions (what a vendor-tuned library sustains on the same box).

FLOPs are counted as 4*B*H*Nq*Nk*d, halved for causal masking. Decode bytes are the algorithmic
HBM bytes: Q, the valid K and V rows, O and lse.
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

METRIC = "attention fwd TFLOP/s (bf16) and % of MFMA peak; decode HBM GB/s"
PEAK_MFMA_BF16_TFLOPS = 2516.6   # MI355X dense bf16: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_MFMA_FP8_TFLOPS = 5033.2    # MI355X dense fp8: 256 CU x 2.4 GHz x 8192 FLOP/clk
PEAK_MFMA_FP32_TFLOPS = 157.3    # MI355X dense fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
# Sources each profiled kernel is built from: a committed counter summary counts for the current
# build only if the hash of its kernel's sources matches.
_COMMON = ["fa_device.h", "fa_params.h"]
KERNEL_SOURCES = {
    "prefill_bf16_pp_kernel": ["fa_prefill_pp.hip", "fa_softmax.h"] + _COMMON,
    "prefill_bf16_kernel": ["fa_prefill_bf16.hip", "fa_softmax.h"] + _COMMON,
    "decode_split_kernel": ["fa_decode.hip"] + _COMMON,
    "prefill_fp8_kernel": ["fa_prefill_fp8.hip"] + _COMMON,
    "bwd_dq_kernel": ["fa_backward.hip"] + _COMMON,
    "bwd_dkdv_kernel": ["fa_backward.hip"] + _COMMON,
}
PREFILL_WORKLOADS = ["gpt2s_causal_b8_h12_n1024_d64", "bertl_padded_b16_h16_n512_d64",
                     "long_causal_b2_h16_n16384_d128"]
LONG_NQ = 2048  # fa_fwd runs prefill_bf16_pp_kernel from this many query rows on


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "io_aware_exact_23_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, workload: str, sha: str):
    """HBM bytes per launch from a committed counter summary, if taken on the current source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}__hbm_counters.txt")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("RESULT "):
                rec = json.loads(line[len("RESULT "):])
    if not rec or rec.get("source_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def time_launches(fn, steps: int, warmup: int, torch):
    """Run fn warmup times, then time `steps` calls with HIP events on the current stream.

    Returns (total seconds over the timed region, list of per-launch seconds).
    """
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total = t_start.elapsed_time(t_end) / 1e3
    per = [s.elapsed_time(e) / 1e3 for s, e in zip(starts, ends)]
    return total, per


def host_identity() -> dict:
    """The host CPU the oracle baseline runs on: model name, logical cores, cores this process may
    use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "logical_cores": os.cpu_count(), "usable_cores": usable}


def run_identity(torch) -> dict:
    """GPU, software versions and host of this run, so that every figure traces to one record."""
    import ctypes

    props = torch.cuda.get_device_properties(0)
    ident = {"gpu": props.name, "arch": getattr(props, "gcnArchName", None),
             "compute_units": props.multi_processor_count, "hbm_bytes": props.total_memory,
             "torch": torch.__version__, "torch_hip": torch.version.hip}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        # hipDeviceAttributeClockRate (= 5 in hip_runtime_api.h): peak engine clock in kHz.
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, torch.cuda.current_device()) == 0:
            ident["peak_sclk_mhz"] = val.value / 1000.0
    except OSError:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            ident["rocm"] = f.read().strip()
    except OSError:
        ident["rocm"] = None
    try:
        import io_aware_exact_23_amd as fa
        ident["library_build"] = fa.fa_build_info()
    except (OSError, AttributeError):
        ident["library_build"] = None
    ident["host"] = host_identity()
    return ident


# O and lse tolerances of the bf16 path against the fp64 oracle (max-abs, mean-abs, lse max-abs).
BF16_TOL = (2e-2, 2e-3, 1e-3)
FP32_TOL = (1e-5, 1e-5, 1e-3)


def cpu_baseline_prefill(w, q, k, v, o, lse, seconds: float):
    """The oracle, untuned, on a bounded sample of the workload; its rows are also compared with the
    GPU output of the timed run (o, lse), so the rate comes with the error on the same rows.

    Heads are taken in order (b, h) = (0, 0), (0, 1), ...; each head's query rows are visited in
    16 interleaved passes (rows r, r+16, r+32, ...), so every pass has the same mix of causal
    row lengths. Sampling stops after the first pass that ends past `seconds`. Only the oracle
    calls are timed.
    """
    import threadpoolctl
    from oracle import attention_fwd

    stride = 16
    flops = 0
    rows_done = 0
    heads = []
    t_oracle = 0.0
    err_max = err_sum = lse_max = 0.0
    n_elem = 0
    done = False
    for b in range(w.B):
        for h in range(w.H):
            qh = q[b:b + 1, h:h + 1].float().cpu().double().numpy()
            kh = k[b:b + 1, h:h + 1].float().cpu().double().numpy()
            vh = v[b:b + 1, h:h + 1].float().cpu().double().numpy()
            og = o[b, h].float().cpu().double().numpy()
            lg = lse[b, h].cpu().double().numpy()
            heads.append((b, h))
            for start in range(stride):
                rows = np.arange(start, w.Nq, stride)
                t0 = time.perf_counter()
                o_ref, lse_ref = attention_fwd(qh, kh, vh, w.scale, causal=w.causal, rows=rows)
                t_oracle += time.perf_counter() - t0
                e = np.abs(og[rows] - o_ref[0, 0])
                err_max = max(err_max, float(e.max()))
                err_sum += float(e.sum())
                n_elem += e.size
                fin = np.isfinite(lse_ref[0, 0])
                if fin.any():
                    lse_max = max(lse_max, float(np.abs(lg[rows][fin] - lse_ref[0, 0][fin]).max()))
                # Same counting convention as the GPU: 4*d per (query, allowed key) pair.
                n_keys = (rows + 1) if w.causal else np.full(len(rows), w.Nk)
                flops += int(4 * w.d * n_keys.sum())
                rows_done += len(rows)
                if t_oracle >= seconds:
                    done = True
                    break
            if done:
                break
        if done:
            break
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    host = host_identity()
    base = {"value": flops / t_oracle / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "blas_threads": threads, "host_logical_cores": host["logical_cores"],
            "host_usable_cores": host["usable_cores"], "host_cpu_model": host["cpu_model"],
            "sample": f"{rows_done} of {w.B * w.H * w.Nq} query rows ({len(heads)} heads, from (b, h) = (0, 0) "
                      f"in order, each head's rows in 16 interleaved passes) of {w.name}: fp64 numpy with "
                      f"{threads} BLAS threads, {t_oracle:.1f} s of oracle time; the value is the rate over this "
                      f"sample, FLOPs counted as 4*d per (query row, allowed key)"}
    mx, mn, lt = BF16_TOL if w.dtype == "bf16" else FP32_TOL
    parity = {"rows_compared": rows_done, "heads": len(heads), "o_max_abs": err_max,
              "o_mean_abs": err_sum / max(n_elem, 1), "lse_max_abs": lse_max,
              "tolerance": {"o_max_abs": mx, "o_mean_abs": mn, "lse_max_abs": lt},
              "what": "GPU output of the last timed step against the fp64 oracle on the cpu_baseline rows"}
    parity["within_tolerance"] = bool(err_max <= mx and parity["o_mean_abs"] <= mn and lse_max <= lt)
    return base, parity


def allowed_scores(w, lens) -> int:
    """Number of (query, key) pairs the mask allows, over all (b, h)."""
    L = np.full(w.B, w.Nk, dtype=np.int64) if lens is None else np.clip(np.asarray(lens, dtype=np.int64), 0, w.Nk)
    i = np.arange(w.Nq, dtype=np.int64)
    per_b = np.array([np.minimum(Lb, i + 1).sum() if w.causal else w.Nq * Lb for Lb in L], dtype=np.int64)
    return int(per_b.sum()) * w.H


def standard_bytes(w, lens) -> int:
    """Algorithmic HBM bytes of the standard algorithm as fa_std_fwd runs it: write S (fp32, full
    Nq x Nk grid), read the allowed part of S, write P (bf16, rows of ld entries), read P, plus
    Q, the valid K and V rows, O and lse."""
    ld = (w.Nk + 127) // 128 * 128
    bh = w.B * w.H
    L = np.full(w.B, w.Nk) if lens is None else np.clip(np.asarray(lens), 0, w.Nk)
    qo = 2 * bh * w.Nq * w.d * 2 + bh * w.Nq * 4
    kv = 2 * int(L.sum()) * w.H * w.d * 2
    return int(qo + kv + bh * w.Nq * w.Nk * 4 + allowed_scores(w, lens) * 4 + 2 * bh * w.Nq * ld * 2)


def bench_standard(fa, configs, inputs, torch, dev, steps, warmup, main_name):
    """Standard algorithm against the tiled path on the prefill workloads."""
    out = {"unit": "ms", "workloads": []}
    for name in PREFILL_WORKLOADS:
        w = configs.BY_NAME[name]
        q, k, v, lens = inputs.make(w, dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        need = fa.fa_std_workspace_bytes(w.B, w.H, w.Nq, w.Nk)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)

        def tiled():
            fa.fa_fwd(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal), lens, None)

        def standard():
            fa.fa_std_fwd(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal), lens,
                          ws, need, None)

        n = steps if w.Nq <= LONG_NQ else max(3, steps // 4)
        t_tiled, _ = time_launches(tiled, n, warmup, torch)
        t_std, per_std = time_launches(standard, n, warmup, torch)
        t_rot = None
        if w.Nq <= LONG_NQ:
            # The short workloads' inputs and outputs fit in the 256 MB Infinity Cache. Also time
            # the tiled call cycling through copies of them whose total exceeds it, so the figure
            # does not rest on a warm cache.
            per_set = sum(t.numel() * t.element_size() for t in (q, k, v, o, lse))
            n_sets = max(2, -(-(320 << 20) // per_set))
            sets = [(q.clone(), k.clone(), v.clone(), torch.empty_like(o), torch.empty_like(lse))
                    for _ in range(n_sets)]
            it = [0]

            def tiled_rotated():
                qs, ks, vs, os_, ls = sets[it[0] % n_sets]
                it[0] += 1
                fa.fa_fwd(qs, ks, vs, os_, ls, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal), lens, None)

            t_rot, _ = time_launches(tiled_rotated, n, warmup, torch)
            del sets
        lens_np = None if lens is None else lens.cpu().numpy()
        nbytes = standard_bytes(w, lens_np)
        avg = float(np.mean(per_std))
        # Forward rate of the tiled call: FLOPs counted as 4*B*H*Nq*Nk*d (halved when causal), and
        # also over the pairs the mask allows (4*d per pair) where key lengths apply.
        fl_tiled = w.counted_flops() / (t_tiled / n)
        rec = {"workload": name, "tiled_ms": round(t_tiled / n * 1e3, 4), "standard_ms": round(t_std / n * 1e3, 4),
               "tiled_TFLOPs": round(fl_tiled / 1e12, 1),
               "tiled_frac_of_peak": round(fl_tiled / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
               "speedup": round(t_std / t_tiled, 2), "workspace_bytes": need,
               "standard_algorithmic_bytes": nbytes,
               "standard_hbm_GBps": round(nbytes / avg / 1e9, 1)}
        if lens_np is not None:
            rec["tiled_TFLOPs_allowed_pairs"] = round(4 * w.d * allowed_scores(w, lens_np) / (t_tiled / n) / 1e12, 1)
        if t_rot is not None:
            rec["tiled_ms_rotated_inputs"] = round(t_rot / n * 1e3, 4)
            rec["speedup_rotated_inputs"] = round(t_std / t_rot, 2)
        if name == main_name:
            rec["roofline"] = {"kernel": "std_scores_kernel + std_softmax_kernel + std_pv_kernel (whole call)",
                               "bound": "hbm", "achieved": round(nbytes / avg / 1e9, 1), "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": round(nbytes / avg / 1e9 / PEAK_HBM_GBS, 4),
                               "avg_launch_ms": round(avg * 1e3, 4)}
        out["workloads"].append(rec)
        del ws, q, k, v, o, lse
        torch.cuda.empty_cache()
    return out


def bench_masks(fa, configs, inputs, torch, dev, steps, warmup):
    """Sliding window and packed sequences on the 16K causal shape."""
    w = configs.LONG_CAUSAL_16K
    q, k, v, _ = inputs.make(w, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    out = {"workload": w.name, "unit": "TFLOP/s", "peak": PEAK_MFMA_BF16_TFLOPS}
    W = 4096
    pairs = int(np.minimum(np.arange(1, w.Nq + 1), W).sum())
    flops = 4 * w.B * w.H * pairs * w.d

    def win():
        fa.fa_fwd_window(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, W - 1, 0, None, None)

    t, per = time_launches(win, steps, warmup, torch)
    avg = float(np.mean(per))
    out["sliding_window"] = {"window": [W - 1, 0], "ms_per_step": round(t / steps * 1e3, 4),
                             "allowed_pairs_per_head": pairs, "counted_flops": flops,
                             "value": round(flops * steps / t / 1e12, 2),
                             "frac": round(flops / avg / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4)}
    H, T = w.H, w.B * w.Nq
    qp = q.permute(1, 0, 2, 3).reshape(H, T, w.d).contiguous()
    kp = k.permute(1, 0, 2, 3).reshape(H, T, w.d).contiguous()
    vp = v.permute(1, 0, 2, 3).reshape(H, T, w.d).contiguous()
    del q, k, v, o
    op = torch.empty_like(qp)
    lp = torch.empty((H, T), dtype=torch.float32, device=dev)
    cu = torch.arange(0, T + 1, w.Nq, dtype=torch.int32, device=dev)

    def packed():
        fa.fa_fwd_varlen(qp, kp, vp, op, lp, w.B, H, T, T, w.Nq, w.d, w.scale, -1, 0, cu, cu, None)

    t, per = time_launches(packed, steps, warmup, torch)
    avg = float(np.mean(per))
    fl = w.counted_flops()
    out["packed_causal"] = {"sequences": w.B, "layout": "[H][T][d]", "ms_per_step": round(t / steps * 1e3, 4),
                            "counted_flops": fl, "value": round(fl * steps / t / 1e12, 2),
                            "frac": round(fl / avg / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4)}
    return out


def bench_backward(fa, configs, inputs, torch, dev, steps, warmup):
    """fa_bwd (dQ, dK, dV from the saved lse) on the 16K causal and GPT-2 shapes.

    FLOPs are counted as the five matrix products of the gradient (S, dP, dV, dK, dQ), 2.5 times
    the forward count; the kernels compute seven (the dQ kernel recomputes S and dP).
    """
    out = {"unit": "TFLOP/s", "peak": PEAK_MFMA_BF16_TFLOPS, "counted_products": 5, "workloads": []}
    for name in ["long_causal_b2_h16_n16384_d128", "gpt2s_causal_b8_h12_n1024_d64"]:
        w = configs.BY_NAME[name]
        q, k, v, lens = inputs.make(w, dev)
        do = inputs.normal((w.B, w.H, w.Nq, w.d), w.seed + 7, dev, "bf16", 1.0)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        fa.fa_fwd(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal), lens, None)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

        def bstep():
            fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal),
                      lens, None)

        n = steps if w.Nq <= LONG_NQ else max(3, steps // 4)
        t, per = time_launches(bstep, n, warmup, torch)
        avg = float(np.mean(per))
        fl = int(2.5 * w.counted_flops())
        rec = {"workload": name, "ms_per_step": round(t / n * 1e3, 4), "counted_flops": fl,
               "value": round(fl * n / t / 1e12, 2)}
        if name == configs.LONG_CAUSAL_16K.name:
            rec["roofline"] = {"kernel": "bwd_delta_kernel + bwd_dq_kernel + bwd_dkdv_kernel (whole call)",
                               "bound": "mfma", "achieved": round(fl / avg / 1e12, 2),
                               "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(fl / avg / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
                               "avg_launch_ms": round(avg * 1e3, 4)}
        out["workloads"].append(rec)
        del q, k, v, do, o, dq, dk, dv
        torch.cuda.empty_cache()
    return out


def bench_fp8(fa, configs, inputs, torch, dev, steps, warmup):
    """e4m3 forward on the 16K causal shape: conversion cost, forward rate, error against bf16.

    The inputs are the bf16 workload, quantised on the GPU (fa_quantize_fp8: Q and K per row, V
    transposed). The forward is timed on codes already resident in HBM; the conversion is timed
    separately (algorithmic bytes: read bf16 once, write e4m3 once, 3 bytes per element).
    """
    w = configs.LONG_CAUSAL_16K
    q, k, v, lens = inputs.make(w, dev)
    o16 = torch.empty_like(q)
    lse16 = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    fa.fa_fwd(q, k, v, o16, lse16, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal), lens, None)
    q8, sq = fa.quantize_fp8(q)
    k8, sk = fa.quantize_fp8(k, kv_seqlens=lens)
    vt8, sv = fa.quantize_fp8(v, kv_seqlens=lens, transpose=True)

    def quant():
        fa.fa_quantize_fp8(q, q8, sq, w.B, w.H, w.Nq, w.d, None, 0, None)
        fa.fa_quantize_fp8(k, k8, sk, w.B, w.H, w.Nk, w.d, lens, 0, None)
        fa.fa_quantize_fp8(v, vt8, sv, w.B, w.H, w.Nk, w.d, lens, 1, None)

    nq = max(3, steps // 2)
    tq, _ = time_launches(quant, nq, warmup, torch)
    o8 = torch.empty_like(q)
    lse8 = torch.empty_like(lse16)

    def fstep():
        fa.fa_fwd_fp8(q8, k8, vt8, sq, sk, sv, o8, lse8, w.B, w.H, w.Nq, w.Nk, w.d, w.scale,
                      int(w.causal), lens, None)

    t, per = time_launches(fstep, steps, warmup, torch)
    avg = float(np.mean(per))
    fl = w.counted_flops()
    elems = 3 * w.B * w.H * w.Nq * w.d
    diff = (o8.float() - o16.float())
    rel = float(torch.linalg.vector_norm(diff) / torch.linalg.vector_norm(o16.float()))
    out = {"workload": w.name, "unit": "TFLOP/s", "ms_per_step": round(t / steps * 1e3, 4),
           "value": round(fl * steps / t / 1e12, 2), "counted_flops": fl,
           "speedup_vs_bf16_forward": None,
           "roofline": {"kernel": "prefill_fp8_kernel", "bound": "mfma", "achieved": round(fl / avg / 1e12, 2),
                        "peak": PEAK_MFMA_FP8_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(fl / avg / 1e12 / PEAK_MFMA_FP8_TFLOPS, 4),
                        "avg_launch_ms": round(avg * 1e3, 4),
                        "traffic": traffic_from_profile("prefill_fp8_kernel", w.name,
                                                        source_sha("prefill_fp8_kernel"))},
           "conversion": {"kernels": "quant_amax_kernel + quant_rows_kernel / quant_transpose_kernel",
                          "ms_per_call_qkv": round(tq / nq * 1e3, 4),
                          "algorithmic_bytes": 3 * elems,
                          "GBps": round(3 * elems * nq / tq / 1e9, 1)},
           "error_vs_bf16_path": {"o_rel_frobenius": round(rel, 5),
                                  "o_max_abs": round(float(diff.abs().max()), 5),
                                  "lse_max_abs": round(float((lse8 - lse16).abs().max()), 5)}}
    del q, k, v, q8, k8, vt8, o8, o16
    torch.cuda.empty_cache()
    return out


def graph_time_per_launch(fn, launches: int, replays: int, warmup: int, torch) -> float:
    """Seconds per launch of fn, measured with HIP events around replays of a HIP graph holding
    `launches` back-to-back calls: the device-side time of the kernels with no host launch gaps,
    which otherwise dominate launches of a few tens of microseconds. fn must launch kernels only
    (no allocation, no memset)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(warmup, 1)):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / 1e3 / (launches * replays)


def bench_short_prefill(fa, configs, inputs, torch, dev, warmup):
    """The short prefill workloads (GPT-2 and BERT shapes, prefill_bf16_kernel) timed per launch
    without host gaps (graph replay), each with its MFMA roofline object."""
    out = []
    for name in PREFILL_WORKLOADS[:2]:
        w = configs.BY_NAME[name]
        q, k, v, lens = inputs.make(w, dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)

        def run():
            fa.fa_fwd(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal), lens, None)

        per = graph_time_per_launch(run, 50, 10, warmup, torch)
        fl = w.counted_flops()
        rec = {"workload": name, "kernel_ms": round(per * 1e3, 5), "counted_flops": fl,
               "roofline": {"kernel": "prefill_bf16_kernel", "bound": "mfma",
                            "achieved": round(fl / per / 1e12, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(fl / per / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
                            "avg_launch_ms": round(per * 1e3, 5),
                            "timing": "HIP events around 10 replays of a graph of 50 launches",
                            "traffic": traffic_from_profile("prefill_bf16_kernel", name,
                                                            source_sha("prefill_bf16_kernel")),
                            "source_sha": source_sha("prefill_bf16_kernel")}}
        if lens is not None:
            pairs = allowed_scores(w, lens.cpu().numpy())
            rec["allowed_pair_flops"] = 4 * w.d * pairs
            rec["TFLOPs_allowed_pairs"] = round(4 * w.d * pairs / per / 1e12, 1)
        out.append(rec)
        del q, k, v, o, lse
    return out


def bench_gemm_reference(torch, dev, warmup):
    """Context for the matrix-core fractions: plain dense bf16 GEMMs (torch.matmul, the vendor
    library) on random N(0,1) square operands, timed like the kernels. It is what a tuned library
    sustains on the same box and data, not part of the attention path."""
    out = {"what": "torch.matmul bf16 on random N(0,1) square operands [n, n] x [n, n]", "shapes": []}
    for n in (8192, 16384):
        a = torch.randn((n, n), device=dev, dtype=torch.float32).to(torch.bfloat16).contiguous()
        b = torch.randn((n, n), device=dev, dtype=torch.float32).to(torch.bfloat16).contiguous()
        c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)

        def run():
            torch.matmul(a, b, out=c)

        _, per = time_launches(run, 10, max(warmup, 3), torch)
        avg = float(np.mean(per))
        fl = 2 * n ** 3
        out["shapes"].append({"n": n, "ms_per_call": round(avg * 1e3, 4), "TFLOP/s": round(fl / avg / 1e12, 1),
                              "frac_of_peak": round(fl / avg / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4)})
        del a, b, c
        torch.cuda.empty_cache()
    return out


def decode_bytes(w, lens) -> int:
    per_key = 2 * w.d * 2                      # one K row and one V row, bf16
    per_bh = 2 * w.d * 2 + 4                   # Q and O rows (bf16) and lse (fp32)
    return int(w.H * (per_key * int(lens.sum()) + per_bh * w.B))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_causal_b2_h16_n16384_d128")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-standard", action="store_true",
                    help="skip the standard-algorithm comparison (fa_std_fwd)")
    ap.add_argument("--no-masks", action="store_true",
                    help="skip the sliding-window and packed-sequence timings")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass timing (fa_bwd)")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the dense bf16 GEMM reference (torch.matmul) reported for context")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the e4m3 forward timing (fa_quantize_fp8, fa_fwd_fp8)")
    ap.add_argument("--no-short", action="store_true",
                    help="skip the graph-replayed timing of the short prefill workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported. Attention over "
              "(batch, head) shards with no communication: each GPU would run fa_fwd on its own "
              "batches or heads.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    import io_aware_exact_23_amd as fa
    from io_aware_exact_23_amd import configs, inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    fa.load_library()
    dev = "cuda"
    w = configs.BY_NAME[args.workload]
    q, k, v, lens = inputs.make(w, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    fn_c = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_f32

    def step():
        fn_c(q, k, v, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.scale, int(w.causal), lens, None)

    total, per = time_launches(step, args.steps, args.warmup, torch)
    flops = w.counted_flops()
    value = flops * args.steps / total / 1e12
    avg_launch = float(np.mean(per))
    achieved = flops / avg_launch / 1e12
    if w.dtype == "fp32":
        kernel, peak = "prefill_f32_kernel", PEAK_MFMA_FP32_TFLOPS
    elif w.Nq == 1:
        kernel, peak = "decode_split_kernel", PEAK_MFMA_BF16_TFLOPS
    else:
        kernel = "prefill_bf16_pp_kernel" if w.Nq >= LONG_NQ else "prefill_bf16_kernel"
        peak = PEAK_MFMA_BF16_TFLOPS
    sha = source_sha(kernel) if kernel in KERNEL_SOURCES else None
    if w.Nq == 1 and w.dtype == "bf16":
        # A decode main workload is bound by HBM: its roofline is bytes, not FLOPs.
        nbytes = decode_bytes(w, (lens.cpu().numpy() if lens is not None else np.full(w.B, w.Nk)))
        roof = {"kernel": "decode_split_kernel + decode_combine_kernel (whole call)", "bound": "hbm",
                "achieved": round(nbytes / avg_launch / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(nbytes / avg_launch / 1e9 / PEAK_HBM_GBS, 4),
                "avg_launch_ms": round(avg_launch * 1e3, 4),
                "traffic": traffic_from_profile(kernel, w.name, sha), "source_sha": sha}
    else:
        roof = {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "avg_launch_ms": round(avg_launch * 1e3, 4),
                "traffic": traffic_from_profile(kernel, w.name, sha) if sha else None, "source_sha": sha}
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "input_std": w.input_std, "seed": w.seed,
                   "counted_flops": flops},
        "pct_mfma_peak": round(100.0 * value / peak, 2),
        "roofline": roof,
        "run": run_identity(torch),
    }

    if not args.no_decode:
        wd = configs.DECODE_SPLIT_KV
        dq, dk, dv, dl = inputs.make(wd, dev)
        do = torch.empty_like(dq)
        dlse = torch.empty((wd.B, wd.H, 1), dtype=torch.float32, device=dev)

        def dstep():
            fa.fa_fwd(dq, dk, dv, do, dlse, wd.B, wd.H, 1, wd.Nk, wd.d, wd.scale, 0, dl, None)

        dtotal, dper = time_launches(dstep, args.steps, args.warmup, torch)
        nbytes = decode_bytes(wd, dl.cpu().numpy())
        davg = float(np.mean(dper))
        result["decode"] = {
            "workload": wd.name, "unit": "GB/s",
            "value": round(nbytes * args.steps / dtotal / 1e9, 1),
            "ms_per_step": round(dtotal / args.steps * 1e3, 4),
            "algorithmic_bytes": nbytes,
            "pct_hbm_peak": round(100.0 * nbytes / davg / 1e9 / PEAK_HBM_GBS, 2),
            "roofline": {"kernel": "decode_split_kernel + decode_combine_kernel (whole call)",
                         "bound": "hbm", "achieved": round(nbytes / davg / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(nbytes / davg / 1e9 / PEAK_HBM_GBS, 4),
                         "avg_launch_ms": round(davg * 1e3, 4),
                         "traffic": traffic_from_profile("decode_split_kernel", wd.name,
                                                         source_sha("decode_split_kernel"))},
        }
        del dq, dk, dv, do

    if not args.no_short:
        result["short_prefill"] = bench_short_prefill(fa, configs, inputs, torch, dev, args.warmup)

    if not args.no_masks:
        result["masks"] = bench_masks(fa, configs, inputs, torch, dev, args.steps, args.warmup)

    if not args.no_fp8:
        result["fp8"] = bench_fp8(fa, configs, inputs, torch, dev, args.steps, args.warmup)
        if w.name == configs.LONG_CAUSAL_16K.name:
            result["fp8"]["speedup_vs_bf16_forward"] = round(result["ms_per_step"] / result["fp8"]["ms_per_step"], 3)

    if not args.no_backward:
        result["backward"] = bench_backward(fa, configs, inputs, torch, dev, args.steps, args.warmup)

    if not args.no_standard and w.Nq > 1 and w.dtype == "bf16":
        result["standard_attention"] = bench_standard(fa, configs, inputs, torch, dev, args.steps,
                                                      args.warmup, w.name)

    if not args.no_gemm_reference:
        result["gemm_reference"] = bench_gemm_reference(torch, dev, args.warmup)

    if args.calibrate_copy:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)  # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = src.numel() * 2

    if not args.no_cpu_baseline and w.Nq > 1:
        result["cpu_baseline"], result["parity"] = cpu_baseline_prefill(w, q, k, v, o, lse, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
