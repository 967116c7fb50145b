#!/usr/bin/env python3
"""Benchmark of the packed variable-length attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense_77k]
    python bench.py --backward [--workload bwd_9728]

A step is one call of attn_varlen_fwd through the C ABI with cu_seqlens on the
device: the cu read-back, the exact tile plan and the kernel launch. Inputs are
resident in HBM before timing starts. Prints ONE JSON line on stdout:
TFLOP/s with FLOPs = sum over segments of 4*Lq*Lk*D*H, the kernel's roofline
figures (its own average duration from HIP events on the launch stream), and
the CPU oracle's throughput on a bounded sample of the same workload.

With --backward a step is one attn_varlen_bwd call (device cu_seqlens): the
preprocessing pass, the dK/dV kernel and the dQ kernel, on the dout layout of
the _bwd_preprocess page (row stride 9728). FLOPs follow the flash-attention
convention for the backward, 10*Lq*Lk*D*H per segment (five matrix products
of the forward's size; the kernels form S and dP twice, so they execute 14).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
# 8-bit score product + bf16 P.V: half the FLOPs at each rate, time-weighted
PEAK_FP8_QK_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
KERNEL_SOURCES = ["varlen_flashattention_forward_amd/csrc/avf_kernel.hip",
                  "varlen_flashattention_forward_amd/csrc/avf_plan.h",
                  "varlen_flashattention_forward_amd/csrc/avf_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """Hash of the forward kernel's code: its sources with // comments and
    blank lines removed, so a comment edit keeps the committed counters."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        for line in (ROOT / p).read_text().splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def roofline_of(flops: int, nbytes: int, kernel_ms: float, peak_tflops: float) -> dict:
    """Roofline figures of one launch: bound by MFMA when its arithmetic
    intensity is at or above the ridge (peak FLOP/s over peak HBM bytes/s),
    reported as TFLOP/s against `peak_tflops`; bound by HBM below it, reported
    as algorithmic GB/s against the HBM peak."""
    if flops / nbytes >= peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = flops / (kernel_ms / 1e3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak_tflops, 1), "unit": "TFLOP/s",
                "frac": round(achieved / peak_tflops, 4)}
    gbs = nbytes / (kernel_ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def traffic_for(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    f = ROOT / "profiles" / f"traffic_avf_fwd_{workload}.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text())
    if d.get("kernel_hash") != kernel_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, t, rows_per_segment: int):
    import numpy as np

    import oracle
    from varlen_flashattention_forward_amd.workloads import sample_rows

    rows = sample_rows(w, rows_per_segment, edge=min(8, rows_per_segment // 2))
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    threads = oracle.default_threads()
    flops = sum(4 * w.visible_keys(r) * w.head_dim * w.num_heads for r in rows)
    t0 = time.perf_counter()
    oracle.attn_varlen_fwd(q, k, v, w.cu_q, w.cu_k, float(np.float32(w.softmax_scale)), rows=rows,
                           threads=threads, causal=w.causal)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} query rows x {w.num_heads} heads of {w.name} against their "
                      f"{'visible ' if w.causal else ''}segments (C fp64 oracle, {dt:.1f} s, {flops / 1e9:.1f} GFLOP)"}


def cpu_baseline_fp8(w, t, rows_per_segment: int, heads: int = 4):
    """The fp8 oracle on sampled rows of the first `heads` heads (its scales
    are per head, so those heads quantize on their own)."""
    import numpy as np

    from oracle import fp8_oracle
    from varlen_flashattention_forward_amd.workloads import sample_rows

    rows = sample_rows(w, rows_per_segment, edge=min(8, rows_per_segment // 2))
    hs = list(range(min(heads, w.num_heads)))
    q, k, v = (t[n][:, hs].contiguous().cpu() for n in ("q", "k", "v"))
    flops = sum(4 * w.visible_keys(r) * w.head_dim * len(hs) for r in rows)
    t0 = time.perf_counter()
    fp8_oracle.attn_varlen_fwd_fp8(q, k, v, w.cu_q, w.cu_k, float(np.float32(w.softmax_scale)), rows=rows,
                                   causal=w.causal)
    dt = time.perf_counter() - t0
    import oracle
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.default_threads(), "kind": "oracle",
            "sample": f"{len(rows)} query rows x {len(hs)} heads of {w.name} with those heads' E4M3 "
                      f"quantization (numpy fp64 oracle, {dt:.1f} s, {flops / 1e9:.1f} GFLOP)"}


def cpu_baseline_bwd(w, t, dout, rows_per_segment: int):
    import numpy as np

    import oracle
    from varlen_flashattention_forward_amd.workloads import sample_rows

    rows = sample_rows(w, rows_per_segment, edge=min(4, rows_per_segment // 2))
    q, k, v = (t[n].contiguous().cpu() for n in ("q", "k", "v"))
    g = dout.contiguous().cpu()
    threads = oracle.default_threads()
    # a dq row forms S, dP and dQ against its segment's keys: 3 of the 5 products
    flops = sum(6 * w.visible_keys(r) * w.head_dim * w.num_heads for r in rows)
    t0 = time.perf_counter()
    oracle.attn_varlen_bwd_dq_rows(q, k, v, g, w.cu_q, w.cu_k, float(np.float32(w.softmax_scale)), rows,
                                   causal=w.causal, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"dq of {len(rows)} query rows x {w.num_heads} heads of {w.name} against their "
                      f"segments (C fp64 oracle, {dt:.1f} s, {flops / 1e9:.1f} GFLOP counted as 6*Lk*D*H "
                      f"per row: S, dP and dQ)"}


def bench_backward(args) -> int:
    import torch

    import varlen_flashattention_forward_amd as avf
    from varlen_flashattention_forward_amd.workloads import WORKLOADS, make_dout, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    avf.lib()
    log(f"[bench-bwd] workload {w.name}: H={w.num_heads} D={w.head_dim} segments={w.num_segments} "
        f"total_q={w.total_q} dout row stride {w.outer_stride or 'contiguous'}")
    t = make_inputs(w, dev, seed=0)
    dout, _ = make_dout(w, dev, seed=1, outer_stride=w.outer_stride)
    out, lse = avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                   softmax_scale=w.softmax_scale, out=t["out"], lse=t["lse"], causal=w.causal)
    dq = torch.empty_like(t["q"], memory_format=torch.contiguous_format)
    dk = torch.empty_like(t["k"], memory_format=torch.contiguous_format)
    dv = torch.empty_like(t["v"], memory_format=torch.contiguous_format)
    delta = torch.empty((w.num_heads, w.total_q), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    flops = w.flops() // 4 * 10
    stream = torch.cuda.current_stream(dev)

    def step(**kw):
        avf.attn_varlen_bwd(t["q"], t["k"], t["v"], out, dout, lse, t["cu_q"], t["cu_k"], w.max_seqlen_q,
                            w.max_seqlen_k, softmax_scale=w.softmax_scale, causal=w.causal, dq=dq, dk=dk, dv=dv,
                            delta=delta, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench-bwd] warmup done ({args.warmup} steps)")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    value = flops / (ms / 1e3) / 1e12
    log(f"[bench-bwd] {args.steps} steps: {ms:.3f} ms/step, {value:.1f} TFLOP/s")

    # the pass's kernels alone: HIP events on the launch stream around the
    # synchronisation-free entry point (three kernels back to back)
    cu_q, cu_k = list(w.cu_q), list(w.cu_k)
    durs = []
    for _ in range(args.steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(cu_seqlens_q_host=cu_q, cu_seqlens_k_host=cu_k, stream=stream.cuda_stream)
        e1.record(stream)
        durs.append((e0, e1))
    torch.cuda.synchronize()
    kms = sum(a.elapsed_time(b) for a, b in durs) / len(durs)
    pre_wg, dkdv_wg, dq_wg, launches = avf.bwd_grid_plan(w.cu_q, w.cu_k, w.num_heads, w.head_dim)
    achieved = flops / (kms / 1e3) / 1e12
    log(f"[bench-bwd] kernels: {kms:.3f} ms/call, {achieved:.1f} TFLOP/s; workgroups pre {pre_wg} "
        f"dkdv {dkdv_wg} dq {dq_wg}")
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "kernel": "backward pass: avf_bwd_pre_kernel + avf_bwd_dkdv_kernel + avf_bwd_dq_kernel",
                "kernel_ms": round(kms, 4), "algorithmic_flops_per_launch": flops,
                "executed_mfma_flops_per_launch": flops // 10 * 14}
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench-bwd] CPU oracle baseline ...")
        cpu = cpu_baseline_bwd(w, t, dout, args.cpu_rows_bwd)
        log(f"[bench-bwd] cpu baseline {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")
    rec = {
        "metric": "attention bwd TFLOP/s (10*Sq*Sk*D*H) and % of MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": w.name, "pass": "backward", "num_heads": w.num_heads, "head_dim": w.head_dim,
                   "segments": w.num_segments, "total_q": w.total_q, "total_k": w.total_k,
                   "dout_row_stride": dout.stride(0), "causal": w.causal, "flops_per_step": flops,
                   "workgroups": {"preprocess": pre_wg, "dkdv": dkdv_wg, "dq": dq_wg}},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


# Operand patterns of the MFMA-rate stream. Each wave's operands are 8
# fragments of 512 bf16 values (64 lanes x 8): fragments 0-3 are the A
# operands, 4-7 the B operands.
MFMA_OPERANDS = {
    "random": "N(0,1) random bf16",
    "ones": "all ones",
    "uniform": "uniform [0, 1) random bf16",
    "lane-constant": "N(0,1) random, one value per fragment (the same in every lane and element)",
    "a-random-b-ones": "A N(0,1) random, B all ones",
    "a-ones-b-random": "A all ones, B N(0,1) random",
}


def mfma_operands(mode: str, n: int, dev, g):
    import torch

    if mode == "ones":
        return torch.ones(n, dtype=torch.bfloat16, device=dev)
    if mode == "uniform":
        return torch.rand(n, device=dev, generator=g).to(torch.bfloat16)
    x = torch.randn(n, dtype=torch.bfloat16, device=dev, generator=g).view(-1, 8, 512)
    if mode == "lane-constant":
        x = x[:, :, :1].expand(-1, -1, 512)
    elif mode == "a-random-b-ones":
        x[:, 4:, :] = 1.0
    elif mode == "a-ones-b-random":
        x[:, :4, :] = 1.0
    return x.contiguous().view(-1)


def bench_mfma_rate(args, dev) -> int:
    """The rate a plain bf16 MFMA stream reaches on this GPU with the given
    operand values (the calibration kernel of libavf_probe.so): under the
    board's power limit the clock, and so the rate, depends on the operands'
    switching activity. Random N(0,1) bf16 operands, like the attention
    workloads' inputs, give the ceiling an MFMA-bound kernel on such data can
    approach; all-ones operands show the clock with little switching."""
    import ctypes

    import torch

    from varlen_flashattention_forward_amd import build as avf_build

    if not avf_build.PROBE_LIB.exists():
        raise RuntimeError(f"{avf_build.PROBE_LIB} is missing: build with python -m varlen_flashattention_forward_amd.build")
    P = ctypes.CDLL(str(avf_build.PROBE_LIB))
    P.avf_probe_operand_bytes.restype = ctypes.c_int64
    P.avf_probe_operand_bytes.argtypes = [ctypes.c_int32]
    P.avf_probe_output_bytes.restype = ctypes.c_int64
    P.avf_probe_output_bytes.argtypes = [ctypes.c_int32]
    P.avf_probe_mfma.restype = ctypes.c_int32
    P.avf_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wgs = 2 * cus            # 256-thread workgroups, two per CU: two waves per SIMD
    iters = 400000           # about 0.1 s per launch
    n = P.avf_probe_operand_bytes(wgs) // 2
    g = torch.Generator(device=dev).manual_seed(0)
    ops = mfma_operands(args.mfma_rate, n, dev, g)
    out = torch.empty(P.avf_probe_output_bytes(wgs) // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch():
        rc = P.avf_probe_mfma(ops.data_ptr(), out.data_ptr(), wgs, iters, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"avf_probe_mfma returned {rc}")

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = wgs * 4 * iters * 8 * 32768
    tf = flops / (ms / 1e3) / 1e12
    print(json.dumps({"metric": "bf16 MFMA rate of a plain v_mfma_f32_32x32x16_bf16 stream", "value": round(tf, 1),
                      "unit": "TFLOP/s", "operands": MFMA_OPERANDS[args.mfma_rate],
                      "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "peak": PEAK_BF16_TFLOPS,
                      "ms_per_launch": round(ms, 3), "workgroups": wgs, "iters": iters, "compute_units": cus,
                      "steps": args.steps, "warmup": args.warmup}), flush=True)
    return 0


COISSUE_VARIANTS = [(0, 0), (4, 0), (8, 0), (16, 0), (0, 1), (0, 2), (0, 4), (3, 1), (4, 2)]


def bench_coissue(args, dev) -> int:
    """What VALU instructions next to the MFMAs cost the MFMA pipe (the
    co-issue kernel of libavf_probe.so): slots of one bf16 MFMA plus nfma
    v_fma_f32 and nexp v_exp_f32, at one and two waves per SIMD. Reports the
    time per MFMA slot per SIMD and its ratio to the MFMA-only slot."""
    import ctypes

    import torch

    from varlen_flashattention_forward_amd import build as avf_build

    if not avf_build.PROBE_LIB.exists():
        raise RuntimeError(f"{avf_build.PROBE_LIB} is missing: build with python -m varlen_flashattention_forward_amd.build")
    P = ctypes.CDLL(str(avf_build.PROBE_LIB))
    P.avf_probe_coissue.restype = ctypes.c_int32
    P.avf_probe_coissue.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 20000
    out = torch.empty(2 * cus * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    rows = []
    for wps in (1, 2):
        wgs = wps * cus  # 4 waves per workgroup: wps waves per SIMD
        base = None
        for nfma, nexp in COISSUE_VARIANTS:
            def launch():
                rc = P.avf_probe_coissue(nfma, nexp, out.data_ptr(), wgs, iters, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"avf_probe_coissue returned {rc}")
            for _ in range(max(1, args.warmup)):
                launch()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            ns_slot = ms * 1e6 / (wps * iters * 8)
            base = ns_slot if base is None else base
            rows.append({"waves_per_simd": wps, "fma_per_slot": nfma, "exp_per_slot": nexp, "ms": round(ms, 4),
                         "ns_per_slot_per_simd": round(ns_slot, 3), "vs_mfma_only": round(ns_slot / base, 3)})
            log(f"[coissue] waves/SIMD {wps} fma {nfma:2d} exp {nexp}: {ns_slot:.3f} ns per MFMA slot per SIMD "
                f"({ns_slot / base:.3f} x MFMA only)")
    print(json.dumps({"metric": "MFMA slot time with VALU co-issue", "unit": "ns per MFMA slot per SIMD",
                      "compute_units": cus, "iters": iters, "slots_per_iter": 8, "steps": args.steps,
                      "results": rows}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-rows", type=int, default=160, help="query rows per segment for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--async", dest="use_async", action="store_true",
                    help="time the sync-free entry point (device planner, no host read-back)")
    ap.add_argument("--batched", action="store_true",
                    help="time the batched-dense entry attn_fwd on [segments, S, H, D] views (uniform segments)")
    ap.add_argument("--fp8", action="store_true",
                    help="time the low-precision forward (E4M3 q and k, 8-bit score product)")
    ap.add_argument("--backward", action="store_true", help="time the backward pass (default workload bwd_9728)")
    ap.add_argument("--cpu-rows-bwd", type=int, default=8, help="dq rows per segment for the backward CPU baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (scales HBM counters)")
    ap.add_argument("--head-major", action="store_true",
                    help="the workload's q, k, v and out as head-major views (row stride D, head stride tokens*D)")
    ap.add_argument("--coissue", action="store_true",
                    help="time MFMA slots with v_fma_f32 / v_exp_f32 co-issued (probe library)")
    ap.add_argument("--mfma-rate", choices=sorted(MFMA_OPERANDS), default=None,
                    help="only time the roofline calibration kernel: a plain stream of bf16 MFMAs "
                         "(v_mfma_f32_32x32x16_bf16) on the given operand pattern, two waves per SIMD")
    ap.add_argument("--copy-rate", type=int, default=0, metavar="MIB",
                    help="only time a plain device-to-device copy of MIB MiB (--warmup, then --steps copies) and "
                         "print its read + write GB/s: the rate a plain stream reaches on this GPU")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2
    if args.workload is None:
        args.workload = "bwd_9728" if args.backward else "dense_77k"
    if args.backward:
        return bench_backward(args)

    import torch

    import varlen_flashattention_forward_amd as avf
    from varlen_flashattention_forward_amd.workloads import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes 3 times")
        return 0
    if args.mfma_rate:
        return bench_mfma_rate(args, dev)
    if args.coissue:
        return bench_coissue(args, dev)
    if args.copy_rate:
        n = args.copy_rate << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            dst.copy_(src)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        print(json.dumps({"metric": "device-to-device copy, read + write bytes per second", "value": 2 * n / ms / 1e6,
                          "unit": "GB/s", "mib": args.copy_rate, "ms_per_copy": ms, "steps": args.steps,
                          "warmup": args.warmup}), flush=True)
        return 0
    w = WORKLOADS[args.workload]
    if args.head_major:
        if w.layout != "contiguous":
            print(f"--head-major needs a contiguous workload ({w.name} is {w.layout})", file=sys.stderr)
            return 2
        w = dataclasses.replace(w, layout="head_major")
    avf.lib()
    log(f"[bench] workload {w.name}: H={w.num_heads} D={w.head_dim} segments={w.num_segments} "
        f"total_q={w.total_q} total_k={w.total_k}")
    t = make_inputs(w, dev, seed=0)
    torch.cuda.synchronize()
    flops = w.flops()
    stream = torch.cuda.current_stream(dev)

    ws = avf.async_workspace(w.num_segments, dev) if args.use_async else None
    ws8 = None
    if args.fp8:
        ws8 = torch.empty(avf.fp8_workspace_bytes(w.total_q, w.total_k, w.num_heads, w.head_dim), dtype=torch.uint8,
                          device=dev)

    if args.batched:
        Ls = {w.cu_q[b + 1] - w.cu_q[b] for b in range(w.num_segments)}
        Lk = {w.cu_k[b + 1] - w.cu_k[b] for b in range(w.num_segments)}
        if len(Ls) != 1 or len(Lk) != 1:
            print(f"--batched needs uniform segments ({w.name} is not)", file=sys.stderr)
            return 2
        W, Sq, Sk = w.num_segments, Ls.pop(), Lk.pop()
        qb, kb, vb = (t[n].view(W, -1, w.num_heads, w.head_dim) for n in ("q", "k", "v"))
        ob = t["out"].view(W, Sq, w.num_heads, w.head_dim)
        lb = torch.empty((W, w.num_heads, Sq), dtype=torch.float32, device=dev)

    def step():
        if args.batched:
            avf.attn_fwd(qb, kb, vb, softmax_scale=w.softmax_scale, causal=w.causal, out=ob, lse=lb)
        elif args.fp8:
            avf.attn_varlen_fwd_fp8(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                    workspace=ws8, softmax_scale=w.softmax_scale, out=t["out"], lse=t["lse"],
                                    causal=w.causal)
        elif args.use_async:
            avf.attn_varlen_fwd_async(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                      workspace=ws, softmax_scale=w.softmax_scale, out=t["out"], lse=t["lse"],
                                      causal=w.causal)
        else:
            avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                softmax_scale=w.softmax_scale, out=t["out"], lse=t["lse"], causal=w.causal)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    # per-step HIP events on the stream inside the timed region give the
    # spread (median, min, max); the value is the wall-clock mean
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3
    value = flops / (ms / 1e3) / 1e12
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    spread = {"median": round(per_step[len(per_step) // 2], 4), "min": round(per_step[0], 4),
              "max": round(per_step[-1], 4)}
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/step, {value:.1f} TFLOP/s (per step {spread})")

    # kernel-only duration: HIP events on the launch stream around `steps`
    # back-to-back calls of the host cu_seqlens entry (no read-back inside the
    # bracket; the host work of a call overlaps the previous call's kernel)
    cu_q, cu_k = list(w.cu_q), list(w.cu_k)

    def launch_only():
        if args.batched:
            avf.attn_fwd(qb, kb, vb, softmax_scale=w.softmax_scale, causal=w.causal, out=ob, lse=lb,
                         stream=stream.cuda_stream)
        elif args.fp8:
            avf.attn_varlen_fwd_fp8(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                    workspace=ws8, softmax_scale=w.softmax_scale, out=t["out"], lse=t["lse"],
                                    cu_seqlens_q_host=cu_q, cu_seqlens_k_host=cu_k, stream=stream.cuda_stream,
                                    causal=w.causal)
        elif args.use_async:
            step()  # planner + attention kernel on the current stream
        else:
            avf.attn_varlen_fwd(t["q"], t["k"], t["v"], t["cu_q"], t["cu_k"], w.max_seqlen_q, w.max_seqlen_k,
                                softmax_scale=w.softmax_scale, out=t["out"], lse=t["lse"],
                                cu_seqlens_q_host=cu_q, cu_seqlens_k_host=cu_k, stream=stream.cuda_stream,
                                causal=w.causal)

    launch_only()
    torch.cuda.synchronize()
    # short kernels: at least ~50 ms of calls in the bracket, so run-to-run
    # clock and cache noise averages out
    nk = args.steps if ms >= 5.0 else max(args.steps, min(1000, int(50.0 / max(ms, 0.01))))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(nk):
        launch_only()
    e1.record(stream)
    torch.cuda.synchronize()
    kms = e0.elapsed_time(e1) / nk
    # the 8-bit forward always takes the general configuration
    max_k_cfg = 1 << 30 if args.fp8 else w.max_seqlen_k
    launches, wgs = avf.grid_plan(w.cu_q, w.num_heads, w.head_dim, max_k_cfg)
    if args.use_async:
        launches, wgs = 1, avf.async_grid(w.total_q, w.num_segments, w.num_heads, w.head_dim, w.max_seqlen_q,
                                          w.max_seqlen_k)
    achieved = flops / launches / (kms / launches / 1e3) / 1e12
    log(f"[bench] kernel: {kms:.3f} ms/call over {launches} launch(es), {wgs} workgroups, {achieved:.1f} TFLOP/s")
    traffic = traffic_for(w.name) if w.layout == "contiguous" else None  # counters: token-major runs
    peak = PEAK_FP8_QK_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
    if args.fp8:
        traffic = None  # the counters were taken on the bf16 kernel
    nbytes = w.algorithmic_bytes()
    roofline = roofline_of(flops // launches, nbytes // launches, kms / launches, peak)
    if roofline["bound"] == "hbm":
        log(f"[bench] below the ridge ({flops / nbytes:.0f} flop/B): {roofline['achieved']} GB/s of algorithmic bytes")
    roofline.update({"traffic": traffic, "kernel_ms": round(kms / launches, 4),
                     "algorithmic_flops_per_launch": flops // launches,
                     "algorithmic_bytes_per_launch": nbytes // launches})

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        cpu = cpu_baseline_fp8(w, t, args.cpu_rows) if args.fp8 else cpu_baseline(w, t, args.cpu_rows)
        log(f"[bench] cpu baseline {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")

    rec = {
        "metric": ("attention fwd TFLOP/s (4*Sq*Sk*D*H), 8-bit q.k, and % of the MI355X fp8/bf16 MFMA peak mix"
                   if args.fp8 else "attention fwd TFLOP/s (4*Sq*Sk*D*H) and % of MI355X bf16 MFMA peak"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": spread,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 q.k, bf16 p.v" if args.fp8 else "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "config": {"workload": w.name, "num_heads": w.num_heads, "head_dim": w.head_dim,
                   "segments": w.num_segments, "total_q": w.total_q, "total_k": w.total_k,
                   "max_seqlen_q": w.max_seqlen_q, "max_seqlen_k": w.max_seqlen_k,
                   "layout": w.layout, "causal": w.causal, "flops_per_step": flops,
                   "workgroups": wgs, "block_m": avf.block_m(w.head_dim, max_k_cfg),
                   "entry": ("attn_fwd_batched" if args.batched else "attn_varlen_fwd_fp8" if args.fp8 else
                             "attn_varlen_fwd_async" if args.use_async else "attn_varlen_fwd")},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
