#!/usr/bin/env python3
"""Benchmark of the fused group-wise affine dequant + matmul on one MI355X.

Headline metric: 4-bit GEMV throughput at M=1 (GB/s and % of HBM peak) on the
decode GEMV set of a 1B-parameter decoder (hidden 2048, FFN 8192: q 2048x2048,
k and v 512x2048, o 2048x2048, gate and up 8192x2048, down 2048x8192; 4-bit
codes, group 64, bf16 scales/biases/activations).  One step = one decode pass
over a stack of `--layers` copies of those seven linears (16 by default, 523
MiB of packed weights, twice the 256 MB Infinity Cache, so each weight is read
cold from HBM).  The step is captured once in a HIP graph and replayed.

Also reported, in the same JSON line: the prefill GEMM figure (M=2048,
K=4096, N=14336, 4-bit and 8-bit, TFLOP/s against the bf16 dense MFMA peak),
the roofline object of the GEMV kernel, and the CPU oracle timed on a bounded
sample of the decode workload.

    python bench.py [--steps K] [--warmup W] [--layers L] [--no-cpu-baseline]
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
METRIC = "q4 GEMV GB/s & %HBM peak (M=1); qGEMM TFLOP/s & %MFMA peak (M=2048)"
G = 64
BITS = 4


def gemv_bytes(M, N, K, bits=BITS, group=G):
    """Algorithmic bytes of one affine GEMV: codes + bf16 scale and bias per
    group + bf16 x in + bf16 y out."""
    return N * K * bits // 8 + N * (K // group) * 4 + M * K * 2 + M * N * 2


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "group_wise_affine_unpack_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_file, key):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE),
    valid only while the kernel source is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(key)
    if not rec or rec.get("src_hash") != src_hash(kernel_file):
        return None
    return rec.get("bytes_per_launch")


def build_stack(layers, device, torch, si):
    """Seeded weights for `layers` copies of the decode set, resident on the GPU.
    Returns device tensors plus host copies of layer 0 for the CPU baseline."""
    dev_layers, host0 = [], None
    for l in range(layers):
        lin = []
        for idx, (name, N, K) in enumerate(si.CFG1_LINEARS):
            packed, s, b = si.affine_weights(N, K, G, BITS, seed=(1, 100 + l, idx), scale_range=(0.005, 0.02),
                                             bias_mode="noise")
            lin.append((name, N, K,
                        torch.from_numpy(packed.view(np.int32)).to(device),
                        torch.from_numpy(s.view(np.int16)).view(torch.bfloat16).to(device),
                        torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(device),
                        (packed, s, b) if l == 0 else None))
        dev_layers.append(lin)
    return dev_layers


def time_gemv_stack(args, torch, qa, si, device):
    stack = build_stack(args.layers, device, torch, si)
    M = 1
    xs = {K: torch.from_numpy(si.activations(M, K, seed=(1, 7, K)).view(np.int16)).view(torch.bfloat16).to(device)
          for K in (2048, 8192)}
    ys = {N: torch.empty((M, N), dtype=torch.bfloat16, device=device) for N in (512, 2048, 8192)}

    def step():
        for lin in stack:
            for name, N, K, w, s, b, _ in lin:
                qa.qmm_affine(xs[K], w, s, b, G, BITS, out=ys[N])

    launches_per_step = sum(len(l) for l in stack)
    bytes_per_step = sum(gemv_bytes(M, N, K) for l in stack for _, N, K, *_ in l)

    # capture one step in a HIP graph (our launches go to torch's current stream)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()                                # first launches outside capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ms_per_step = ms / args.steps
    gbs = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    avg_launch_us = ms_per_step * 1e3 / launches_per_step
    host0 = [(N, K, h) for _, N, K, _, _, _, h in stack[0]]
    return dict(ms_per_step=ms_per_step, gbs=gbs, bytes_per_step=bytes_per_step,
                launches_per_step=launches_per_step, avg_launch_us=avg_launch_us,
                bytes_per_launch=bytes_per_step / launches_per_step, host0=host0,
                x_host={K: si.activations(M, K, seed=(1, 7, K)) for K in (2048, 8192)})


def time_gemm(torch, qa, si, device, bits, N=14336, K=4096, M=2048, iters=20, warmup=5):
    """Prefill GEMM on the largest cfg shape; returns None when the path is not built."""
    case = si.cfg2_case(N, K, bits, M=M, seed=(2, N, K))
    x = torch.from_numpy(case.x.view(np.int16)).view(torch.bfloat16).to(device)
    w = torch.from_numpy(case.packed.view(np.int32)).to(device)
    s = torch.from_numpy(case.scales.view(np.int16)).view(torch.bfloat16).to(device)
    b = torch.from_numpy(case.biases.view(np.int16)).view(torch.bfloat16).to(device)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    try:
        qa.qmm_affine(x, w, s, b, G, bits, out=y)
    except qa.QaffError as e:
        if e.status == 2:
            return None
        raise
    for _ in range(warmup):
        qa.qmm_affine(x, w, s, b, G, bits, out=y)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(iters):
        qa.qmm_affine(x, w, s, b, G, bits, out=y)
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / iters
    tflops = 2.0 * M * N * K / (us * 1e-6) / 1e12
    return {"bits": bits, "M": M, "N": N, "K": K, "us_per_call": round(us, 2), "tflops": round(tflops, 1),
            "frac_of_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4)}


def cpu_baseline(res, seconds):
    """The fp64 oracle on the host cores over layer-0 linears of the same decode
    workload (M=1), repeated until `seconds` of work or one full layer pass."""
    import oracle
    done_bytes, t0, passes = 0, time.perf_counter(), 0
    while True:
        for N, K, (packed, s, b) in res["host0"]:
            x = res["x_host"][K]
            oracle.qmm_affine(x, "bf16", packed, s, b, "bf16", 1, N, K, G, BITS)
            done_bytes += gemv_bytes(1, N, K)
        passes += 1
        if time.perf_counter() - t0 >= seconds or passes >= 1000:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{passes} pass(es) over layer 0 of the decode set (7 linears, M=1, 4-bit G=64), "
                      f"{dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--skip-gemv", action="store_true", help="time only the prefill GEMM (for profiling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import group_wise_affine_unpack_amd as qa
    import synth_inputs as si
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    qa.lib()

    if args.skip_gemv:
        for bits in (4, 8):
            print(json.dumps({"gemm_m2048": time_gemm(torch, qa, si, device, bits)}), flush=True)
        return
    res = time_gemv_stack(args, torch, qa, si, device)
    print(f"[bench] gemv stack: {res['ms_per_step']*1e3:.1f} us/step, {res['gbs']:.0f} GB/s, "
          f"{res['avg_launch_us']:.2f} us/launch avg", file=sys.stderr, flush=True)

    gemm = None
    if not args.no_gemm:
        gemm = [g for g in (time_gemm(torch, qa, si, device, 4), time_gemm(torch, qa, si, device, 8)) if g]
        for g in gemm:
            print(f"[bench] gemm b{g['bits']}: {g['us_per_call']} us, {g['tflops']} TFLOP/s", file=sys.stderr,
                  flush=True)

    achieved = res["bytes_per_launch"] / (res["avg_launch_us"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": load_traffic("gemv_affine.hip", "gemv_decode_stack_m1"),
                "kernel": "gemv_affine_kernel (4-bit, bf16, M=1)",
                "bytes_per_launch": round(res["bytes_per_launch"]), "avg_launch_us": round(res["avg_launch_us"], 3)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(res, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(res["gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode GEMV set of a 1B decoder (hidden 2048, FFN 8192), M=1, 4-bit codes, G=64, "
                               f"bf16 scales/biases/activations, {args.layers}-layer stack, HIP-graph replay",
                   "M": 1, "layers": args.layers, "linears_per_layer": 7, "bits": BITS, "group_size": G,
                   "bytes_per_step": res["bytes_per_step"], "frac_of_hbm_peak": round(res["gbs"] / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "gemm_m2048": gemm,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
