#!/usr/bin/env python3
"""Benchmark of the fused group-wise affine dequant + matmul on one MI355X.

Headline metric: 4-bit GEMV throughput at M=1 (GB/s and fraction of the HBM
peak) on the decode GEMV set of a 1B-parameter decoder (hidden 2048, FFN 8192:
q 2048x2048, k and v 512x2048, o 2048x2048, gate and up 8192x2048, down
2048x8192; 4-bit codes, group 64, bf16 scales/biases/activations), over a
stack of `--layers` copies of those seven linears (16 by default: 523 MiB of
packed weights, twice the 256 MB Infinity Cache, so weights stream from HBM).

One step = every linear of the stack once, at M=1, through the grouped GEMV
entry point (qgemv_affine_grouped: 56 problems per launch, so 2 launches for
16 layers).  This is the steady-state figure: the kernel streams weights
with almost no launch gaps.  In the same JSON line:
  decode_chain   the same linears in decoder dependency order, one grouped
                 call per dependent step (qkv, o, gate+up, down): 64 launches
  decode_chain_one_launch
                 a decoder chain of the same weights whose stages really depend
                 on each other (o reads q and adds h, gate/up read o, down reads
                 silu(gate)*up and adds o, the next layer reads down), all 64
                 stages in one launch (qgemv_affine_chain_run)
  per_linear     one qmm_affine launch per linear: 112 launches
  cfg0_hot       the single 2048x2048 linear relaunched on the same weights
                 (cache-resident: NOT an HBM figure)
  decode_set_multirow
                 the grouped decode set at M = 4 and 16 (the MFMA GEMV kernel)
  gptq_k4096_n11008
                 GPTQ layout (K=4096, N=11008, G=128, act-order) at M = 1 and
                 32: the direct kernel and the repacked affine path, eager and
                 replayed from a HIP graph; and the direct kernel on a layer
                 without act-order (g_idx passed as NULL), from a HIP graph
  gemm_m2048     prefill GEMM of an 8B decoder, M=2048: K=4096 with N = 4096,
                 1024, 14336 and K=14336 with N=4096, 4- and 8-bit, TFLOP/s
                 against the bf16 dense MFMA peak
  w4a8_m2048     W4A8 GEMM (quantize + int8 MFMA), M=2048 N=4096 K=1024,
                 eager and from a HIP graph
  w4a8_shapes    every W4A8 shape of the speech-encoder set, graph replays
  stream_read    the achievable HBM read rate: a plain streaming read of
                 1 GiB (qaff_stream_read), beside the 8 TB/s published peak
  gemv_cold      one GEMV launch per call for each decode-set shape (2048x2048
                 is also the single-linear configuration) at M = 1, 4, 16:
                 cold = weights rotated over >= 1 GiB of replicas (every
                 launch streams from HBM, gaps between launches included),
                 hot = the same launches on one replica (NOT an HBM figure)
  dequant_n14336_k4096, silu_gate_down, w4a8_smooth_m2048
                 the standalone dequantize, the SiLU-gated down projection
                 and W4A8 with the SmoothQuant divide
  roofline       the grouped GEMV kernel of the headline step
  gemm_roofline  the 4-bit M=2048 N=14336 K=4096 prefill call
  cpu_baseline   the fp64 CPU oracle on a bounded sample of the same
                 workload, and (per_config) on every configuration: median
                 of 3 runs, all host threads, plus one thread for the decode
                 shapes; row samples for the M=2048 shapes, scaled to full M
Every GPU figure is timed with HIP events on the stream the kernels run on:
the headline step is launched directly (two launches, one host call), the
many-launch figures as replays of a captured HIP graph.  Figures with p10/p90
come from one event pair per call (or per graph replay).

    python bench.py [--steps K] [--warmup W] [--layers L] [--no-cpu-baseline] [--no-cold]
    python bench.py --traffic-probe   (short run for rocprofv3 --pmc passes)
    python bench.py --summarize DB [FILTER]   (kernel-trace percentiles, no GPU)
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
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published
METRIC = "q4 GEMV GB/s & %HBM peak (M=1); qGEMM TFLOP/s & %MFMA peak (M=2048)"
G = 64
BITS = 4
PER_LAUNCH = 56                # problems per grouped GEMV launch
REPS = 20                      # calls per captured graph in the graph-replay figures


def gemv_bytes(M, N, K, bits=BITS, group=G):
    """Algorithmic bytes of one affine GEMV: codes + bf16 scale and bias per
    group + bf16 x in + bf16 y out."""
    return N * K * bits // 8 + N * (K // group) * 4 + M * K * 2 + M * N * 2


def src_hash(*names):
    """Hash of the code in the named kernel sources, ignoring // comments and
    blank lines (a changed comment does not change the kernel)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "group_wise_affine_unpack_amd", "csrc", n), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
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
    """Seeded weights for `layers` copies of the decode set, resident on the GPU."""
    stack = []
    for l in range(layers):
        lin = []
        for idx, (name, N, K) in enumerate(si.CFG1_LINEARS):
            packed, s, b = si.affine_weights(N, K, G, BITS, seed=(1, 100 + l, idx), scale_range=(0.005, 0.02),
                                             bias_mode="noise")
            lin.append(dict(name=name, N=N, K=K,
                            w=torch.from_numpy(packed.view(np.int32)).to(device),
                            s=torch.from_numpy(s.view(np.int16)).view(torch.bfloat16).to(device),
                            b=torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(device),
                            host=(packed, s, b) if l == 0 else None))
        stack.append(lin)
    return stack


def eager_time(torch, fn, steps, warmup):
    """Run fn() on the current stream, timing `steps` calls with events on that
    stream (for steps whose host work is far shorter than their GPU work)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def graph_time(torch, fn, steps, warmup):
    """Capture fn() in a HIP graph, replay it, time the replays with events on
    the replay stream.  Returns ms per step.  The eager warm-up call runs on
    the capture stream, so the library's per-stream workspace is sized before
    the capture."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def pct(v):
    """median, p10, p90 of a list (microseconds)."""
    a = np.asarray(v, dtype=np.float64)
    return {"median_us": round(float(np.median(a)), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def event_times(torch, fn, iters, warmup):
    """Per-call durations (us) of fn() on the current stream, one event pair
    around each call (for calls of tens of microseconds and more)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def graph_replay_times(torch, fn, replays, warmup=2):
    """Capture fn() once (after one eager call on the capture stream) and
    return the duration (us) of each of `replays` replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    del g
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def time_stream_read(torch, qa, device, nbytes=1 << 30, iters=20):
    """The achievable streaming-read rate: qaff_stream_read over 1 GiB, the
    best of five grid sizes (2 to 32 workgroups per CU), median of `iters`
    launches each.  The rate depends on the grid: 4 workgroups per CU read
    faster than 8 or more."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    buf.fill_(3)
    best, by_grid = None, {}
    for blocks in (512, 1024, 2048, 4096, 8192):
        sink = torch.empty(blocks * 256, dtype=torch.int32, device=device)
        t = pct(event_times(torch, lambda: qa.stream_read(buf, sink, blocks), iters, 3))
        gbs = nbytes / (t["median_us"] * 1e-6) / 1e9
        by_grid[str(blocks)] = round(gbs, 1)
        if best is None or gbs > best["gbs"]:
            best = {"bytes": nbytes, "blocks": blocks, **t, "gbs": round(gbs, 1),
                    "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del buf
    torch.cuda.empty_cache()
    return {**best, "gbs_by_grid": by_grid}


def time_cold_gemv(torch, qa, si, device, N, K, Ms=(1, 4, 16), min_bytes=1 << 30, replays=5):
    """One affine GEMV launch per call (qmm_affine), cold and hot.

    Cold: R replicas of (codes, scales, biases) with R x weight bytes >= 1 GiB,
    more than four times the Infinity Cache, one launch per replica in a
    captured graph, so every launch streams its weights from HBM; time per
    launch includes the gaps between launches.  Hot: the same number of
    launches on one replica (cache-resident: NOT an HBM figure)."""
    packed, sc, bi = si.affine_weights(N, K, G, BITS, seed=(1, 900, N, K), scale_range=(0.005, 0.02),
                                       bias_mode="noise")
    wbytes = N * K * BITS // 8 + N * (K // G) * 4
    R = -(-min_bytes // wbytes)
    w = torch.from_numpy(packed.view(np.int32)).to(device).unsqueeze(0).repeat(R, 1, 1)
    s = torch.from_numpy(sc.view(np.int16)).view(torch.bfloat16).to(device).unsqueeze(0).repeat(R, 1, 1)
    b = torch.from_numpy(bi.view(np.int16)).view(torch.bfloat16).to(device).unsqueeze(0).repeat(R, 1, 1)
    out = []
    for M in Ms:
        x = torch.from_numpy(si.activations(M, K, seed=(1, 901, K, M)).view(np.int16)).view(torch.bfloat16).to(device)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=device)
        cold = lambda: [qa.qmm_affine(x, w[r], s[r], b[r], G, BITS, out=y) for r in range(R)]
        hot = lambda: [qa.qmm_affine(x, w[0], s[0], b[0], G, BITS, out=y) for _ in range(R)]
        tc = [t / R for t in graph_replay_times(torch, cold, replays)]
        th = [t / R for t in graph_replay_times(torch, hot, replays)]
        byts = gemv_bytes(M, N, K)
        pc, ph = pct(tc), pct(th)
        gc = byts / (pc["median_us"] * 1e-6) / 1e9
        out.append({"M": M, "N": N, "K": K, "replicas": R, "bytes_per_launch": byts,
                    "cold_us": pc["median_us"], "cold_p10_us": pc["p10_us"], "cold_p90_us": pc["p90_us"],
                    "cold_gbs": round(gc, 1), "cold_frac_of_hbm_peak": round(gc / HBM_PEAK_GBS, 4),
                    "hot_us": ph["median_us"], "hot_gbs_not_hbm": round(byts / (ph["median_us"] * 1e-6) / 1e9, 1)})
    del w, s, b
    torch.cuda.empty_cache()
    return out


class Decode:
    """The decode set on the GPU plus the three ways of running it."""

    def __init__(self, args, torch, qa, si, device):
        self.stack = build_stack(args.layers, device, torch, si)
        self.M = 1
        self.x_host = {K: si.activations(self.M, K, seed=(1, 7, K)) for K in (2048, 8192)}
        self.x = {K: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).to(device) for K, v in self.x_host.items()}
        # one output per linear, so grouped launches never share an output
        self.y = [[torch.empty((self.M, d["N"]), dtype=torch.bfloat16, device=device) for d in lin]
                  for lin in self.stack]
        prob = lambda l, i: (self.x[self.stack[l][i]["K"]], self.stack[l][i]["w"], self.stack[l][i]["s"],
                             self.stack[l][i]["b"])
        L = len(self.stack)
        flat = [(l, i) for l in range(L) for i in range(7)]
        self.set_call = qa.GroupedGemv([prob(l, i) for l, i in flat], G, BITS, outs=[self.y[l][i] for l, i in flat])
        # decoder order: q/k/v share x; o; gate/up share x; down
        self.chain = []
        for l in range(L):
            for idx in ((0, 1, 2), (3,), (4, 5), (6,)):
                self.chain.append(qa.GroupedGemv([prob(l, i) for i in idx], G, BITS, outs=[self.y[l][i] for i in idx]))
        self.qa = qa
        self.bytes_per_step = sum(gemv_bytes(self.M, d["N"], d["K"]) for lin in self.stack for d in lin)
        self.n_linears = 7 * L

    def run_set(self):
        self.set_call()

    def run_chain(self):
        for c in self.chain:
            c()

    def chain_plan(self):
        """The decoder chain with real dependencies, one plan for the stack:
        q/k/v read h; o reads q (the attention output's stand-in) plus h;
        gate/up read o; down reads silu(gate) * up plus o, and is the next h."""
        lins, h = [], self.x[2048][0]
        for l, lin in enumerate(self.stack):
            y = [t[0] for t in self.y[l]]
            d = lambda i, **kw: dict(w=lin[i]["w"], s=lin[i]["s"], b=lin[i]["b"], y=y[i], **kw)
            st = 4 * l
            lins += [d(0, x=h, stage=st), d(1, x=h, stage=st), d(2, x=h, stage=st),
                     d(3, x=y[0], resid=h, stage=st + 1),
                     d(4, x=y[3], stage=st + 2), d(5, x=y[3], stage=st + 2),
                     d(6, x=y[5], gate=y[4], resid=y[3], stage=st + 3)]
            h = y[6]
        return self.qa.GemvChain(lins, G, BITS)

    def run_per_linear(self):
        for l, lin in enumerate(self.stack):
            for i, d in enumerate(lin):
                self.qa.qmm_affine(self.x[d["K"]], d["w"], d["s"], d["b"], G, BITS, out=self.y[l][i])


def time_gemm(torch, qa, si, device, bits, N=14336, K=4096, M=2048, iters=50, warmup=10):
    """One qmm_affine call at M=2048 (the pre-pass kernel plus the GEMM
    kernel): per-call event pairs, median with p10/p90."""
    case = si.cfg2_case(N, K, bits, M=M, seed=(2, N, K))
    x = torch.from_numpy(case.x.view(np.int16)).view(torch.bfloat16).to(device)
    w = torch.from_numpy(case.packed.view(np.int32)).to(device)
    s = torch.from_numpy(case.scales.view(np.int16)).view(torch.bfloat16).to(device)
    b = torch.from_numpy(case.biases.view(np.int16)).view(torch.bfloat16).to(device)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    t = pct(event_times(torch, lambda: qa.qmm_affine(x, w, s, b, G, bits, out=y), iters, warmup))
    us = t["median_us"]
    tflops = 2.0 * M * N * K / (us * 1e-6) / 1e12
    return {"bits": bits, "M": M, "N": N, "K": K, "us_per_call": us, "p10_us": t["p10_us"], "p90_us": t["p90_us"],
            "tflops": round(tflops, 1), "frac_of_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4)}


def time_extras(torch, qa, si, device, dec, iters=50):
    """The other entry points on the hot path's shapes: the standalone
    dequantize (N=14336, K=4096, 4-bit, to bf16), the SiLU-gated down
    projection of the decode stack (M=1, one launch per layer, graph-timed),
    and W4A8 with the SmoothQuant divide (M=2048, N=4096, K=1024)."""
    out = {}
    N, K = 14336, 4096
    packed, sc, bi = si.affine_weights(N, K, G, BITS, seed=(5, N, K), scale_range=(0.002, 0.01), bias_mode="exact")
    w = torch.from_numpy(packed.view(np.int32)).to(device)
    s = torch.from_numpy(sc.view(np.int16)).view(torch.bfloat16).to(device)
    b = torch.from_numpy(bi.view(np.int16)).view(torch.bfloat16).to(device)
    o = torch.empty((N, K), dtype=torch.bfloat16, device=device)
    t = pct(event_times(torch, lambda: qa.dequantize_affine(w, s, b, K, G, BITS, out=o), iters, 5))
    byts = N * K * BITS // 8 + N * (K // G) * 4 + N * K * 2
    gbs = byts / (t["median_us"] * 1e-6) / 1e9
    out["dequant_n14336_k4096"] = {"bits": BITS, "out": "bf16", **t, "bytes": byts, "gbs": round(gbs, 1),
                                   "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del w, s, b, o
    # SiLU-gated down projection: y = W_down (silu(g) * u) + resid, one per layer
    downs = [lin[6] for lin in dec.stack]
    Kd, Nd = downs[0]["K"], downs[0]["N"]
    gt = torch.from_numpy(si.activations(1, Kd, seed=(5, 1)).view(np.int16)).view(torch.bfloat16).to(device)
    up = torch.from_numpy(si.activations(1, Kd, seed=(5, 2)).view(np.int16)).view(torch.bfloat16).to(device)
    rs = torch.from_numpy(si.activations(1, Nd, seed=(5, 3)).view(np.int16)).view(torch.bfloat16).to(device)
    ys = [torch.empty((1, Nd), dtype=torch.bfloat16, device=device) for _ in downs]
    fn = lambda: [qa.qgemv_affine_silu_gate(gt, up, d["w"], d["s"], d["b"], G, BITS, resid=rs, out=y)
                  for d, y in zip(downs, ys)]
    t = pct([v / len(downs) for v in graph_replay_times(torch, fn, 20)])
    byts = gemv_bytes(1, Nd, Kd) + Kd * 2 + Nd * 2  # + the up row and the residual
    gbs = byts / (t["median_us"] * 1e-6) / 1e9
    out["silu_gate_down"] = {"M": 1, "N": Nd, "K": Kd, "launches": len(downs), "us_per_launch": t["median_us"],
                             "p10_us": t["p10_us"], "p90_us": t["p90_us"], "bytes_per_launch": byts,
                             "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    # W4A8 with smoothing
    M, N, K = 2048, 4096, 1024
    case = si.w4a8_case(M, N, K, seed=(4, N, K, M))
    x = torch.from_numpy(case.x.view(np.int16)).view(torch.float16).to(device)
    wq = torch.from_numpy(case.w_q4.view(np.int32)).to(device)
    sw = torch.from_numpy(case.s_w.view(np.int16)).view(torch.float16).to(device)
    sm = torch.from_numpy(np.random.default_rng(6).uniform(0.5, 2.0, K).astype(np.float32)).to(device)
    fn = lambda: qa.qgemm_w4a8_smooth(x, sm, wq, sw)
    t = pct([v / REPS for v in graph_replay_times(torch, lambda: [fn() for _ in range(REPS)], 20)])
    ops = 2.0 * M * N * K
    out["w4a8_smooth_m2048"] = {"M": M, "N": N, "K": K, "graph_us_per_call": t["median_us"], "p10_us": t["p10_us"],
                                "p90_us": t["p90_us"], "tops": round(ops / (t["median_us"] * 1e-6) / 1e12, 1),
                                "frac_of_int8_peak": round(ops / (t["median_us"] * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)}
    torch.cuda.empty_cache()
    return out


def time_decode_m(torch, qa, si, device, dec, M, steps, warmup):
    """The decode set at M x rows (the configuration's M = 4 and 16), grouped
    as in the headline; M >= 2 runs the MFMA GEMV kernel."""
    xs = {K: torch.from_numpy(si.activations(M, K, seed=(1, 8, K, M)).view(np.int16)).view(torch.bfloat16).to(device)
          for K in (2048, 8192)}
    lins = [d for lin in dec.stack for d in lin]
    outs = [torch.empty((M, d["N"]), dtype=torch.bfloat16, device=device) for d in lins]
    call = qa.GroupedGemv([(xs[d["K"]], d["w"], d["s"], d["b"]) for d in lins], G, BITS, outs=outs)
    ms = eager_time(torch, call, steps, warmup)
    byts = sum(gemv_bytes(M, d["N"], d["K"]) for d in lins)
    gbs = byts / (ms * 1e-3) / 1e9
    return {"M": M, "us_per_step": round(ms * 1e3, 1), "gbs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def time_gptq(torch, qa, si, device, M, iters=200, warmup=20):
    """GPTQ layout, K=4096 N=11008 G=128 act-order: the direct kernel and the
    repacked affine path, at M x rows."""
    c = si.cfg3_case(M)
    x = torch.from_numpy(c.x.view(np.int16)).view(torch.float16).to(device)
    qw = torch.from_numpy(c.qweight.view(np.int32)).to(device)
    qz = torch.from_numpy(c.qzeros.view(np.int32)).to(device)
    sc = torch.from_numpy(c.scales.view(np.int16)).view(torch.float16).to(device)
    gi = torch.from_numpy(c.g_idx.astype(np.int32)).to(device)
    byts = (c.K * c.N // 2 + (c.K // c.G) * c.N * 2 + (c.K // c.G) * c.N // 2 + c.K * 4
            + M * c.K * 2 + M * c.N * 2)
    direct = lambda: qa.qmm_gptq(x, qw, qz, sc, gi, c.G)
    ms_d = eager_time(torch, direct, iters, warmup)
    w, s2, b2, kp = qa.gptq_to_affine_repack(qw, qz, sc, gi, c.G)
    repacked = lambda: qa.qmm_affine(x, w, s2, b2, c.G, 4, k_perm=kp)
    ms_r = eager_time(torch, repacked, iters, warmup)
    # the same calls, REPS per captured HIP graph: device time per call
    # without the per-call host work (Python binding, launches) or the cost of
    # launching the graph itself
    ms_dg = graph_time(torch, lambda: [direct() for _ in range(REPS)], iters // REPS + 1, 2) / REPS
    ms_rg = graph_time(torch, lambda: [repacked() for _ in range(REPS)], iters // REPS + 1, 2) / REPS
    return {"M": M, "N": c.N, "K": c.K, "G": c.G,
            "direct_us": round(ms_d * 1e3, 2), "direct_gbs": round(byts / (ms_d * 1e-3) / 1e9, 1),
            "repacked_affine_us": round(ms_r * 1e3, 2),
            "direct_graph_us": round(ms_dg * 1e3, 2), "direct_graph_gbs": round(byts / (ms_dg * 1e-3) / 1e9, 1),
            "repacked_affine_graph_us": round(ms_rg * 1e3, 2),
            "repacked_affine_graph_gbs": round(byts / (ms_rg * 1e-3) / 1e9, 1),
            **time_gptq_no_act(torch, qa, si, device, M, iters)}


def time_gptq_no_act(torch, qa, si, device, M, iters):
    """The direct kernel on the same shape without act-order, g_idx NULL (each
    workgroup's table then holds only its K slice's groups), graph-timed."""
    c = si.gptq_case(M, si.CFG3["K"], si.CFG3["N"], si.CFG3["G"], seed=(3, 0, M), act_order=False)
    x = torch.from_numpy(c.x.view(np.int16)).view(torch.float16).to(device)
    qw = torch.from_numpy(c.qweight.view(np.int32)).to(device)
    qz = torch.from_numpy(c.qzeros.view(np.int32)).to(device)
    sc = torch.from_numpy(c.scales.view(np.int16)).view(torch.float16).to(device)
    byts = (c.K * c.N // 2 + (c.K // c.G) * c.N * 2 + (c.K // c.G) * c.N // 2 + M * c.K * 2 + M * c.N * 2)
    direct = lambda: qa.qmm_gptq(x, qw, qz, sc, None, c.G)
    ms = graph_time(torch, lambda: [direct() for _ in range(REPS)], iters // REPS + 1, 2) / REPS
    return {"no_act_direct_graph_us": round(ms * 1e3, 2), "no_act_direct_graph_gbs": round(byts / (ms * 1e-3) / 1e9, 1)}


def time_w4a8(torch, qa, si, device, M=2048, N=4096, K=1024, iters=20, warmup=5):
    """One W4A8 call (quantize + int8 GEMM): eager, and REPS calls per
    captured HIP graph (device time without the per-call host work)."""
    case = si.w4a8_case(M, N, K, seed=(4, N, K, M))
    x = torch.from_numpy(case.x.view(np.int16)).view(torch.float16).to(device)
    w = torch.from_numpy(case.w_q4.view(np.int32)).to(device)
    sw = torch.from_numpy(case.s_w.view(np.int16)).view(torch.float16).to(device)
    fn = lambda: qa.qgemm_w4a8(x, w, sw)
    us = eager_time(torch, fn, iters, warmup) * 1e3
    usg = graph_time(torch, lambda: [fn() for _ in range(REPS)], iters, 2) * 1e3 / REPS
    ops = 2.0 * M * N * K
    return {"M": M, "N": N, "K": K, "us_per_call": round(us, 2), "tops": round(ops / (us * 1e-6) / 1e12, 1),
            "frac_of_int8_peak": round(ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4),
            "graph_us_per_call": round(usg, 2), "graph_tops": round(ops / (usg * 1e-6) / 1e12, 1)}


def time_w4a8_shapes(torch, qa, si, device, iters=20, warmup=5):
    """Every W4A8 shape of the speech-encoder set (d = 1024, FFN 4096): REPS
    calls per captured graph, microseconds per call."""
    out = []
    for N, K in si.CFG4_SHAPES:
        for M in si.CFG4_M:
            case = si.w4a8_case(M, N, K, seed=(4, N, K, M))
            x = torch.from_numpy(case.x.view(np.int16)).view(torch.float16).to(device)
            w = torch.from_numpy(case.w_q4.view(np.int32)).to(device)
            sw = torch.from_numpy(case.s_w.view(np.int16)).view(torch.float16).to(device)
            fn = lambda: qa.qgemm_w4a8(x, w, sw)
            us = graph_time(torch, lambda: [fn() for _ in range(REPS)], iters, 2) * 1e3 / REPS
            out.append({"M": M, "N": N, "K": K, "graph_us": round(us, 2),
                        "tops": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 1)})
    return out


W4A8_TILES = [(32, 128), (64, 128), (64, 256), (128, 256)]


def time_w4a8_sweep(torch, qa, si, device, replays=10):
    """Both W4A8 lowerings (staged: quantize inside the GEMM; full-K:
    quantize kernel, then the GEMM) at every built tile, for each shape of
    the set with M > 16.  Each configuration is checked first (x_q, s_x, acc
    and y the same bits as the default call), then timed: REPS calls per
    captured graph, median of `replays`.  The fastest passing configuration
    is reported beside the default's time."""
    out = []
    for N, K in si.CFG4_SHAPES:
        for M in si.CFG4_M:
            if M <= 16:
                continue
            case = si.w4a8_case(M, N, K, seed=(4, N, K, M))
            x = torch.from_numpy(case.x.view(np.int16)).view(torch.float16).to(device)
            w = torch.from_numpy(case.w_q4.view(np.int32)).to(device)
            sw = torch.from_numpy(case.s_w.view(np.int16)).view(torch.float16).to(device)
            ref = qa.qgemm_w4a8(x, w, sw, want_acc=True)
            fn = lambda: qa.qgemm_w4a8(x, w, sw)
            t = pct([v / REPS for v in graph_replay_times(torch, lambda: [fn() for _ in range(REPS)], replays)])
            row = {"M": M, "N": N, "K": K, "default_us": t["median_us"], "configs": []}
            for staged in (0, 1):
                for bm, bn in W4A8_TILES:
                    got = qa.qgemm_w4a8_tiled(x, w, sw, staged, bm, bn, want_acc=True)
                    ok = all(torch.equal(a.view(torch.int8) if a.dtype == torch.int8 else a, b)
                             for a, b in ((got[1], ref[1]), (got[3], ref[3]))) and \
                        torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)) and \
                        torch.equal(got[2].view(torch.int32), ref[2].view(torch.int32))
                    c = {"staged": staged, "bm": bm, "bn": bn, "same_bits": bool(ok)}
                    if ok:
                        f = lambda: qa.qgemm_w4a8_tiled(x, w, sw, staged, bm, bn)
                        tc = pct([v / REPS for v in graph_replay_times(torch, lambda: [f() for _ in range(REPS)],
                                                                       replays)])
                        c["us"] = tc["median_us"]
                    row["configs"].append(c)
            passing = [c for c in row["configs"] if c["same_bits"]]
            best = min(passing, key=lambda c: c["us"]) if passing else None
            row["best"] = best
            ops = 2.0 * M * N * K
            if best:
                row["best_tops"] = round(ops / (best["us"] * 1e-6) / 1e12, 1)
            out.append(row)
            torch.cuda.empty_cache()
    return out


def cpu_baseline(dec, seconds):
    """The fp64 oracle on the host cores over the layer-0 linears of the same
    decode workload (M=1), repeated until `seconds` of work."""
    import oracle
    done_bytes, t0, passes = 0, time.perf_counter(), 0
    while True:
        for d in dec.stack[0]:
            packed, s, b = d["host"]
            oracle.qmm_affine(dec.x_host[d["K"]], "bf16", packed, s, b, "bf16", 1, d["N"], d["K"], G, BITS)
            done_bytes += gemv_bytes(1, d["N"], d["K"])
        passes += 1
        if time.perf_counter() - t0 >= seconds or passes >= 1000:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{passes} pass(es) over layer 0 of the decode set (7 linears, M=1, 4-bit G=64), "
                      f"{dt:.1f} s wall"}


def oracle_timings(si):
    """The fp64 oracle per configuration on the host cores: wall-clock median
    of 3 runs, all threads, plus one thread for cfg0/cfg1.  cfg2 and the
    M=2048 cfg4 shapes run on a sample of rows (stated), scaled to the full M."""
    import oracle

    def med3(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    cores = oracle.num_threads()
    rows = []

    def affine_row(name, case, sample_rows=None, one_thread=False):
        x = case.x if sample_rows is None else case.x[:sample_rows]
        m = x.shape[0]
        fn = lambda: oracle.qmm_affine(x, case.act_dtype, case.packed, case.scales, case.biases, case.sb_dtype, m,
                                       case.N, case.K, case.G, case.bits)
        t = med3(fn)
        r = {"config": name, "M": case.M, "N": case.N, "K": case.K, "bits": case.bits, "rows_run": m,
             "s": round(t, 4), "s_full_M": round(t * case.M / m, 3)}
        if one_thread:
            oracle.set_num_threads(1)
            r["s_1thread"] = round(med3(fn), 4)
            oracle.set_num_threads(cores)
        rows.append(r)

    affine_row("cfg0", si.cfg0_case(), one_thread=True)
    for _, N, K in si.CFG1_LINEARS:
        if (N, K) in [(rr["N"], rr["K"]) for rr in rows if rr["config"] == "cfg1"]:
            continue
        for M in si.CFG1_M:
            affine_row("cfg1", si.cfg1_case(N, K, M, seed=(1, N, K, M)), one_thread=True)
    for bits in si.CFG2_BITS:
        for N, K in si.CFG2_SHAPES:
            affine_row("cfg2", si.cfg2_case(N, K, bits, seed=(2, N, K)), sample_rows=8)
    for M in si.CFG3_M:
        c = si.cfg3_case(M)
        t = med3(lambda: oracle.qmm_gptq(c.x, c.qweight, c.qzeros, c.scales, c.g_idx, M, c.K, c.N, c.G))
        rows.append({"config": "cfg3", "M": M, "N": c.N, "K": c.K, "G": c.G, "rows_run": M, "s": round(t, 4),
                     "s_full_M": round(t, 4)})
    for N, K in si.CFG4_SHAPES:
        for M in si.CFG4_M:
            c = si.cfg4_case(N, K, M, seed=(4, N, K, M))
            m = min(M, 256)
            t = med3(lambda: oracle.w4a8(c.x[:m], c.w_q4, c.s_w, m, N, K))
            rows.append({"config": "cfg4", "M": M, "N": N, "K": K, "rows_run": m, "s": round(t, 4),
                         "s_full_M": round(t * M / m, 3)})
    return {"cores": cores, "runs": "median of 3 wall-clock runs per row", "rows": rows}


def traffic_probe(torch, qa, si, device, dec):
    """A short, eager run for rocprofv3 --pmc passes: a plain copy of known size
    (calibration), then three headline steps, then three 4-bit prefill calls
    at M=2048, N=14336, K=4096."""
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    for _ in range(3):
        dec.run_set()
    torch.cuda.synchronize()
    case = si.cfg2_case(14336, 4096, 4, seed=(2, 14336, 4096))
    x = torch.from_numpy(case.x.view(np.int16)).view(torch.bfloat16).to(device)
    w = torch.from_numpy(case.packed.view(np.int32)).to(device)
    s = torch.from_numpy(case.scales.view(np.int16)).view(torch.bfloat16).to(device)
    b = torch.from_numpy(case.biases.view(np.int16)).view(torch.bfloat16).to(device)
    for _ in range(3):
        qa.qmm_affine(x, w, s, b, G, 4)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "set_bytes_per_step": dec.bytes_per_step,
                      "launches_per_step": -(-dec.n_linears // PER_LAUNCH)}), flush=True)


def gemm_bytes(M, N, K, bits=4, group=G):
    """Algorithmic bytes of one prefill call: codes, bf16 scales and biases,
    bf16 x in and bf16 y out (each once)."""
    return N * K * bits // 8 + N * (K // group) * 4 + M * K * 2 + M * N * 2


def record_traffic(fetch_db, write_db):
    """Turn two rocprofv3 --pmc databases of `bench.py --traffic-probe` (one
    with FETCH_SIZE, one with WRITE_SIZE) into profiles/traffic.json.  The
    copy kernel of known size calibrates each counter's unit."""
    import sqlite3

    def per_kernel(db, counter, key):
        rows = sqlite3.connect(db).execute(
            "select kernel_name, value from counters_collection where counter_name = ?", (counter,)).fetchall()
        copy = [v for n, v in rows if "copyBuffer" in n or "copy" in n.lower()]
        sel = [v for n, v in rows if key in n]
        return max(copy), sum(sel) / len(sel)

    copy_bytes = 256 << 20
    rec = {}
    for name, key, src, alg in (
            ("gemv_decode_set_m1", "gemv_affine_kernel", "gemv_affine.hip", None),
            ("gemm_m2048_n14336_b4", "gemm_affine_kernel<4, 1, 4>", "gemm_affine.hip",
             gemm_bytes(2048, 14336, 4096)),
            ("gemm_prep_m2048_n14336_b4", "prep_kernel<4, 1, 2>", "gemm_affine.hip", None)):
        fc, fg = per_kernel(fetch_db, "FETCH_SIZE", key)
        wc, wg = per_kernel(write_db, "WRITE_SIZE", key)
        f_factor = copy_bytes / (fc * 1024)
        w_factor = copy_bytes / (wc * 1024)
        traffic = fg * 1024 * f_factor + wg * 1024 * w_factor
        rec[name] = {
            "kernel": key, "src_hash": src_hash(src),
            "bytes_per_launch": round(traffic),
            "fetch_kib_per_launch": round(fg, 1), "write_kib_per_launch": round(wg, 1),
            "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
            "calibration": "256 MiB device copy: FETCH_SIZE and WRITE_SIZE of that kernel against 256 MiB",
            "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -- python3 bench.py --traffic-probe"}
        if alg:
            rec[name]["algorithmic_bytes"] = alg
    path = os.path.join(ROOT, "profiles", "traffic.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def summarize(db, filt=""):
    """Markdown table of per-kernel durations (calls, mean, median, p10, p90,
    min; microseconds) from a rocprofv3 --kernel-trace database."""
    import sqlite3
    c = sqlite3.connect(db)
    tables = [r[0] for r in c.execute("select name from sqlite_master where type in ('table', 'view')")]
    tab = "kernels" if "kernels" in tables else [t for t in tables if "kernel" in t][0]
    cols = [r[1] for r in c.execute(f"pragma table_info({tab})")]
    name = "name" if "name" in cols else "kernel_name"
    grid = "grid_x" if "grid_x" in cols else ("grid_size" if "grid_size" in cols else None)
    by = {}
    q = f"select {name}, {grid or 0}, start, end from {tab}"
    for n, gx, a, b in c.execute(q):
        by.setdefault((n, gx), []).append((b - a) / 1000.0)
    print("| kernel | grid (threads) | calls | mean us | median us | p10 us | p90 us | min us |")
    print("|---|---|---|---|---|---|---|---|")
    for (n, gx), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        if filt and filt not in n:
            continue
        v = np.asarray(v)
        short = n.replace("void ", "").replace("qaff::(anonymous namespace)::", "").split("(")[0]
        print(f"| `{short[:90]}` | {gx} | {v.size} | {v.mean():.2f} | {np.median(v):.2f} | "
              f"{np.percentile(v, 10):.2f} | {np.percentile(v, 90):.2f} | {v.min():.2f} |")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--skip-gemv", action="store_true", help="time only the prefill GEMMs (for profiling)")
    ap.add_argument("--traffic-probe", action="store_true", help="short eager run for rocprofv3 --pmc")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write profiles/traffic.json from two --pmc runs of --traffic-probe (no GPU needed)")
    ap.add_argument("--summarize", nargs="+", metavar=("DB", "FILTER"),
                    help="print per-kernel duration percentiles of a rocprofv3 --kernel-trace database (no GPU)")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold per-kernel GEMV figures")
    ap.add_argument("--w4a8-sweep", action="store_true",
                    help="only the W4A8 lowering x tile sweep (checked, then timed) as one JSON line")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return
    if args.summarize:
        summarize(*args.summarize[:2])
        return
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
        for bits in si.CFG2_BITS:
            for N, K in si.CFG2_SHAPES:
                print(json.dumps({"gemm_m2048": time_gemm(torch, qa, si, device, bits, N=N, K=K)}), flush=True)
        print(json.dumps({"w4a8_m2048": time_w4a8(torch, qa, si, device)}), flush=True)
        return
    if args.w4a8_sweep:
        print(json.dumps({"w4a8_sweep": time_w4a8_sweep(torch, qa, si, device)}), flush=True)
        return

    dec = Decode(args, torch, qa, si, device)
    if args.traffic_probe:
        traffic_probe(torch, qa, si, device, dec)
        return

    launches_set = -(-dec.n_linears // PER_LAUNCH)
    ms_set = eager_time(torch, dec.run_set, args.steps, args.warmup)
    gbs_set = dec.bytes_per_step / (ms_set * 1e-3) / 1e9
    print(f"[bench] decode set (grouped, {launches_set} launches): {ms_set*1e3:.1f} us/step, {gbs_set:.0f} GB/s",
          file=sys.stderr, flush=True)
    chain_steps = max(args.steps // 4, 10)  # the GPU clock needs ~100 ms of load to settle
    ms_chain = graph_time(torch, dec.run_chain, chain_steps, args.warmup)
    ms_lin = graph_time(torch, dec.run_per_linear, chain_steps, args.warmup)
    chain = dec.chain_plan()
    ms_chain1 = eager_time(torch, chain, chain_steps, args.warmup)
    chain_timed_out = chain.timed_out()
    chain.close()
    print(f"[bench] decode chain in one launch: {ms_chain1*1e3:.1f} us/step", file=sys.stderr, flush=True)
    print(f"[bench] decode chain (64 launches): {ms_chain*1e3:.1f} us/step; per linear (112 launches): "
          f"{ms_lin*1e3:.1f} us/step", file=sys.stderr, flush=True)

    # cfg0 shape relaunched on the same weights: cache-resident latency figure
    d0 = dec.stack[0][0]
    y0 = torch.empty((1, d0["N"]), dtype=torch.bfloat16, device=device)
    hot = lambda: [qa.qmm_affine(dec.x[2048], d0["w"], d0["s"], d0["b"], G, BITS, out=y0) for _ in range(20)]
    us_hot = graph_time(torch, hot, 20, 5) * 1e3 / 20

    decode_m = [time_decode_m(torch, qa, si, device, dec, M, max(args.steps // 4, 10), args.warmup // 4 + 1)
                for M in (4, 16)]
    for d in decode_m:
        print(f"[bench] decode set M={d['M']}: {d['us_per_step']} us/step, {d['gbs']} GB/s", file=sys.stderr,
              flush=True)
    gptq = [time_gptq(torch, qa, si, device, M) for M in (1, 32)]

    stream = time_stream_read(torch, qa, device)
    print(f"[bench] streaming read: {stream['gbs']} GB/s", file=sys.stderr, flush=True)
    cold = None
    if not args.no_cold:
        shapes = []
        for _, N, K in si.CFG1_LINEARS:
            if (N, K) not in shapes:
                shapes.append((N, K))
        cold = [r for N, K in shapes for r in time_cold_gemv(torch, qa, si, device, N, K)]
        for r in cold:
            print(f"[bench] cold M={r['M']} {r['N']}x{r['K']}: {r['cold_us']} us, {r['cold_gbs']} GB/s "
                  f"(hot {r['hot_us']} us)", file=sys.stderr, flush=True)
    extras = time_extras(torch, qa, si, device, dec)

    gemm = w4a8 = w4a8_shapes = gemm_roofline = None
    if not args.no_gemm:
        gemm = [time_gemm(torch, qa, si, device, bits, N=N, K=K) for bits in si.CFG2_BITS for N, K in si.CFG2_SHAPES]
        w4a8 = time_w4a8(torch, qa, si, device)
        w4a8_shapes = time_w4a8_shapes(torch, qa, si, device)
        for g in gemm:
            print(f"[bench] gemm b{g['bits']}: {g['us_per_call']} us, {g['tflops']} TFLOP/s", file=sys.stderr,
                  flush=True)
        print(f"[bench] w4a8: {w4a8['us_per_call']} us, {w4a8['tops']} TOPS", file=sys.stderr, flush=True)
        g = [r for r in gemm if r["bits"] == 4 and r["N"] == 14336 and r["K"] == 4096][0]
        flops = 2.0 * g["M"] * g["N"] * g["K"]
        gemm_roofline = {"bound": "mfma", "achieved": g["tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": g["frac_of_bf16_peak"],
                         "traffic": load_traffic("gemm_affine.hip", "gemm_m2048_n14336_b4"),
                         "algorithmic_bytes": gemm_bytes(g["M"], g["N"], g["K"]),
                         "kernel": "prep_kernel<4, 1, 2> + gemm_affine_kernel<4, 1, 4> (one qmm_affine call; "
                                   "the achieved figure counts both kernels)",
                         "flops_per_call": flops, "median_call_us": g["us_per_call"]}

    bytes_per_launch = dec.bytes_per_step / launches_set
    avg_launch_us = ms_set * 1e3 / launches_set
    achieved = bytes_per_launch / (avg_launch_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": load_traffic("gemv_affine.hip", "gemv_decode_set_m1"),
                "kernel": "gemv_affine_kernel<4, bf16, M=1> (grouped, 56 linears per launch)",
                "bytes_per_launch": round(bytes_per_launch), "avg_launch_us": round(avg_launch_us, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(dec, args.cpu_seconds)
        cpu["per_config"] = oracle_timings(si)

    out = {
        "metric": METRIC,
        "value": round(gbs_set, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_set, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode GEMV set of a 1B decoder (hidden 2048, FFN 8192) x {args.layers} layers, "
                               "M=1, 4-bit codes, G=64, bf16 scales/biases/activations; every linear once per step "
                               f"through the grouped GEMV ({launches_set} launches per step)",
                   "M": 1, "layers": args.layers, "linears_per_layer": 7, "bits": BITS, "group_size": G,
                   "bytes_per_step": dec.bytes_per_step, "frac_of_hbm_peak": round(gbs_set / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "decode_chain": {"launches_per_step": 4 * args.layers, "us_per_step": round(ms_chain * 1e3, 1),
                         "gbs": round(dec.bytes_per_step / (ms_chain * 1e-3) / 1e9, 1)},
        "decode_chain_one_launch": {"launches_per_step": 1, "stages": 4 * args.layers,
                                    "us_per_step": round(ms_chain1 * 1e3, 1),
                                    "gbs": round(dec.bytes_per_step / (ms_chain1 * 1e-3) / 1e9, 1),
                                    "frac_of_hbm_peak": round(dec.bytes_per_step / (ms_chain1 * 1e-3) / 1e9
                                                              / HBM_PEAK_GBS, 4),
                                    "wait_gave_up": chain_timed_out},
        "per_linear": {"launches_per_step": dec.n_linears, "us_per_step": round(ms_lin * 1e3, 1),
                       "gbs": round(dec.bytes_per_step / (ms_lin * 1e-3) / 1e9, 1)},
        "cfg0_hot": {"us_per_launch": round(us_hot, 2), "gbs_not_hbm": round(gemv_bytes(1, 2048, 2048) / us_hot / 1e3, 1)},
        "stream_read": stream,
        "gemv_cold": cold,
        "gemm_roofline": gemm_roofline,
        **extras,
        "decode_set_multirow": decode_m,
        "gptq_k4096_n11008": gptq,
        "gemm_m2048": gemm,
        "w4a8_m2048": w4a8,
        "w4a8_shapes": w4a8_shapes,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
