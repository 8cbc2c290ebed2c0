"""The paths that use scratch memory (GEMM pre-pass and split-K partials,
GPTQ direct partials, permuted activations) draw it from a per-stream
workspace, so after one eager call they capture into a HIP graph.  Every
replay must reproduce the eager output bit for bit (the kernels are
deterministic), with eager work on the same stream between replays."""
import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import synth_inputs as si
from gpu_util import affine_to_device, dev16, require_gpu

pytestmark = pytest.mark.gpu


def _check_replays(fn, what):
    dev = require_gpu()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ref = fn().clone()  # eager call: sizes the stream's workspace
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            out = fn()
        for i in range(3):
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"{what}: replay {i} differs from the eager result"
            fn()  # eager work on the same stream and workspace between replays
            torch.cuda.synchronize()
    torch.cuda.current_stream().wait_stream(s)
    print(f"[graph] {what}: 3 replays match", flush=True)
    del dev


def test_graph_gemv_with_k_perm():
    dev = require_gpu()
    case = si.affine_case(1, 600, 2048, 64, 4, seed=(50,), name="graph_gemv_kperm")
    case.k_perm = np.random.default_rng(51).permutation(case.K).astype(np.int32)
    x, w, s, b, kp = affine_to_device(case, dev)
    _check_replays(lambda: qa.qmm_affine(x, w, s, b, case.G, 4, k_perm=kp), case.name)


def test_graph_gemm_split_k():
    dev = require_gpu()
    case = si.affine_case(56, 520, 4096, 64, 4, seed=(52,), name="graph_gemm_split")
    x, w, s, b, kp = affine_to_device(case, dev)
    _check_replays(lambda: qa.qmm_affine(x, w, s, b, case.G, 4), case.name)


def test_graph_gptq_direct():
    dev = require_gpu()
    case = si.gptq_case(3, 1024, 400, 128, seed=(53,), name="graph_gptq")
    x = dev16(case.x, "f16", dev)
    qw = torch.from_numpy(np.ascontiguousarray(case.qweight)).to(dev)
    qz = torch.from_numpy(np.ascontiguousarray(case.qzeros)).to(dev)
    sc = dev16(case.scales, "f16", dev)
    gi = torch.from_numpy(np.ascontiguousarray(case.g_idx)).to(dev)
    _check_replays(lambda: qa.qmm_gptq(x, qw, qz, sc, gi, case.G), case.name)


def test_graph_gptq_matrix_core_without_act_order():
    dev = require_gpu()
    case = si.gptq_case(40, 8192, 264, 32, seed=(54,), act_order=False, name="graph_gptq_mfma_slices")
    x = dev16(case.x, "f16", dev)
    qw = torch.from_numpy(np.ascontiguousarray(case.qweight)).to(dev)
    qz = torch.from_numpy(np.ascontiguousarray(case.qzeros)).to(dev)
    sc = dev16(case.scales, "f16", dev)
    _check_replays(lambda: qa.qmm_gptq(x, qw, qz, sc, None, case.G), case.name)


def test_graph_mfma_gemv():
    # M = 8 on the MFMA GEMV with K split in two (nine 64-column workgroups
    # per slice) and the partial sum
    dev = require_gpu()
    case = si.affine_case(8, 520, 2048, 64, 4, seed=(55,), name="graph_mfma_gemv")
    x, w, s, b, kp = affine_to_device(case, dev)
    _check_replays(lambda: qa.qmm_affine(x, w, s, b, case.G, 4), case.name)


@pytest.mark.parametrize("M,N,K", [(8, 1024, 1024), (128, 1024, 4096)])
def test_graph_w4a8(M, N, K):
    # M = 8: the fused quantize + GEMV; M = 128, K = 4096: quantize, split-K
    # GEMM and the partial sum.  The codes, scales and y all replay exactly.
    dev = require_gpu()
    case = si.w4a8_case(M, N, K, seed=(56, M, N, K), name=f"graph_w4a8_M{M}")
    x = dev16(case.x, "f16", dev)
    w = torch.from_numpy(np.ascontiguousarray(case.w_q4).view(np.int32)).to(dev)
    sw = dev16(case.s_w, "f16", dev)

    def call():
        y, xq, sx, _ = qa.qgemm_w4a8(x, w, sw)
        return torch.cat([y.view(torch.int16).flatten().to(torch.int32), xq.flatten().to(torch.int32),
                          sx.view(torch.int32)])
    _check_replays(call, case.name)
