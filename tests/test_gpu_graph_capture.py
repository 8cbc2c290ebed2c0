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
    case = si.affine_case(48, 520, 4096, 64, 4, seed=(52,), name="graph_gemm_split")
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
