"""The library's scratch: qaff_release_workspaces frees it, and calls made
after a release allocate again and give the same results."""
import ctypes as C

import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import affine_to_device, assert_float_bar, host_f64, require_gpu

pytestmark = pytest.mark.gpu


def test_release_between_calls():
    dev = require_gpu()
    # the GEMM path (pre-pass buffers) and a k_perm GEMV (permuted x) both
    # take scratch from the stream's buffer
    gemm = si.affine_case(40, 300, 1024, 64, 8, seed=(60, 0), name="release_gemm")
    gemv = si.affine_case(3, 200, 2048, 64, 4, seed=(60, 1), name="release_gemv")
    gemv.k_perm = np.random.default_rng(61).permutation(gemv.K).astype(np.int32)
    args = [affine_to_device(c, dev) for c in (gemm, gemv)]
    print("[case] release: GEMM M=40 8-bit, GEMV M=3 with k_perm", flush=True)

    def run():
        out = []
        for c, (x, w, s, b, kp) in zip((gemm, gemv), args):
            out.append(qa.qmm_affine(x, w, s, b, c.G, c.bits, k_perm=kp))
        torch.cuda.synchronize()
        return [host_f64(y) for y in out]

    first = run()
    freed = qa.release_workspaces()
    assert freed > 0
    again = qa.release_workspaces()  # nothing left to free
    assert again == 0
    second = run()
    for c, a, b in zip((gemm, gemv), first, second):
        np.testing.assert_array_equal(a, b)
        assert_float_bar(b, oracle.qmm_affine_case(c), c.name)
    qa.release_workspaces()
