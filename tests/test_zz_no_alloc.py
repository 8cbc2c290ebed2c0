"""qmm_affine_noalloc through the C ABI: the same bits as qmm_affine, on two
calls in a row (the second smaller), for the GEMM path and for a GEMV with
k_perm (both take scratch), and a clear error past the array's size."""
import ctypes as C

import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import affine_to_device, assert_float_bar, host_f64, require_gpu

pytestmark = pytest.mark.gpu

UNSUP = 2


def _call(fn, case, dev, out):
    x, w, s, b, kp = affine_to_device(case, dev)
    L = qa.lib()
    st = getattr(L, fn)(x.data_ptr(), w.data_ptr(), s.data_ptr(), b.data_ptr(), None if kp is None else kp.data_ptr(),
                        out.data_ptr(), case.M, case.N, case.K, case.G, case.bits, qa.DTYPE[x.dtype],
                        qa.DTYPE[s.dtype], qa.DTYPE[b.dtype], torch.cuda.current_stream().cuda_stream)
    return st


def _pair(case, dev):
    print(f"[case] noalloc {case.name} M={case.M} N={case.N} K={case.K} bits={case.bits} "
          f"kperm={case.k_perm is not None}", flush=True)
    y_ref = torch.full((case.M, case.N), float("nan"), dtype=torch.bfloat16, device=dev)
    y_na = torch.full((case.M, case.N), float("nan"), dtype=torch.bfloat16, device=dev)
    assert _call("qmm_affine", case, dev, y_ref) == 0
    assert _call("qmm_affine_noalloc", case, dev, y_na) == 0, qa.lib().qaff_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16))
    assert_float_bar(host_f64(y_na), oracle.qmm_affine_case(case), "noalloc " + case.name)


def test_gemm_then_smaller_gemm():
    dev = require_gpu()
    _pair(si.affine_case(300, 1000, 2048, 64, 4, seed=(110, 0), name="gemm_big"), dev)
    _pair(si.affine_case(40, 520, 1024, 32, 8, seed=(110, 1), name="gemm_small"), dev)


def test_gemv_with_k_perm_then_smaller():
    dev = require_gpu()
    c1 = si.affine_case(9, 700, 4096, 128, 4, seed=(111, 0), name="gemv_kperm_big")
    c1.k_perm = np.random.default_rng(112).permutation(c1.K).astype(np.int32)
    c2 = si.affine_case(3, 200, 1024, 64, 4, seed=(111, 1), name="gemv_kperm_small")
    c2.k_perm = np.random.default_rng(113).permutation(c2.K).astype(np.int32)
    _pair(c1, dev)
    _pair(c2, dev)


def test_scratch_beyond_the_array_is_rejected():
    dev = require_gpu()
    # M = 4096, K = 8192: the pre-pass copy of x alone is 64 MiB
    M, N, K = 4096, 256, 8192
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((N, K // 8), dtype=torch.int32, device=dev)
    s = torch.zeros((N, K // 64), dtype=torch.bfloat16, device=dev)
    y = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
    print("[case] noalloc too large", flush=True)
    st = qa.lib().qmm_affine_noalloc(x.data_ptr(), w.data_ptr(), s.data_ptr(), s.data_ptr(), None, y.data_ptr(),
                                     M, N, K, 64, 4, 0, 0, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == UNSUP
    assert "scratch" in qa.lib().qaff_last_error().decode()
    # and the entry point still works afterwards
    _pair(si.affine_case(64, 256, 1024, 64, 4, seed=(114,), name="after_reject"), dev)
