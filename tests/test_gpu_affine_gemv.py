"""GPU parity of the affine decode GEMV (M <= 16) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import affine_to_device, assert_float_bar, host_f64, require_gpu

pytestmark = pytest.mark.gpu


def _run(case, fn=qa.qmm_affine):
    dev = require_gpu()
    x, w, s, b, kp = affine_to_device(case, dev)
    print(f"[case] {case.name} M={case.M} N={case.N} K={case.K} G={case.G} bits={case.bits} "
          f"act={case.act_dtype} s={case.sb_dtype} b={case.bias_dtype} kperm={case.k_perm is not None}", flush=True)
    y = fn(x, w, s, b, case.G, case.bits, k_perm=kp)
    torch.cuda.synchronize()
    return host_f64(y)


def test_cfg0_single_linear():
    case = si.cfg0_case()
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), "cfg0")


@pytest.mark.parametrize("M", si.CFG1_M)
@pytest.mark.parametrize("name,N,K", si.CFG1_LINEARS[:1] + si.CFG1_LINEARS[1:2] + si.CFG1_LINEARS[4:5] + si.CFG1_LINEARS[6:])
def test_cfg1_decode_set(name, N, K, M):
    case = si.cfg1_case(N, K, M, seed=(1, N, K, M))
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_small_all_widths_groups_dtypes(bits, G, act):
    # ragged N (not a multiple of any row tile), several K chunks and a chunk tail
    case = si.affine_case(3, 77, 2560 if bits != 2 else 2560, G, bits, seed=(5, bits, G), act_dtype=act,
                          name=f"small_b{bits}_G{G}_{act}")
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("sdt,bdt", [("f16", "f16"), ("f32", "f32"), ("f16", "f32"), ("bf16", "f32")])
def test_scale_bias_dtypes(sdt, bdt):
    case = si.affine_case(2, 130, 1024, 64, 4, seed=(6,), sb_dtype=sdt, name=f"sb_{sdt}_{bdt}")
    if bdt != sdt:
        case.biases = si.store(si.bits_to_f32(case.biases, sdt), bdt)
        case.bias_dtype = bdt
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("M", [1, 5, 16])
def test_k_perm_gather(M):
    case = si.affine_case(M, 96, 4096, 128, 4, seed=(7, M), act_dtype="f16", name=f"kperm_M{M}")
    case.k_perm = np.random.default_rng(8).permutation(case.K).astype(np.int32)
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 16])
def test_gemv_every_m_boundary(M):
    case = si.affine_case(M, 264, 2048, 64, 4, seed=(9, M), name=f"gemv_M{M}")
    y = _run(case, qa.qgemv_affine)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


def test_extreme_codes_all_zero_and_all_max():
    for word in (0x00000000, 0xFFFFFFFF):
        case = si.affine_case(2, 64, 1024, 64, 4, seed=(10,), name=f"codes_{word:#x}")
        case.packed[:] = np.uint32(word)
        y = _run(case)
        assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


def test_long_rows_k14336():
    case = si.affine_case(1, 200, 14336, 64, 4, seed=(11,), name="k14336")
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


def test_short_rows_smaller_than_a_wave():
    # K*bits/128 < 64: part of each wave idles
    for bits, K in ((4, 256), (8, 96), (2, 512)):
        case = si.affine_case(2, 40, K, 32, bits, seed=(12, bits), name=f"short_b{bits}_K{K}")
        y = _run(case)
        assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


def test_output_not_written_past_n():
    dev = require_gpu()
    case = si.affine_case(2, 70, 512, 64, 4, seed=(13,))
    x, w, s, b, _ = affine_to_device(case, dev)
    out = torch.full((2 * 70 + 64,), 7.0, dtype=torch.bfloat16, device=dev)
    qa.qmm_affine(x, w, s, b, 64, 4, out=out[: 2 * 70].view(2, 70))
    torch.cuda.synchronize()
    assert torch.all(out[2 * 70:] == 7.0)
