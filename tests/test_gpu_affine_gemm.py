"""GPU parity of the affine prefill GEMM path (M > 16) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import affine_to_device, assert_float_bar, host_f64, require_gpu

pytestmark = pytest.mark.gpu


def _run(case):
    dev = require_gpu()
    x, w, s, b, kp = affine_to_device(case, dev)
    print(f"[case] {case.name} M={case.M} N={case.N} K={case.K} G={case.G} bits={case.bits} act={case.act_dtype} "
          f"s={case.sb_dtype} b={case.bias_dtype} kperm={case.k_perm is not None}", flush=True)
    y = qa.qmm_affine(x, w, s, b, case.G, case.bits, k_perm=kp)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("bits", si.CFG2_BITS)
@pytest.mark.parametrize("N,K", si.CFG2_SHAPES)
def test_cfg2_prefill_sampled(N, K, bits):
    # full-size run; the oracle recomputes a sample of rows and columns
    case = si.cfg2_case(N, K, bits, seed=(2, N, K))
    y = _run(case)
    rows = si.sample_indices(case.M, 24, seed=(2, 1, N))
    cols = si.sample_indices(N, 160, seed=(2, 2, N))
    ysub = host_f64(y[torch.from_numpy(rows).to(y.device)][:, torch.from_numpy(cols).to(y.device)])
    assert_float_bar(ysub, oracle.qmm_affine_case(case, rows=rows, cols=cols), case.name)
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_small_full_compare(bits, G):
    case = si.affine_case(70, 300, 1024, G, bits, seed=(20, bits, G), scale_range=(0.002, 0.01),
                          name=f"gemm_b{bits}_G{G}")
    y = _run(case)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("M", [17, 32, 48, 49, 64, 65, 255, 257])
def test_m_boundaries_and_tiles(M):
    # M <= 48 (4-bit, MFMA-eligible) runs as 16-row slices on the MFMA GEMV
    # (M = 17: a slice of 16 and one of 1); from 49 the GEMM's 64-, 128- and
    # 256-row tiles, each M at or just past a tile edge
    case = si.affine_case(M, 264, 2048, 64, 4, seed=(21, M), name=f"gemm_M{M}")
    y = _run(case)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("sdt,bdt", [("f16", "f16"), ("f32", "f32"), ("f16", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("bits", [4, 8])
def test_scale_bias_dtypes(sdt, bdt, bits):
    case = si.affine_case(40, 130, 1024, 64, bits, seed=(22, bits), sb_dtype=sdt, name=f"gemm_sb_{sdt}_{bdt}_b{bits}")
    if bdt != sdt:
        case.biases = si.store(si.bits_to_f32(case.biases, sdt), bdt)
        case.bias_dtype = bdt
    y = _run(case)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_k_perm_and_activation_dtype(act):
    case = si.affine_case(72, 256, 4096, 128, 4, seed=(23,), act_dtype=act, name=f"gemm_kperm_{act}")
    case.k_perm = np.random.default_rng(24).permutation(case.K).astype(np.int32)
    y = _run(case)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("M,act", [(40, "f16"), (24, "bf16")])
def test_row_slices_with_k_perm(M, act):
    # M <= 48 on 16-row slices of the MFMA GEMV: each slice permutes its own
    # rows of x, and N = 256 gives a narrow grid, so K is split as well
    case = si.affine_case(M, 256, 4096, 128, 4, seed=(24, M), act_dtype=act, name=f"slices_kperm_M{M}_{act}")
    case.k_perm = np.random.default_rng(24).permutation(case.K).astype(np.int32)
    y = _run(case)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name)


def test_wide_dynamic_range_rows():
    # rows of x at very different magnitudes (the per-row power-of-two scaling
    # keeps fp16 operands in range), including an all-zero row
    case = si.affine_case(36, 200, 512, 64, 8, seed=(25,), name="gemm_range")
    xf = si.bits_to_f32(case.x, "bf16").copy()
    xf[1] *= 1e25
    xf[2] *= 1e-20
    xf[3] = 0.0
    xf[4, ::7] *= 3e4
    case.x = si.bf16_bits(xf)
    y = _run(case)
    ref = oracle.qmm_affine_case(case)
    for m in range(case.M):   # relative bar row by row (rows differ by 1e45)
        scale = max(np.abs(ref[m]).max(), 1e-300)
        assert_float_bar(host_f64(y)[m] / scale, ref[m] / scale, f"row{m}")


def test_k_not_multiple_of_tile():
    # K % 64 != 0 (G = 32): served by the GEMV kernel in 4-row chunks
    case = si.affine_case(20, 96, 160, 32, 4, seed=(26,), name="gemm_k160")
    y = _run(case)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("M,N,K,bits", [(40, 100, 4160, 4), (33, 520, 1024, 8), (300, 1100, 2048, 2)])
def test_split_k_partials(M, N, K, bits):
    # few tiles: K is split over workgroups (65 K tiles into 13 splits of 5
    # for the first shape) and the fp32 partials are summed by a second kernel
    case = si.affine_case(M, N, K, 64, bits, seed=(27, M, N, K), name=f"gemm_split_M{M}_N{N}_K{K}_b{bits}")
    y = _run(case)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name)
