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
    # K % 64 != 0 (G = 32): served by the GEMV kernel on 16-row slices
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


@pytest.mark.parametrize("bits", si.CFG2_BITS)
def test_cfg2_full_compare(bits):
    # one whole prefill shape per bit width, every output against the oracle
    N, K = 1024, 4096
    case = si.cfg2_case(N, K, bits, seed=(2, N, K))
    y = _run(case)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name + "_full")


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("M", [17, 70])
def test_k_equals_group(bits, G, M):
    # one group per row: K = G (K = 32 at 2 bits is a row of 8 bytes, the
    # GEMV's tail path; K = 64 and 128 are whole GEMM K tiles)
    case = si.affine_case(M, 136, G, G, bits, seed=(28, bits, G, M), scale_range=(0.002, 0.01),
                          name=f"gemm_K_eq_G{G}_b{bits}_M{M}")
    y = _run(case)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_scales_spanning_2_pow_22_in_a_row(bits):
    # Each row's scales spread over 2^22: groups 0-7 within 2^-6 of the row's
    # largest (group 0), groups 8-63 between 2^-22 and 2^-15 of it
    # (log-uniform), below fp16's normal range if the largest were brought
    # to 1.  x is zero over groups 0-7, so every output comes from the small
    # scales alone.  The kernel's fp16 scale pieces keep them exact
    # (scales down to 2^-(14+ESHIFT) of the row's largest are normal fp16
    # numbers), so against each row's largest output the error is the f16
    # rounding of y (2^-11) and fp32 sums: bounded here by 2e-3.  Pieces
    # rounded as subnormals (the row's largest scale brought to 1) miss it.
    M, N, K, G = 80, 96, 2048, 32
    case = si.affine_case(M, N, K, G, bits, seed=(29, bits), act_dtype="f16", name=f"gemm_wide_scales_b{bits}")
    r = np.random.default_rng((29, bits, 1))
    ng = K // G
    e = np.concatenate([r.uniform(-6.0, 0.0, size=(N, 8)), r.uniform(-22.0, -15.0, size=(N, ng - 8))], axis=1)
    e[:, 0] = 0.0
    s32 = (4.0 * np.exp2(e)).astype(np.float32)
    case.scales = si.bf16_bits(s32)
    sb = si.bits_to_f32(case.scales, "bf16")
    case.biases = si.bf16_bits((-(2 ** (bits - 1)) * sb).astype(np.float32))
    xf = si.bits_to_f32(case.x, "f16").copy()
    xf[:, :8 * G] = 0.0
    case.x = si.store(xf, "f16")
    y = host_f64(_run(case))
    ref = oracle.qmm_affine_case(case)
    worst = 0.0
    for m in range(M):
        sc = max(np.abs(ref[m]).max(), 1e-300)
        assert_float_bar(y[m] / sc, ref[m] / sc, f"{case.name}_row{m}")
        worst = max(worst, float(np.abs(y[m] - ref[m]).max() / sc))
    print(f"[parity] {case.name} worst error / row max = {worst:.3e}", flush=True)
    assert worst <= 2e-3, worst


def test_padded_rows_offset_guard():
    # M = 17 with 2-bit codes at K = 64 runs the GEMM with 64-row tiles: the
    # padded rows' y offsets (Mp*N*2 bytes) pass 2^31 although M*N*2 does
    # not, so the call must be refused, not wrap around into valid rows
    dev = require_gpu()
    M, N, K, G, bits = 17, 20_000_000, 64, 64, 2
    assert M * N * 2 < 2 ** 31 <= 64 * N * 2
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((N, K * bits // 32), dtype=torch.int32, device=dev)
    s = torch.zeros((N, K // G), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    print("[case] padded-row guard M=17 N=2e7 K=64 2-bit", flush=True)
    with pytest.raises(qa.QaffError) as ei:
        qa.qmm_affine(x, w, s, s, G, bits, out=y)
    torch.cuda.synchronize()
    assert ei.value.status == 2, str(ei.value)   # QAFF_E_UNSUPPORTED


@pytest.mark.parametrize("K,G,bits", [(17408, 32, 4), (8704, 32, 8), (8192, 64, 2), (16384, 128, 4)])
def test_prepass_row_lengths(K, G, bits):
    # the pre-pass holds a row of x in registers up to K = 16384 and reads it
    # twice past that (17408); W rows take every scale and bias load at once
    # up to 256 groups and a loop past that (G = 32 at K = 8704, 17408)
    case = si.affine_case(70, 264, K, G, bits, seed=(23, K, G, bits), scale_range=(0.002, 0.01),
                          name=f"gemm_prepass_K{K}_G{G}_b{bits}")
    y = _run(case)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_prepass_row_maximum_special_rows(act):
    # rows whose maximum |x| the pre-pass takes on the raw bits: a NaN (left
    # out of the maximum; the row's outputs are all NaN on both sides), a
    # maximum near the dtype's top, subnormals only (their scale 2^-e is
    # past fp32's range for bf16), all zeros, and negative zeros
    M, N, K, G = 70, 130, 1024, 64
    case = si.affine_case(M, N, K, G, 4, seed=(24, act == "f16"), act_dtype=act, scale_range=(0.002, 0.004),
                          name=f"gemm_rowmax_{act}")
    xf = si.bits_to_f32(case.x, act).astype(np.float64).reshape(M, K)
    big = 65504.0 / 64 if act == "f16" else 3.0e36
    tiny = 2.0 ** -20 if act == "f16" else 2.0 ** -130
    xf[3, 5] = np.nan
    xf[10, :] *= big / np.abs(xf[10]).max()       # the row's maximum at the dtype's top
    xf[20, :] = tiny * np.sign(xf[20])             # subnormal values only
    xf[30, :] = 0.0
    xf[40, :] = -0.0
    case.x = si.store(xf.astype(np.float32), act).reshape(case.x.shape)
    y = host_f64(_run(case))
    ref = oracle.qmm_affine_case(case)
    assert np.isnan(y[3]).all() and np.isnan(ref[3]).all()
    keep = np.ones(M, bool)
    keep[3] = False
    assert_float_bar(y[keep], ref[keep], case.name)
    assert (y[30] == 0).all() and (y[40] == 0).all()


@pytest.mark.parametrize("bits", [4, 8])
def test_long_k_split_of_256_row_tiles(bits):
    # From K = 8192, 256-row tiles that fill half the CUs take K in two
    # splits (fp32 partials, then the summing pass): M = 2048, N = 3072 gives
    # 8 x 12 = 96 tiles.  Every column of 40 rows (tile edges included).
    M, N, K = 2048, 3072, 8192
    case = si.affine_case(M, N, K, 64, bits, seed=(25, bits), scale_range=(0.002, 0.01),
                          name=f"gemm_longk_split_b{bits}")
    y = _run(case)
    rows = np.unique(np.concatenate([si.sample_indices(M, 32, seed=(25, 1, bits)),
                                     np.array([0, 255, 256, 1023, 1024, 1791, 1792, 2047])])).astype(np.int64)
    cols = np.arange(N, dtype=np.int64)
    ysub = host_f64(y[torch.from_numpy(rows).to(y.device)])
    assert_float_bar(ysub, oracle.qmm_affine_case(case, rows=rows, cols=cols), case.name)
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("M", [512, 500])
@pytest.mark.parametrize("bits", [2, 4])
def test_256_row_tiles_wide_n(M, bits):
    # 256-row tiles without a K split: M = 512 (500: a ragged last row tile)
    # x N = 24576 is 192 of them.  Every column of 40 rows, edges of the
    # 128- and 256-row blocks included.
    N, K = 24576, 1024
    case = si.affine_case(M, N, K, 64, bits, seed=(26, M, bits), scale_range=(0.002, 0.01),
                          name=f"gemm_wide_M{M}_b{bits}")
    y = _run(case)
    rows = np.unique(np.concatenate([si.sample_indices(M, 32, seed=(26, 1, M)),
                                     np.array([0, 127, 128, 255, 256, 383, 384, M - 1])])).astype(np.int64)
    ysub = host_f64(y[torch.from_numpy(rows).to(y.device)])
    assert_float_bar(ysub, oracle.qmm_affine_case(case, rows=rows, cols=np.arange(N, dtype=np.int64)), case.name)
    assert torch.isfinite(y.float()).all()


@pytest.mark.parametrize("bits", [4, 8])
def test_xcd_tile_rectangles_ragged(bits):
    # Without a K split, a tile grid divisible 4 x 2 is dealt to the XCDs as
    # rectangles: M = 1000, N = 12200 is 4 x 48 tiles of 256 x 256, with a
    # ragged last row tile (768..999) and a ragged last column tile.  Every
    # column of 40 rows, tile edges included.
    M, N, K = 1000, 12200, 1024
    case = si.affine_case(M, N, K, 64, bits, seed=(27, bits), scale_range=(0.002, 0.01),
                          name=f"gemm_rect_b{bits}")
    y = _run(case)
    rows = np.unique(np.concatenate([si.sample_indices(M, 32, seed=(27, 1, bits)),
                                     np.array([0, 255, 256, 511, 512, 767, 768, 999])])).astype(np.int64)
    ysub = host_f64(y[torch.from_numpy(rows).to(y.device)])
    assert_float_bar(ysub, oracle.qmm_affine_case(case, rows=rows, cols=np.arange(N, dtype=np.int64)), case.name)
    assert torch.isfinite(y.float()).all()
