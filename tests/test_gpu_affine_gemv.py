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


def _grouped(cases, share_x=False):
    dev = require_gpu()
    probs = []
    x_shared = None
    for c in cases:
        x, w, s, b, kp = affine_to_device(c, dev)
        if share_x:
            x_shared = x if x_shared is None else x_shared
            x = x_shared
        probs.append((x, w, s, b, kp))
    c0 = cases[0]
    print(f"[case] grouped count={len(cases)} M={c0.M} bits={c0.bits} G={c0.G} act={c0.act_dtype} "
          f"shapes={[(c.N, c.K) for c in cases][:8]}", flush=True)
    ys = qa.qgemv_affine_grouped(probs, c0.G, c0.bits)
    torch.cuda.synchronize()
    return [host_f64(y) for y in ys]


@pytest.mark.parametrize("M", si.CFG1_M)
def test_grouped_decode_layer(M):
    # the seven linears of one decoder layer in one call, q/k/v and gate/up style sharing of x
    cases = [si.cfg1_case(N, K, M, seed=(20, i, N, K, M)) for i, (_, N, K) in enumerate(si.CFG1_LINEARS)]
    ys = _grouped(cases)
    for c, y in zip(cases, ys):
        assert_float_bar(y, oracle.qmm_affine_case(c), "grouped_" + c.name)


def test_grouped_shared_x():
    cases = [si.cfg1_case(N, 2048, 1, seed=(21, N)) for N in (2048, 512, 512)]
    for c in cases[1:]:
        c.x = cases[0].x
    ys = _grouped(cases, share_x=True)
    for c, y in zip(cases, ys):
        assert_float_bar(y, oracle.qmm_affine_case(c), "shared_x_" + c.name)


@pytest.mark.parametrize("bits,act", [(4, "bf16"), (8, "f16"), (2, "bf16")])
def test_grouped_many_problems_span_launches(bits, act):
    # more problems than one launch's descriptor table, ragged N, mixed K and one empty problem
    rng = np.random.default_rng(22)
    cases = []
    for i in range(41):
        N = 0 if i == 17 else int(rng.integers(1, 300))
        K = int(rng.choice([256, 512, 2048, 4096]))
        cases.append(si.affine_case(3, N, K, 64, bits, seed=(23, i), act_dtype=act, name=f"g{i}_N{N}_K{K}"))
    ys = _grouped(cases)
    for c, y in zip(cases, ys):
        if c.N == 0:
            assert y.shape == (3, 0)
            continue
        assert_float_bar(y, oracle.qmm_affine_case(c), c.name)


def test_grouped_with_k_perm_and_plain_mixed():
    cases = [si.affine_case(5, 120, 4096, 128, 4, seed=(24, i), act_dtype="f16", name=f"kp{i}") for i in range(3)]
    cases[1].k_perm = np.random.default_rng(25).permutation(4096).astype(np.int32)
    ys = _grouped(cases)
    for c, y in zip(cases, ys):
        assert_float_bar(y, oracle.qmm_affine_case(c), c.name)


@pytest.mark.parametrize("bits,act", [(4, "bf16"), (8, "f16"), (2, "bf16")])
def test_grouped_large_launch(bits, act):
    # one grouped launch with >= 64 MiB of weights at M = 1 (the headline's
    # launch size); ragged N and a K that splits across waves are mixed in
    shapes = [(8192, 2048)] * (8 if bits == 4 else (4 if bits == 8 else 16)) + [(1001, 4096), (300, 8192)]
    cases = [si.affine_case(1, N, K, 64, bits, seed=(26, i, bits), act_dtype=act, name=f"big{i}_N{N}_K{K}")
             for i, (N, K) in enumerate(shapes)]
    assert sum(c.N * c.K * bits // 8 for c in cases) >= 64 << 20
    ys = _grouped(cases)
    for c, y in zip(cases, ys):
        assert_float_bar(y, oracle.qmm_affine_case(c), c.name)


@pytest.mark.parametrize("K", [2048, 4096, 8192])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_4bit_m1_rows_split_over_waves(K, G, act):
    # rows of 1, 2 and 4 KiB: K split over 1, 2 or 4 waves of a workgroup;
    # ragged N leaves a partly filled last workgroup
    case = si.affine_case(1, 333, K, G, 4, seed=(27, K, G), act_dtype=act, name=f"m1_K{K}_G{G}_{act}")
    y = _run(case, qa.qgemv_affine)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


def test_grouped_mixed_k_m1():
    cases = [si.affine_case(1, N, K, 64, 4, seed=(28, i), name=f"mix{i}_N{N}_K{K}")
             for i, (N, K) in enumerate([(512, 2048), (77, 8192), (2048, 4096), (5, 2048), (1000, 8192)])]
    ys = _grouped(cases)
    for c, y in zip(cases, ys):
        assert_float_bar(y, oracle.qmm_affine_case(c), c.name)


@pytest.mark.parametrize("K", [512, 1536, 2560, 8192])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("M", [2, 9, 16])
def test_4bit_several_rows_matrix_core_path(K, G, M, act):
    # 4-bit codes with 2..16 x rows and K a multiple of 512 take the MFMA
    # kernel (at M <= 4 only with 128 or more 64-column workgroups: M = 2
    # here runs the dot2 kernel): 1, 3, 5 and 16 stages of 512 codes (5
    # leaves the last round of three with an empty stage), ragged N leaves a
    # partly filled 64-column tile
    case = si.affine_case(M, 333, K, G, 4, seed=(29, K, G, M), act_dtype=act, name=f"mfma_M{M}_K{K}_G{G}_{act}")
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("M,N,K,G,act", [(2, 8200, 512, 64, "bf16"), (3, 8250, 1536, 32, "f16"),
                                        (4, 8192, 2560, 128, "bf16"), (4, 8130, 512, 64, "f16")])
def test_4bit_few_rows_matrix_core_path_wide(M, N, K, G, act):
    # M <= 4 takes the MFMA kernel once N gives 128 or more 64-column
    # workgroups: exactly 128 (N = 8130, the last one ragged) and a few more
    case = si.affine_case(M, N, K, G, 4, seed=(37, M, N, K), act_dtype=act, name=f"mfma_wide_M{M}_N{N}_K{K}")
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("sdt,bdt", [("f32", "f32"), ("f16", "f32"), ("bf16", "bf16")])
@pytest.mark.parametrize("G", [32, 128])
def test_matrix_core_path_scale_bias_dtypes(sdt, bdt, G):
    case = si.affine_case(16, 200, 1024, G, 4, seed=(30, G), sb_dtype=sdt, name=f"mfma_sb_{sdt}_{bdt}_G{G}")
    if bdt != sdt:
        case.biases = si.store(si.bits_to_f32(case.biases, sdt), bdt)
        case.bias_dtype = bdt
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


def test_matrix_core_path_extreme_codes():
    # all codes 0 or all 15 over long rows: the offset values 128 + q (bf16)
    # and 1024 + q (f16) must cancel against the group sums of x accurately
    for act in ("bf16", "f16"):
        for word in (0x00000000, 0xFFFFFFFF):
            case = si.affine_case(16, 130, 8192, 64, 4, seed=(31,), act_dtype=act, name=f"mfma_{act}_{word:#x}")
            case.packed[:] = np.uint32(word)
            y = _run(case)
            assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("K", [128, 384, 2112])
def test_several_rows_k_not_multiple_of_512(K):
    # the MFMA kernel needs whole 512-code stages; the dot2 kernel runs
    case = si.affine_case(8, 100, K, 64, 4, seed=(32, K), name=f"m8_K{K}")
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("M", [1, 2, 9, 16])
def test_k_perm_every_width_and_kernel(bits, M):
    # the permuted copy of x feeds the scalar kernel (M = 1, 2- and 8-bit
    # codes, and M = 2 at this N) and the matrix-core kernel (4-bit, M = 9
    # and 16, K % 512 == 0)
    case = si.affine_case(M, 200, 2048, 64, bits, seed=(34, bits, M), name=f"kperm_b{bits}_M{M}")
    case.k_perm = np.random.default_rng(35).permutation(case.K).astype(np.int32)
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


def test_grouped_k_perm_shared_and_distinct():
    # problems 0, 1 and 3 share one x tensor and one permutation tensor (one
    # permuted copy serves them); 2 shares x with another permutation; 4 has
    # its own x and K
    dev = require_gpu()
    K = 1024
    base = si.affine_case(4, 72, K, 64, 4, seed=(36,), name="kp_shared")
    perm_a = np.random.default_rng(37).permutation(K).astype(np.int32)
    perm_b = np.random.default_rng(38).permutation(K).astype(np.int32)
    cases = [si.affine_case(4, N, K, 64, 4, seed=(39, i), name=f"kp_shared{i}") for i, N in enumerate((72, 40, 96, 8))]
    for c, p in zip(cases, (perm_a, perm_a, perm_b, perm_a)):
        c.x = base.x
        c.k_perm = p
    other = si.affine_case(4, 56, 2048, 64, 4, seed=(40,), name="kp_other")
    other.k_perm = np.random.default_rng(41).permutation(2048).astype(np.int32)
    cases.append(other)
    x0 = None
    kp_dev = {}
    probs = []
    for c in cases:
        x, w, s, b, kp = affine_to_device(c, dev)
        if c.x is base.x:
            x0 = x if x0 is None else x0
            x = x0
            kp = kp_dev.setdefault(id(c.k_perm), kp)
        probs.append((x, w, s, b, kp))
    print(f"[case] grouped k_perm shared/distinct count={len(cases)}", flush=True)
    ys = qa.qgemv_affine_grouped(probs, 64, 4)
    torch.cuda.synchronize()
    for c, y in zip(cases, ys):
        assert_float_bar(host_f64(y), oracle.qmm_affine_case(c), c.name)


# Rows that are not whole 16-byte chunks: 2-bit codes, G = 32, K an odd
# multiple of 32 (K*bits % 128 != 0).  They run the plain tail kernel, for
# M <= 16 directly and for larger M in 16-row slices.
@pytest.mark.parametrize("K", [32, 96, 160, 1056])
@pytest.mark.parametrize("M", [1, 5, 16, 33])
def test_ragged_rows_two_bit(K, M):
    case = si.affine_case(M, 70, K, 32, 2, seed=(40, K, M), name=f"ragged_b2_K{K}_M{M}")
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("act,sdt", [("f16", "f16"), ("bf16", "f32")])
def test_ragged_rows_dtypes_and_k_perm(act, sdt):
    case = si.affine_case(4, 33, 224, 32, 2, seed=(41,), act_dtype=act, sb_dtype=sdt, name=f"ragged_{act}_{sdt}")
    case.k_perm = np.random.default_rng(42).permutation(case.K).astype(np.int32)
    y = _run(case)
    assert_float_bar(y, oracle.qmm_affine_case(case), case.name)


def test_ragged_rows_in_a_grouped_call():
    # a ragged problem between two regular ones: each output as alone
    dev = require_gpu()
    cases = [si.affine_case(2, 64, 2048, 32, 2, seed=(43, 0), name="regular0"),
             si.affine_case(2, 40, 96, 32, 2, seed=(43, 1), name="ragged"),
             si.affine_case(2, 48, 1024, 32, 2, seed=(43, 2), name="regular2")]
    probs = [affine_to_device(c, dev)[:4] for c in cases]
    ys = qa.qgemv_affine_grouped(probs, 32, 2)
    torch.cuda.synchronize()
    for c, y in zip(cases, ys):
        assert_float_bar(host_f64(y), oracle.qmm_affine_case(c), "grouped " + c.name)
