"""Seeded random shapes across every affine path (GEMV, MFMA GEMV, row
slices, GEMM with and without split K), bit widths, group sizes, dtypes and
k_perm, each against the fp64 oracle at every output.  Shapes are drawn so
that each case runs in well under a second on the oracle."""
import numpy as np
import pytest

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import affine_to_device, assert_float_bar, host_f64, require_gpu

pytestmark = pytest.mark.gpu

N_CASES = 40


def _draw(i):
    r = np.random.default_rng((60, i))
    bits = int(r.choice([2, 4, 8]))
    G = int(r.choice([32, 64, 128]))
    # K: whole groups; sometimes not a whole 64-code K tile or 512-code stage
    K = G * int(r.integers(1, 48 if G == 32 else (24 if G == 64 else 12)))
    M = int(r.choice([1, 2, 3, 5, 8, 13, 16, 17, 31, 48, 49, 64, 100, 150, 257]))
    N = int(r.integers(1, 80)) * 8 + int(r.choice([0, 0, 0, 3, 5]))  # mostly N % 8 == 0
    act = str(r.choice(["bf16", "f16"]))
    sdt = str(r.choice(["bf16", "f16", "f32"]))
    kperm = bool(r.random() < 0.25)
    return bits, G, K, M, N, act, sdt, kperm


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_affine_shape(i):
    bits, G, K, M, N, act, sdt, kperm = _draw(i)
    dev = require_gpu()
    case = si.affine_case(M, N, K, G, bits, seed=(61, i), act_dtype=act, sb_dtype=sdt,
                          scale_range=(0.002, 0.02), name=f"rand{i}_M{M}_N{N}_K{K}_G{G}_b{bits}_{act}_{sdt}")
    if kperm:
        case.k_perm = np.random.default_rng((62, i)).permutation(K).astype(np.int32)
    x, w, s, b, kp = affine_to_device(case, dev)
    print(f"[case] {case.name} kperm={kperm}", flush=True)
    y = qa.qmm_affine(x, w, s, b, G, bits, k_perm=kp)
    assert_float_bar(host_f64(y), oracle.qmm_affine_case(case), case.name)


@pytest.mark.parametrize("i", range(20))
def test_random_w4a8_shape(i):
    # codes, scales and int32 sums exact at every output; both lowerings at a
    # random tile when M > 16
    import torch
    from gpu_util import dev16
    r = np.random.default_rng((63, i))
    M = int(r.choice([1, 4, 9, 16, 17, 40, 129, 300]))
    N = int(r.integers(1, 96)) * 8 + int(r.choice([0, 0, 1, 7]))
    K = 32 * int(r.integers(1, 80))
    case = si.w4a8_case(M, N, K, seed=(64, i), name=f"w4a8_rand{i}_M{M}_N{N}_K{K}")
    dev = require_gpu()
    x = dev16(case.x, "f16", dev)
    w = torch.from_numpy(np.ascontiguousarray(case.w_q4).view(np.int32)).to(dev)
    sw = dev16(case.s_w, "f16", dev)
    print(f"[case] {case.name}", flush=True)
    if M > 16:
        bm, bn = [(32, 128), (64, 128), (64, 256), (128, 256)][int(r.integers(0, 4))]
        y, xq, sx, acc = qa.qgemm_w4a8_tiled(x, w, sw, bool(r.integers(0, 2)), bm, bn, want_acc=True)
    else:
        y, xq, sx, acc = qa.qgemm_w4a8(x, w, sw, want_acc=True)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.w4a8_quantize_act(case.x, M, K)
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    acc_ref = oracle.w4a8_acc(q_ref, case.w_q4, M, N, K)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    y_ref = acc_ref.astype(np.float64) * s_ref.astype(np.float64)[:, None] * oracle.to_f64(case.s_w, "f16")[None, :]
    assert_float_bar(host_f64(y), y_ref, case.name)
