"""GPU parity of the W4A8 path: int8 codes, per-token scales and int32
accumulators bit-exact against the oracle; y within the float bar."""
import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import assert_float_bar, dev16, host_f64, require_gpu

pytestmark = pytest.mark.gpu


def _run(case):
    dev = require_gpu()
    print(f"[case] {case.name} M={case.M} N={case.N} K={case.K}", flush=True)
    x = dev16(case.x, "f16", dev)
    w = torch.from_numpy(np.ascontiguousarray(case.w_q4).view(np.int32)).to(dev)
    sw = dev16(case.s_w, "f16", dev)
    y, xq, sx, acc = qa.qgemm_w4a8(x, w, sw, want_acc=True)
    torch.cuda.synchronize()
    return y, xq.cpu().numpy(), sx.cpu().numpy(), acc


def _check(case, rows=None):
    y, xq, sx, acc = _run(case)
    q_ref, s_ref = oracle.w4a8_quantize_act(case.x, case.M, case.K)
    np.testing.assert_array_equal(xq, q_ref)
    np.testing.assert_array_equal(sx.view(np.uint32), s_ref.view(np.uint32))
    rows = np.arange(case.M) if rows is None else rows
    acc_ref = oracle.w4a8_acc(q_ref[rows], case.w_q4, len(rows), case.N, case.K)
    acc_gpu = acc.cpu().numpy()[rows].astype(np.int64)
    np.testing.assert_array_equal(acc_gpu, acc_ref)
    y_ref = acc_ref.astype(np.float64) * s_ref[rows].astype(np.float64)[:, None] * \
        oracle.to_f64(case.s_w, "f16")[None, :]
    assert_float_bar(host_f64(y)[rows], y_ref, case.name)


@pytest.mark.parametrize("M", si.CFG4_M)
@pytest.mark.parametrize("N,K", si.CFG4_SHAPES)
def test_cfg4(N, K, M):
    case = si.cfg4_case(N, K, M, seed=(4, N, K, M))
    rows = None if M <= 128 else si.sample_indices(M, 48, seed=(4, 9, M))
    _check(case, rows)


def test_cfg4_every_row_at_m2048():
    # one M = 2048 shape of the set with every row of x_q, s_x and acc
    # against the oracle (the other M = 2048 shapes check sampled rows)
    case = si.cfg4_case(1024, 1024, 2048, seed=(4, 1024, 1024, 2048))
    _check(case)


def test_every_nibble_and_ragged_shapes():
    case = si.w4a8_case(13, 200, 192, seed=(40,), name="w4a8_ragged")
    r = np.random.default_rng(41)
    codes = np.stack([r.permutation(np.tile(np.arange(-8, 8), 192 // 16)) for _ in range(200)])
    case.w_q4 = si.pack_nibbles_along_last(codes & 0xF)
    _check(case)


def test_ties_zero_rows_and_extremes():
    case = si.w4a8_case(8, 64, 128, seed=(42,), name="w4a8_ties")
    xf = si.bits_to_f32(case.x, "f16").copy()
    e = 2.0 ** -3
    xf[0, :] = 0.0
    xf[1, :] = (np.arange(128) % 40 - 20 + 0.5) * e       # exact ties after scaling
    xf[1, 0] = 127 * e                                    # amax = 127 * 2^-3 -> s_x = 2^-3
    xf[2, :] = 65504.0 * np.sign(np.random.default_rng(43).standard_normal(128))
    xf[3, :] = 2.0 ** -24                                  # smallest subnormal everywhere
    case.x = si.f16_bits(xf)
    _check(case)


@pytest.mark.parametrize("M,N,K", [(5, 70, 32), (40, 130, 96), (200, 300, 1056), (300, 520, 4000)])
def test_k_not_multiple_of_stage(M, N, K):
    # K % 32 == 0 is all the entry point asks; the GEMM walks K in stages of
    # 128 codes, so these shapes end on a partial stage (32, 96, 32, 32 codes)
    # and span several row and column tiles with ragged edges
    case = si.w4a8_case(M, N, K, seed=(44, M, N, K), name=f"w4a8_M{M}_N{N}_K{K}")
    _check(case)


@pytest.mark.parametrize("K", [32, 512, 544, 1024, 2048, 4096, 8192, 16384, 16416])
def test_quantize_row_lengths(K):
    # the quantizer holds a row in the registers of one wave (K <= 512), two
    # (K <= 1024) or four (chunks of 8 values, 1, 2, 4 or 8 per thread up to
    # K = 16384); K = 16416 takes the one-row-per-block loop.  M = 7 leaves
    # the last block partly empty.
    case = si.w4a8_case(7, 40, K, seed=(45, K), name=f"w4a8_quant_K{K}")
    _check(case)


def test_unaligned_activations_rejected():
    # x one element past a 16-byte boundary: refused before any launch
    case = si.w4a8_case(7, 96, 256, seed=(46,), name="w4a8_unaligned_x")
    dev = require_gpu()
    big = dev16(np.concatenate([np.zeros(1, np.uint16), case.x.reshape(-1)]), "f16", dev)
    x = big[1:].view(case.M, case.K)
    assert x.data_ptr() % 16 == 2
    w = torch.from_numpy(np.ascontiguousarray(case.w_q4).view(np.int32)).to(dev)
    sw = dev16(case.s_w, "f16", dev)
    with pytest.raises(qa.QaffError, match="QAFF_E_ALIGN"):
        qa.qgemm_w4a8(x, w, sw)


def test_quantize_every_f16_activation_and_scale():
    # Every positive finite f16 maximum a (0x0001 .. 0x7BFF) meets every f16
    # value of magnitude 0 .. a, odd columns negated: rows of 1024 hold a
    # followed by 1023 of those values (zeros pad the last row of each a).
    # Codes and scales must match the oracle bit for bit, which holds the
    # quantizer's division to the IEEE quotient over its whole domain.
    dev = require_gpu()
    K, P = 1024, 1023
    a = np.arange(1, 0x7C00, dtype=np.int64)
    per_a = (a + P) // P
    R = int(per_a.sum())
    row_a = np.repeat(a, per_a)
    j = np.arange(R) - np.repeat(np.cumsum(per_a) - per_a, per_a)
    x = np.zeros((R, K), np.uint16)
    x[:, 0] = row_a
    for r0 in range(0, R, 1 << 16):
        r1 = min(R, r0 + (1 << 16))
        vals = j[r0:r1, None] * P + np.arange(P)[None, :]
        x[r0:r1, 1:] = np.where(vals <= row_a[r0:r1, None], vals, 0)
    x[:, 1::2] |= 0x8000
    print(f"[case] w4a8 quantize, every f16 pair: M={R} K={K}", flush=True)
    xd = dev16(x, "f16", dev)
    w = torch.zeros((32, K // 8), dtype=torch.int32, device=dev)
    sw = torch.ones((32,), dtype=torch.float16, device=dev)
    _, xq, sx, _ = qa.qgemm_w4a8(xd, w, sw)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.w4a8_quantize_act(x, R, K)
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    got = xq.cpu().numpy()
    bad = np.argwhere(got != q_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: x=0x{x[tuple(bad[0])]:04x}"


@pytest.mark.parametrize("M,N,K", [(1, 37, 32), (2, 64, 2048), (3, 130, 4096), (16, 70, 1056), (5, 2060, 512),
                                   (16, 4100, 4096), (9, 300, 8192), (17, 300, 4096), (100, 260, 8192)])
def test_small_m_paths(M, N, K):
    # M <= 16, K <= 4096: the fused quantize + dot4 GEMV, 1, 2 or 4 columns
    # per wave (N below 2048, from 2048, from 4096; N not a multiple of the
    # workgroup's columns, K down to one 32-code chunk, M = 16 at K = 4096
    # fills its 64 KiB of LDS); M = 9 at K = 8192: the quantize kernel, then
    # the GEMV; M = 17 and 100: the MFMA GEMM with K split over workgroups
    # and int32 partials
    case = si.w4a8_case(M, N, K, seed=(47, M, N, K), name=f"w4a8_small_M{M}_N{N}_K{K}")
    _check(case)


def test_largest_tile():
    # K = 2048 (a long loop) and 2048 x 4096: one 128 x 256 tile per CU, the
    # largest tile (sampled rows against the oracle)
    case = si.w4a8_case(2048, 4096, 2048, seed=(48,), name="w4a8_tile_128x256")
    _check(case, si.sample_indices(2048, 48, seed=(48, 1)))


TILES = [(32, 128), (64, 128), (64, 256), (128, 256)]


def _check_tiled(case, staged, bm, bn, rows=None):
    dev = require_gpu()
    print(f"[case] {case.name} staged={staged} tile={bm}x{bn} M={case.M} N={case.N} K={case.K}", flush=True)
    x = dev16(case.x, "f16", dev)
    w = torch.from_numpy(np.ascontiguousarray(case.w_q4).view(np.int32)).to(dev)
    sw = dev16(case.s_w, "f16", dev)
    y, xq, sx, acc = qa.qgemm_w4a8_tiled(x, w, sw, staged, bm, bn, want_acc=True)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.w4a8_quantize_act(case.x, case.M, case.K)
    np.testing.assert_array_equal(xq.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(sx.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    rows = np.arange(case.M) if rows is None else rows
    acc_ref = oracle.w4a8_acc(q_ref[rows], case.w_q4, len(rows), case.N, case.K)
    np.testing.assert_array_equal(acc.cpu().numpy()[rows].astype(np.int64), acc_ref)
    y_ref = acc_ref.astype(np.float64) * s_ref[rows].astype(np.float64)[:, None] * \
        oracle.to_f64(case.s_w, "f16")[None, :]
    assert_float_bar(host_f64(y)[rows], y_ref, case.name)
    return y, acc


@pytest.mark.parametrize("staged", [0, 1])
@pytest.mark.parametrize("bm,bn", TILES)
@pytest.mark.parametrize("M", [128, 2048])
@pytest.mark.parametrize("N,K", si.CFG4_SHAPES)
def test_cfg4_each_lowering_and_tile(N, K, M, bm, bn, staged):
    # both lowerings, every built tile, on the set's M > 16 shapes: codes,
    # scales and accumulators exact against the oracle (sampled rows at
    # M = 2048), y within the float bar
    case = si.cfg4_case(N, K, M, seed=(4, N, K, M))
    rows = None if M <= 128 else si.sample_indices(M, 40, seed=(4, 10, M))
    _check_tiled(case, staged, bm, bn, rows)


@pytest.mark.parametrize("M,N,K", [(17, 1000, 1056), (100, 520, 4128), (300, 2056, 160), (33, 136, 8192)])
@pytest.mark.parametrize("bm,bn", [(32, 128), (128, 256)])
def test_staged_ragged_and_split(M, N, K, bm, bn):
    # rows past M, columns past N, a last K tile of 32 or 96 codes; few
    # tiles with a long K split it over workgroups (int32 partials)
    case = si.w4a8_case(M, N, K, seed=(49, M, N, K), name=f"w4a8_staged_M{M}_N{N}_K{K}")
    _check_tiled(case, 1, bm, bn)


def test_staged_same_bits_as_full_k():
    # the two lowerings give the same y bits (the same integer sums, scales
    # and rounding), on a shape where each runs its own kernels
    case = si.w4a8_case(256, 1024, 2048, seed=(50,), name="w4a8_staged_vs_fullk")
    y0, a0 = _check_tiled(case, 0, 64, 128)
    y1, a1 = _check_tiled(case, 1, 64, 128)
    assert torch.equal(a0, a1)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


def test_tiled_rejects_small_m_and_unbuilt_tiles():
    dev = require_gpu()
    case = si.w4a8_case(16, 256, 256, seed=(51,), name="w4a8_small")
    x = dev16(case.x, "f16", dev)
    w = torch.from_numpy(np.ascontiguousarray(case.w_q4).view(np.int32)).to(dev)
    sw = dev16(case.s_w, "f16", dev)
    with pytest.raises(qa.QaffError) as e1:
        qa.qgemm_w4a8_tiled(x, w, sw, True, 64, 128)
    assert e1.value.status == 2
    x2 = torch.zeros((64, 256), dtype=torch.float16, device=dev)
    with pytest.raises(qa.QaffError) as e2:
        qa.qgemm_w4a8_tiled(x2, w, sw, True, 96, 128)
    assert e2.value.status == 2


@pytest.mark.parametrize("M,N,K,bm,bn,staged", [
    (2048, 4096, 1024, 128, 256, False), (256, 1000, 2048, 64, 256, False), (300, 1024, 1024, 64, 128, False),
    (128, 520, 4096, 32, 128, True), (2048, 1024, 1024, 128, 256, True)])
def test_epilogue_paths_same_bits(M, N, K, bm, bn, staged):
    # Without accumulators asked for, tiles whose rows all exist store y from
    # scalar row bases and packed conversions; with them (or in a ragged last
    # row tile) the per-value path runs.  Both round the same product, so y
    # must be the same bits (M = 300 and N = 1000 / 520: ragged tiles).
    from gpu_util import dev16
    case = si.w4a8_case(M, N, K, seed=(65, M, N), name=f"w4a8_epi_M{M}_N{N}_K{K}_{bm}x{bn}_{staged}")
    dev = require_gpu()
    x = dev16(case.x, "f16", dev)
    w = torch.from_numpy(np.ascontiguousarray(case.w_q4).view(np.int32)).to(dev)
    sw = dev16(case.s_w, "f16", dev)
    print(f"[case] {case.name}", flush=True)
    y0, _, _, _ = qa.qgemm_w4a8_tiled(x, w, sw, staged, bm, bn, want_acc=False)
    y1, _, _, acc = qa.qgemm_w4a8_tiled(x, w, sw, staged, bm, bn, want_acc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y0.cpu().numpy().view(np.uint16), y1.cpu().numpy().view(np.uint16))
    if M == 2048 and not staged:
        y2, _, _, _ = qa.qgemm_w4a8(x, w, sw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y2.cpu().numpy().view(np.uint16), y1.cpu().numpy().view(np.uint16))
