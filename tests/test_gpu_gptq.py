"""GPU parity of the GPTQ paths: the direct kernel, the repack (bit-exact
against the oracle's repack) and repack followed by qmm_affine with k_perm."""
import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import assert_float_bar, dev16, dev32, host_f64, require_gpu

pytestmark = pytest.mark.gpu


def _dev(case, dev):
    x = dev16(case.x, "f16", dev)
    qw = torch.from_numpy(np.ascontiguousarray(case.qweight)).to(dev)
    qz = torch.from_numpy(np.ascontiguousarray(case.qzeros)).to(dev)
    s = dev16(case.scales, "f16", dev)
    gi = None if case.g_idx is None else torch.from_numpy(np.ascontiguousarray(case.g_idx)).to(dev)
    return x, qw, qz, s, gi


def _log(case, what):
    print(f"[case] {what} {case.name} M={case.M} K={case.K} N={case.N} G={case.G} act_order={case.g_idx is not None}",
          flush=True)


@pytest.mark.parametrize("M", si.CFG3_M)
def test_cfg3_direct(M):
    dev = require_gpu()
    case = si.cfg3_case(M)
    _log(case, "direct")
    x, qw, qz, s, gi = _dev(case, dev)
    y = qa.qmm_gptq(x, qw, qz, s, gi, case.G)
    torch.cuda.synchronize()
    cols = si.sample_indices(case.N, 1024 if M > 1 else case.N, seed=(3, 5, M))
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, M, case.K, case.N, case.G)
    assert_float_bar(host_f64(y)[:, cols], ref[:, cols], case.name)


@pytest.mark.parametrize("bias_dtype", ["f32", "f16"])
def test_cfg3_repack_bit_exact(bias_dtype):
    dev = require_gpu()
    case = si.cfg3_case(1)
    _log(case, "repack")
    x, qw, qz, s, gi = _dev(case, dev)
    tdt = torch.float32 if bias_dtype == "f32" else torch.float16
    w, s_aff, b_aff, kp = qa.gptq_to_affine_repack(qw, qz, s, gi, case.G, bias_dtype=tdt)
    torch.cuda.synchronize()
    rp, rs, rb, rk = oracle.gptq_to_affine_repack(case.qweight, case.qzeros, case.scales, case.g_idx, case.K, case.N,
                                                  case.G, bias_dtype)
    np.testing.assert_array_equal(kp.cpu().numpy(), rk)
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint32), rp)
    np.testing.assert_array_equal(s_aff.cpu().view(torch.int16).numpy().view(np.uint16), rs)
    if bias_dtype == "f32":
        np.testing.assert_array_equal(b_aff.cpu().numpy(), rb)
    else:
        np.testing.assert_array_equal(b_aff.cpu().view(torch.int16).numpy().view(np.uint16), rb)


@pytest.mark.parametrize("M", si.CFG3_M)
@pytest.mark.parametrize("bias_dtype", ["f32", "f16"])
def test_cfg3_repack_then_qmm_affine(M, bias_dtype):
    dev = require_gpu()
    case = si.cfg3_case(M)
    _log(case, f"repack+affine bias={bias_dtype}")
    x, qw, qz, s, gi = _dev(case, dev)
    tdt = torch.float32 if bias_dtype == "f32" else torch.float16
    w, s_aff, b_aff, kp = qa.gptq_to_affine_repack(qw, qz, s, gi, case.G, bias_dtype=tdt)
    y = qa.qmm_affine(x, w, s_aff, b_aff, case.G, 4, k_perm=kp)
    torch.cuda.synchronize()
    cols = si.sample_indices(case.N, 1024 if M > 1 else case.N, seed=(3, 6, M))
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, M, case.K, case.N, case.G)
    assert_float_bar(host_f64(y)[:, cols], ref[:, cols], case.name)


@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("act_order", [True, False])
@pytest.mark.parametrize("M", [1, 3, 20])
def test_small_direct_and_repack(G, act_order, M):
    dev = require_gpu()
    case = si.gptq_case(M, 1024, 200, G, seed=(31, G, M), act_order=act_order, name=f"gptq_small_G{G}")
    if not act_order:
        case.g_idx = None
    _log(case, "small")
    x, qw, qz, s, gi = _dev(case, dev)
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, M, case.K, case.N, case.G)
    y = qa.qmm_gptq(x, qw, qz, s, gi, G)
    w, sa, ba, kp = qa.gptq_to_affine_repack(qw, qz, s, gi, G)
    y2 = qa.qmm_affine(x, w, sa, ba, G, 4, k_perm=kp)
    torch.cuda.synchronize()
    assert_float_bar(host_f64(y), ref, case.name + " direct")
    assert_float_bar(host_f64(y2), ref, case.name + " repack")


def test_repack_rejects_uneven_groups():
    dev = require_gpu()
    case = si.gptq_case(1, 256, 16, 64, seed=(32,))
    g = case.g_idx.copy()
    g[int(np.flatnonzero(g == 0)[0])] = 1
    case.g_idx = g
    x, qw, qz, s, gi = _dev(case, dev)
    with pytest.raises(qa.QaffError) as ei:
        qa.gptq_to_affine_repack(qw, qz, s, gi, 64)
    assert ei.value.status == 1


@pytest.mark.parametrize("M,N,K,G", [
    (1, 1000, 1024, 128),   # 4 columns per lane, a partial last column group
    (5, 2040, 4096, 64),    # 64 groups: 2 columns per lane
    (9, 264, 4096, 32),     # 128 groups: 1 column per lane, a 64 KiB table
    (2, 136, 6144, 32),     # 192 groups: a 96 KiB table
    (20, 520, 2048, 128),   # three passes of x rows (8, 8, 4)
])
@pytest.mark.parametrize("act_order", [True, False])
def test_direct_shapes(M, N, K, G, act_order):
    dev = require_gpu()
    case = si.gptq_case(M, K, N, G, seed=(33, M, N, K, G), act_order=act_order, name=f"gptq_M{M}_N{N}_K{K}_G{G}")
    if not act_order:
        case.g_idx = None
    _log(case, "direct shapes")
    x, qw, qz, s, gi = _dev(case, dev)
    y = qa.qmm_gptq(x, qw, qz, s, gi, G)
    torch.cuda.synchronize()
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, M, case.K, case.N, case.G)
    assert_float_bar(host_f64(y), ref, case.name)


@pytest.mark.parametrize("M,N,K,G", [
    (1, 520, 8192, 32),     # 256 groups: more than a whole table can hold
    (3, 264, 16384, 32),    # 512 groups, four columns per lane
    (9, 136, 8192, 32),     # the matrix-core kernel past 96 groups
    (40, 264, 16384, 64),   # the same with two 32-row blocks
])
def test_direct_without_act_order_many_groups(M, N, K, G):
    # g_idx NULL: each workgroup's table holds only its K slice's groups (and
    # on the matrix cores the slice's own largest scale exponent), so K/G is
    # not limited by LDS
    dev = require_gpu()
    case = si.gptq_case(M, K, N, G, seed=(58, M, N, K, G), act_order=False, name=f"gptq_noact_M{M}_N{N}_K{K}_G{G}")
    case.g_idx = None
    _log(case, "direct, slice tables")
    x, qw, qz, s, gi = _dev(case, dev)
    y = qa.qmm_gptq(x, qw, qz, s, gi, G)
    torch.cuda.synchronize()
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, M, case.K, case.N, case.G)
    assert_float_bar(host_f64(y), ref, case.name)


@pytest.mark.parametrize("M,N,K,G", [
    (8, 200, 1024, 128),     # the smallest M of the matrix-core kernel, a partial column group
    (33, 1000, 2048, 64),    # two 32-row blocks, the second with one row
    (64, 136, 6144, 64),     # 96 groups: the largest table it takes
    (100, 264, 1024, 32),    # two passes of 64 rows
])
@pytest.mark.parametrize("act_order", [True, False])
def test_direct_matrix_core_shapes(M, N, K, G, act_order):
    dev = require_gpu()
    case = si.gptq_case(M, K, N, G, seed=(54, M, N, K, G), act_order=act_order,
                        name=f"gptq_mfma_M{M}_N{N}_K{K}_G{G}")
    if not act_order:
        case.g_idx = None
    _log(case, "direct matrix core")
    x, qw, qz, s, gi = _dev(case, dev)
    y = qa.qmm_gptq(x, qw, qz, s, gi, G)
    torch.cuda.synchronize()
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, M, case.K, case.N, case.G)
    assert_float_bar(host_f64(y), ref, case.name)


def test_direct_matrix_core_scale_range():
    # scales over three decades inside each column: the fp16 weight pieces
    # are taken relative to the column's largest scale exponent
    dev = require_gpu()
    case = si.gptq_case(16, 2048, 256, 128, seed=(55,), scale_range=(1e-3, 4.0), name="gptq_mfma_scale_range")
    _log(case, "direct matrix core")
    x, qw, qz, s, gi = _dev(case, dev)
    y = qa.qmm_gptq(x, qw, qz, s, gi, case.G)
    torch.cuda.synchronize()
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, case.M, case.K, case.N, case.G)
    assert_float_bar(host_f64(y), ref, case.name)


def test_split_k_sums_on_every_call():
    # K split over workgroups: every call writes every output afresh.  Calls
    # alternate between the kernels and shapes on one stream, each into an
    # output filled with NaN first, so that a partial sum left from another
    # call, or an output no workgroup wrote, shows as a wrong value or NaN.
    dev = require_gpu()
    shapes = [(1, 1000, 1024, 128), (3, 2040, 4096, 64), (8, 200, 1024, 128), (64, 136, 6144, 64),
              (1, 264, 4096, 32)]
    cases = []
    for i, (M, N, K, G) in enumerate(shapes):
        case = si.gptq_case(M, K, N, G, seed=(56, i), name=f"gptq_rep_M{M}_N{N}_K{K}_G{G}")
        ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, M, K, N, G)
        cases.append((case, _dev(case, dev), ref))
    for rep in range(3):
        for case, (x, qw, qz, s, gi), ref in cases:
            _log(case, f"repeated calls, pass {rep}")
            y = torch.full((case.M, case.N), float("nan"), dtype=torch.float16, device=dev)
            qa.qmm_gptq(x, qw, qz, s, gi, case.G, out=y)
            torch.cuda.synchronize()
            assert_float_bar(host_f64(y), ref, f"{case.name} pass {rep}")


@pytest.mark.parametrize("M,N,G", [(2, 2040, 64), (1, 2040, 64), (1, 4104, 128)])
def test_split_k_sums_under_graph_replay(M, N, G):
    # a captured call replayed into an output refilled with NaN each time
    dev = require_gpu()
    case = si.gptq_case(M, 4096, N, G, seed=(57, M, N), name=f"gptq_rep_graph_M{M}_N{N}")
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, case.M, case.K, case.N, case.G)
    x, qw, qz, s, gi = _dev(case, dev)
    _log(case, "graph replays")
    y = torch.empty((case.M, case.N), dtype=torch.float16, device=dev)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        qa.qmm_gptq(x, qw, qz, s, gi, case.G, out=y)  # sizes the stream's buffers
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        qa.qmm_gptq(x, qw, qz, s, gi, case.G, out=y)
    torch.cuda.synchronize()
    for rep in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_float_bar(host_f64(y), ref, f"{case.name} replay {rep}")


# One x row over shapes that stress the direct kernel's split of columns
# and K: few and many column groups, one group, a short last K slice.
@pytest.mark.parametrize("N,K,G", [
    (2040, 4096, 64),    # 64 groups
    (136, 2048, 32),     # 64 groups, most lanes of the last column group past N
    (8, 4096, 128),      # one column group, most lanes past N
    (512, 128, 128),     # one group
    (11008, 1024, 32),   # 32 groups, many column groups
    (1000, 2816, 128),   # 22 groups, a short last slice
])
@pytest.mark.parametrize("act_order", [True, False])
def test_one_row_shapes(N, K, G, act_order):
    dev = require_gpu()
    case = si.gptq_case(1, K, N, G, seed=(59, N, K, G), act_order=act_order, name=f"gptq_row_N{N}_K{K}_G{G}")
    if not act_order:
        case.g_idx = None
    _log(case, "direct, one row")
    x, qw, qz, s, gi = _dev(case, dev)
    y = torch.full((1, N), float("nan"), dtype=torch.float16, device=dev)
    qa.qmm_gptq(x, qw, qz, s, gi, G, out=y)
    torch.cuda.synchronize()
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, 1, K, N, G)
    assert_float_bar(host_f64(y), ref, case.name)


def test_one_row_scale_range():
    # scales over three decades and activations 8x the usual (outputs up to
    # about 2e4, inside fp16): the weights are exact in fp32 whatever the
    # range
    dev = require_gpu()
    case = si.gptq_case(1, 4096, 1024, 128, seed=(60,), scale_range=(1e-3, 4.0), name="gptq_row_scale_range")
    case.x = si.f16_bits(si.bits_to_f32(case.x, "f16") * np.float32(8.0))
    _log(case, "direct, one row")
    x, qw, qz, s, gi = _dev(case, dev)
    y = qa.qmm_gptq(x, qw, qz, s, gi, case.G)
    torch.cuda.synchronize()
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, 1, case.K, case.N, case.G)
    assert_float_bar(host_f64(y), ref, case.name)


# Act-order with more groups than the per-workgroup LDS table holds (above
# 192): the (scale, bias) entries come from a table in device memory.
@pytest.mark.parametrize("M", [1, 2, 3, 8, 33])
@pytest.mark.parametrize("K,N,G", [(8192, 1024, 32), (6272, 520, 32), (16384, 256, 64)])
def test_direct_act_order_beyond_lds_table(M, K, N, G):
    dev = require_gpu()
    case = si.gptq_case(M, K, N, G, seed=(3, 50, M, K), act_order=True)
    _log(case, "direct global table")
    x, qw, qz, s, gi = _dev(case, dev)
    y = qa.qmm_gptq(x, qw, qz, s, gi, case.G)
    torch.cuda.synchronize()
    ref = oracle.qmm_gptq(case.x, case.qweight, case.qzeros, case.scales, case.g_idx, M, case.K, case.N, case.G)
    assert_float_bar(host_f64(y), ref, case.name)
