"""GPU parity of qgemv_affine_silu_gate: y = W (silu(gate) * up) [+ resid]
against the fp64 oracle."""
import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import affine_to_device, assert_float_bar, dev16, host_f64, require_gpu

pytestmark = pytest.mark.gpu


def _run(M, N, K, G, bits, act, sdt="bf16", resid=False, alias=False, seed=(90,)):
    dev = require_gpu()
    c = si.affine_case(M, N, K, G, bits, seed=seed, act_dtype=act, sb_dtype=sdt, name="silu")
    up = si.activations(M, K, seed=(*seed, 7), dtype=act)
    r = si.activations(M, N, seed=(*seed, 8), dtype=act) if resid else None
    print(f"[case] silu_gate M={M} N={N} K={K} G={G} bits={bits} act={act} s={sdt} resid={resid} alias={alias}",
          flush=True)
    gate, w, s, b, _ = affine_to_device(c, dev)
    upd = dev16(up, act, dev)
    rd = None if r is None else dev16(r, act, dev)
    y = qa.qgemv_affine_silu_gate(gate, upd, w, s, b, G, bits, resid=rd, out=rd if alias else None)
    torch.cuda.synchronize()
    ref = oracle.qmm_affine_silu_gate(c.x, up, r, act, c.packed, c.scales, c.biases, sdt, M, N, K, G, bits)
    assert_float_bar(host_f64(y), ref, f"silu M={M} N={N} K={K} b{bits} {act}")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decoder_down_projection(M):
    # the down projection of the 1B decode set: N = 2048, K = 8192, 4-bit, G = 64
    _run(M, 2048, 8192, 64, 4, "bf16", resid=True, seed=(91, M))


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("resid", [False, True])
def test_widths_dtypes_residual(bits, act, resid):
    _run(3, 77, 1024, 64, bits, act, resid=resid, seed=(92, bits, act == "f16", resid))


@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("sdt", ["f16", "f32"])
def test_groups_and_parameter_dtypes(G, sdt):
    _run(2, 130, 2048, G, 4, "f16", sdt=sdt, resid=True, seed=(93, G))


def test_residual_updated_in_place():
    _run(5, 256, 4096, 64, 4, "bf16", resid=True, alias=True, seed=(94,))


def test_short_and_long_rows():
    # K split over 1, 2 and 4 waves of a workgroup
    for K in (256, 768, 14336):
        _run(1, 64, K, 64, 4, "bf16", resid=True, seed=(95, K))


def test_rejects_ragged_rows_and_large_m():
    dev = require_gpu()
    x = torch.zeros((17, 256), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((8, 32), dtype=torch.int32, device=dev)
    sc = torch.zeros((8, 4), dtype=torch.bfloat16, device=dev)
    with pytest.raises(qa.QaffError):
        qa.qgemv_affine_silu_gate(x, x, w, sc, sc, 64, 4)
    x2 = torch.zeros((1, 96), dtype=torch.bfloat16, device=dev)
    w2 = torch.zeros((8, 6), dtype=torch.int32, device=dev)
    s2 = torch.zeros((8, 3), dtype=torch.bfloat16, device=dev)
    with pytest.raises(qa.QaffError):
        qa.qgemv_affine_silu_gate(x2, x2, w2, s2, s2, 32, 2)
