"""GPU parity of dequantize_affine: every weight, bit for bit, equal to the
oracle's exact value rounded once to the output type."""
import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import dev16, dev32, require_gpu

pytestmark = pytest.mark.gpu

_TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _ref_bits(ref: np.ndarray, out: str) -> np.ndarray:
    return ref.view(np.uint32) if out == "f32" else ref


def _run(N, K, G, bits, sdt, bdt, out, seed, scale_range=(0.003, 0.03)):
    dev = require_gpu()
    packed, s, b = si.affine_weights(N, K, G, bits, seed=seed, scale_range=scale_range, bias_mode="noise",
                                     sb_dtype=sdt)
    if bdt != sdt:
        b = si.store(si.bits_to_f32(b, sdt), bdt)
    print(f"[case] dequant N={N} K={K} G={G} bits={bits} s={sdt} b={bdt} out={out}", flush=True)
    y = qa.dequantize_affine(dev32(packed, dev), dev16(s, sdt, dev), dev16(b, bdt, dev), K, G, bits, out_dtype=_TDT[out])
    torch.cuda.synchronize()
    ref = oracle.dequant_affine_to(packed, s, b, sdt, N, K, G, bits, out, bias_dtype=bdt)
    np.testing.assert_array_equal(_bits(y), _ref_bits(ref, out))


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_every_width_group_and_output(out, bits, G):
    _run(37, 512, G, bits, "bf16", "bf16", out, seed=(80, bits, G))


@pytest.mark.parametrize("sdt,bdt", [("f16", "f16"), ("f32", "f32"), ("bf16", "f32"), ("f16", "bf16")])
@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_parameter_dtypes(sdt, bdt, out):
    _run(19, 1024, 64, 4, sdt, bdt, out, seed=(81, len(sdt), len(bdt), ord(sdt[0]), ord(bdt[0])))


def test_ragged_two_bit_rows():
    # rows of K*bits/32 = 24 words: not whole 16-byte chunks
    _run(9, 96, 32, 2, "bf16", "bf16", "bf16", seed=(82,))


def test_rounding_ties_and_wide_scales():
    # scales over six decades and biases of every magnitude, so that many
    # exact values sit near bf16 and f16 rounding boundaries
    for out in ("bf16", "f16"):
        _run(64, 2048, 64, 8, "f32", "f32", out, seed=(83, len(out)), scale_range=(1e-6, 1.0))


def test_prefill_weight_every_element():
    # a whole prefill weight (N = 4096, K = 4096, 4-bit, G = 64) into bf16
    _run(4096, 4096, 64, 4, "bf16", "bf16", "bf16", seed=(84,), scale_range=(0.002, 0.01))
