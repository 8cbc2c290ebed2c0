"""GPU parity of quantize_pack_affine: codes, scales and biases bit-exact
against the oracle (same IEEE fp32 rule); the packed result feeds qmm_affine."""
import numpy as np
import pytest
import torch

import group_wise_affine_unpack_amd as qa
import oracle
import synth_inputs as si
from gpu_util import TORCH_DT, assert_float_bar, dev16, host_f64, require_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("wdt,sbdt", [("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16"), ("bf16", "f32")])
def test_bit_exact(bits, G, wdt, sbdt):
    dev = require_gpu()
    N, K = 96, 1024
    print(f"[case] quantize_pack bits={bits} G={G} w={wdt} sb={sbdt}", flush=True)
    w = si.dense_weights(N, K, seed=(50, bits, G), dtype=wdt)
    wt = dev16(w, wdt, dev)
    packed, s, b = qa.quantize_pack_affine(wt, G, bits, sb_dtype=TORCH_DT[sbdt])
    torch.cuda.synchronize()
    rp, rs, rb = oracle.quantize_pack_affine(w, wdt, N, K, G, bits, sbdt)
    np.testing.assert_array_equal(packed.cpu().numpy().view(np.uint32), rp)
    np.testing.assert_array_equal(_bits(s), rs)
    np.testing.assert_array_equal(_bits(b), rb)


def test_quantized_weights_feed_qmm_affine():
    dev = require_gpu()
    N, K, G, bits = 256, 2048, 64, 4
    w = si.dense_weights(N, K, seed=(51,), dtype="bf16")
    x = si.activations(3, K, seed=(52,))
    packed, s, b = qa.quantize_pack_affine(dev16(w, "bf16", dev), G, bits)
    y = qa.qmm_affine(dev16(x, "bf16", dev), packed, s, b, G, bits)
    torch.cuda.synchronize()
    ref = oracle.qmm_affine(x, "bf16", packed.cpu().numpy().view(np.uint32), _bits(s), _bits(b), "bf16", 3, N, K, G,
                            bits)
    assert_float_bar(host_f64(y), ref, "quantize_pack->qmm_affine")
