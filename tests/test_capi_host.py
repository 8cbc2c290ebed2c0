"""Host-side checks of the C ABI (no GPU needed).

The library must load on a machine without a GPU, export every function that
include/qaff.h declares, and reject bad arguments before touching the HIP
runtime: argument checks run first, so these calls (with fake pointer values)
never launch anything.
"""
import ctypes as C
import os
import re

import pytest

import group_wise_affine_unpack_amd as qa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVAL, UNSUP, ALIGN = 0, 1, 2, 3
A = 0x10000          # a fake, 16-byte aligned "device" address; never dereferenced


def _declared_functions():
    with open(os.path.join(ROOT, "include", "qaff.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)) - {"if"})


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"qmm_affine", "qgemv_affine", "qmm_gptq", "qgemm_w4a8", "gptq_to_affine_repack",
            "quantize_pack_affine", "qaff_last_error", "qaff_version"} <= set(names)
    lib = qa.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.qaff_version() >= 100


def _affine(fn="qmm_affine", x=A, w=A, s=A, b=A, kp=None, y=A, M=1, N=64, K=256, G=64, bits=4, adt=0, sdt=0, bdt=0):
    return getattr(qa.lib(), fn)(x, w, s, b, kp, y, M, N, K, G, bits, adt, sdt, bdt, None)


def _msg():
    return qa.lib().qaff_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(bits=3), INVAL), (dict(bits=16), INVAL), (dict(G=48), INVAL), (dict(G=256), INVAL),
    (dict(K=96, G=64), INVAL), (dict(M=-1), INVAL), (dict(N=-5), INVAL), (dict(K=0), INVAL),
    (dict(adt=2), INVAL), (dict(adt=7), INVAL), (dict(sdt=3), INVAL), (dict(bdt=-1), INVAL),
    (dict(x=None), INVAL), (dict(w=None), INVAL), (dict(s=None), INVAL), (dict(b=None), INVAL),
    (dict(y=None), INVAL), (dict(x=A + 2), ALIGN), (dict(w=A + 4), ALIGN),
    (dict(K=(1 << 30) + 64), UNSUP),
])
@pytest.mark.parametrize("fn", ["qmm_affine", "qgemv_affine"])
def test_affine_argument_errors(fn, kw, code):
    assert _affine(fn, **kw) == code
    assert _msg() != ""


def test_affine_empty_batch_is_ok_without_launch():
    assert _affine(M=0, x=None, y=None) == OK
    assert _affine(N=0, w=None, s=None, b=None, y=None) == OK
    assert _msg() == ""


def test_gemv_rejects_large_m():
    assert _affine("qgemv_affine", M=17) == INVAL
    assert "M <= 16" in _msg()


def test_gptq_argument_errors():
    f = qa.lib().qmm_gptq
    assert f(A, A, A, A, None, A, 1, 64, 256, 100, None) == INVAL      # bad G
    assert f(A, A, A, A, None, A, 1, 60, 256, 64, None) == INVAL       # N % 8
    assert f(A, A, A, A, None, A, 1, 64, 200, 64, None) == INVAL       # K % G
    assert f(None, A, A, A, None, A, 1, 64, 256, 64, None) == INVAL
    assert f(A + 8, A, A, A, None, A, 1, 64, 256, 64, None) == ALIGN
    assert f(None, None, None, None, None, None, 0, 64, 256, 64, None) == OK


def test_w4a8_argument_errors():
    f = qa.lib().qgemm_w4a8
    assert f(A, A, A, A, A, A, None, 8, 64, 100, None) == INVAL        # K % 32
    assert f(A, A, A, None, A, A, None, 8, 64, 128, None) == INVAL
    assert f(A, A + 4, A, A, A, A, None, 8, 64, 128, None) == ALIGN
    assert f(A, A, A, A, A, A, None, 8, 64, 1 << 18, None) == UNSUP    # int32 overflow guard
    assert f(None, None, None, None, None, None, None, 0, 64, 128, None) == OK


def test_repack_argument_errors():
    f = qa.lib().gptq_to_affine_repack
    assert f(A, A, A, None, A, A, A, 0, A, 256, 64, 64, None) == INVAL  # bias dtype bf16 refused
    assert f(A, A, A, None, A, A, A, 2, A, 256, 60, 64, None) == INVAL  # N % 8
    assert f(A, A, A, None, A, None, A, 2, A, 256, 64, 64, None) == INVAL


def test_quantize_pack_argument_errors():
    f = qa.lib().quantize_pack_affine
    assert f(A, 0, A, A, A, 0, 4, 256, 64, 5, None) == INVAL
    assert f(A, 0, A, A, A, 0, 4, 250, 64, 4, None) == INVAL
    assert f(A, 9, A, A, A, 0, 4, 256, 64, 4, None) == INVAL
    assert f(None, 0, None, None, None, 0, 0, 256, 64, 4, None) == OK


def test_binding_has_no_cpu_path():
    import torch
    x = torch.zeros((1, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qa.qmm_affine(x, torch.zeros((8, 32), dtype=torch.int32), torch.zeros((8, 4), dtype=torch.bfloat16),
                      torch.zeros((8, 4), dtype=torch.bfloat16), 64, 4)


def _grouped(probs, M=1, G=64, bits=4, adt=0, sdt=0, bdt=0, count=None):
    arr = (qa.GemvProblem * max(len(probs), 1))(*[qa.GemvProblem(*p) for p in probs])
    n = len(probs) if count is None else count
    return qa.lib().qgemv_affine_grouped(C.cast(arr, C.c_void_p), n, M, G, bits, adt, sdt, bdt, None)


def test_grouped_argument_errors():
    good = (A, A, A, A, None, A, 64, 256)
    assert _grouped([]) == OK
    assert qa.lib().qgemv_affine_grouped(None, 0, 1, 64, 4, 0, 0, 0, None) == OK
    assert qa.lib().qgemv_affine_grouped(None, 2, 1, 64, 4, 0, 0, 0, None) == INVAL
    assert _grouped([good], count=-1) == INVAL
    assert _grouped([good], count=65537) == INVAL
    assert _grouped([good], M=17) == INVAL and "M <= 16" in _msg()
    assert _grouped([good], bits=3) == INVAL
    # the first bad problem names itself and nothing is launched
    assert _grouped([good, (A, A, A, A, None, A, 64, 96)]) == INVAL and "problem 1" in _msg()
    assert _grouped([good, good, (A + 2, A, A, A, None, A, 64, 256)]) == ALIGN and "problem 2" in _msg()
    assert _grouped([good, (A, A, A, A, None, None, 64, 256)]) == INVAL
    # empty problems are skipped without needing pointers; M = 0 launches nothing
    assert _grouped([(None, None, None, None, None, None, 0, 256)]) == OK
    assert _grouped([(None, A, A, A, None, None, 64, 256)], M=0) == OK


def test_release_with_nothing_held_makes_no_hip_call():
    # no scratch was ever taken in this process, so the release touches no
    # device (it runs on a machine without a GPU)
    freed = C.c_uint64(123)
    assert qa.lib().qaff_release_workspaces(C.byref(freed)) == OK
    assert freed.value == 0
    assert qa.lib().qaff_release_workspaces(None) == OK


class _ChainLin(C.Structure):
    _fields_ = [("x", C.c_void_p), ("gate", C.c_void_p), ("resid", C.c_void_p), ("w_packed", C.c_void_p),
                ("scales", C.c_void_p), ("biases", C.c_void_p), ("y", C.c_void_p), ("N", C.c_int64),
                ("K", C.c_int64), ("stage", C.c_int32)]


def _chain(lins, G=64, bits=4, adt=0, out=True):
    arr = (_ChainLin * max(len(lins), 1))(*[_ChainLin(**{**dict(x=A, w_packed=A, scales=A, biases=A, y=A, N=64,
                                                                  K=256, stage=0), **l}) for l in lins])
    h = C.c_void_p()
    return qa.lib().qgemv_affine_chain_plan(C.cast(arr, C.c_void_p), len(lins), G, bits, adt,
                                            C.byref(h) if out else None)


@pytest.mark.parametrize("lins,kw,code", [
    ([{}], dict(bits=8), UNSUP),                       # 4-bit codes only
    ([{}], dict(adt=2), INVAL),                        # act dtype BF16 or F16
    ([{}], dict(G=48), INVAL),
    ([{"K": 96}], {}, INVAL),                          # K not a multiple of G
    ([{"K": 80}], dict(G=16 * 2), INVAL),              # K % 32 != 0 is also not a multiple of G=32
    ([{"x": None}], {}, INVAL),
    ([{"gate": A + 2}], {}, ALIGN),
    ([{"x": A + 2}], {}, ALIGN),
    ([{"N": 0}], {}, INVAL),
    ([{"stage": 1}, {"stage": 0}], {}, INVAL),        # stages nondecreasing
    ([{"stage": -1}], {}, INVAL),
    ([], {}, INVAL),                                   # at least one linear
    ([{}], dict(out=False), INVAL),                    # null plan_out
])
def test_chain_plan_argument_errors(lins, kw, code):
    assert _chain(lins, **kw) == code
    assert _msg() != ""


def test_chain_null_plan_calls():
    lib = qa.lib()
    assert lib.qgemv_affine_chain_run(None, None) == INVAL
    v = C.c_int32(7)
    assert lib.qgemv_affine_chain_status(None, C.byref(v)) == INVAL
    assert lib.qgemv_affine_chain_free(None) == OK
