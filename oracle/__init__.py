"""ctypes front end of the CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg.  The HIP library and its Python binding never
import it.  It computes in fp64 from the definitions on the pages; see the
header of oracle.c for the sources and readings.

All arrays are numpy.  16-bit storage types are passed as their raw patterns
(``np.uint16``) with a dtype tag "bf16" / "f16" / "f32".
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_DT = {"bf16": 0, "f16": 1, "f32": 2}
_ERR = {-1: "bad argument", -2: "a group does not hold exactly G columns", -3: "value out of range",
        -4: "out of memory"}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = C.CDLL(_LIB_PATH)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERR.get(rc, rc)}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _sb(a, dtype):
    return _c(a, np.float32 if dtype == "f32" else np.uint16)


I64 = C.c_int64


def set_num_threads(n: int) -> None:
    """Threads for later calls (timing only: no result depends on it)."""
    _load().oracle_set_num_threads(C.c_int(n))


def num_threads() -> int:
    lib = _load()
    lib.oracle_num_threads.restype = C.c_int
    return int(lib.oracle_num_threads())


# ------------------------------------------------------------- conversions

def to_f64(bits, dtype: str) -> np.ndarray:
    a = _sb(bits, dtype)
    out = np.empty(a.shape, dtype=np.float64)
    _load().oracle_to_f64(_p(a), C.c_int(_DT[dtype]), I64(a.size), _p(out))
    return out


def f64_to_f16(v) -> np.ndarray:
    a = _c(v, np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_f64_to_f16(_p(a), I64(a.size), _p(out))
    return out


def f32_to_bf16(v) -> np.ndarray:
    a = _c(v, np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16(_p(a), I64(a.size), _p(out))
    return out


# ------------------------------------------------------------- affine

def unpack_affine(packed, N: int, K: int, bits: int) -> np.ndarray:
    p = _c(packed, np.uint32)
    out = np.empty((N, K), dtype=np.uint8)
    _check(_load().oracle_unpack_affine(_p(p), I64(N), I64(K), C.c_int(bits), _p(out)), "unpack_affine")
    return out


def dequant_affine(packed, scales, biases, sb_dtype: str, N: int, K: int, G: int, bits: int,
                   bias_dtype: str = None) -> np.ndarray:
    """``sb_dtype`` is the scale dtype; the bias dtype defaults to it."""
    bias_dtype = bias_dtype or sb_dtype
    p, s, b = _c(packed, np.uint32), _sb(scales, sb_dtype), _sb(biases, bias_dtype)
    out = np.empty((N, K), dtype=np.float64)
    _check(_load().oracle_dequant_affine(_p(p), _p(s), C.c_int(_DT[sb_dtype]), _p(b), C.c_int(_DT[bias_dtype]),
                                         I64(N), I64(K), C.c_int(G), C.c_int(bits), _p(out)), "dequant_affine")
    return out


def qmm_affine(x, act_dtype: str, packed, scales, biases, sb_dtype: str, M: int, N: int, K: int,
               G: int, bits: int, k_perm=None, bias_dtype: str = None) -> np.ndarray:
    """``sb_dtype`` is the scale dtype; the bias dtype defaults to it."""
    bias_dtype = bias_dtype or sb_dtype
    xa = _c(x, np.uint16 if act_dtype != "f32" else np.float32)
    p, s, b = _c(packed, np.uint32), _sb(scales, sb_dtype), _sb(biases, bias_dtype)
    kp = None if k_perm is None else _c(k_perm, np.int32)
    y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_qmm_affine(_p(xa), C.c_int(_DT[act_dtype]), _p(p), _p(s), C.c_int(_DT[sb_dtype]), _p(b),
                                   C.c_int(_DT[bias_dtype]), _p(kp), I64(M), I64(N), I64(K), C.c_int(G),
                                   C.c_int(bits), _p(y))
    _check(rc, "qmm_affine")
    return y


def qmm_affine_case(case, rows=None, cols=None) -> np.ndarray:
    """Oracle output for an ``AffineCase``; ``rows``/``cols`` select a sample of
    output rows m and columns n (the inputs are sliced, nothing is recomputed
    differently)."""
    x = case.x if rows is None else case.x[rows]
    packed, scales, biases = case.packed, case.scales, case.biases
    if cols is not None:
        packed, scales, biases = packed[cols], scales[cols], biases[cols]
    M, N = x.shape[0], packed.shape[0]
    return qmm_affine(x, case.act_dtype, packed, scales, biases, case.sb_dtype, M, N, case.K, case.G,
                      case.bits, case.k_perm, bias_dtype=case.bias_dtype)


# ------------------------------------------------------------- GPTQ

def dequant_gptq(qweight, qzeros, scales, g_idx, K: int, N: int, G: int) -> np.ndarray:
    qw, qz, s = _c(qweight, np.int32), _c(qzeros, np.int32), _c(scales, np.uint16)
    gi = None if g_idx is None else _c(g_idx, np.int32)
    out = np.empty((N, K), dtype=np.float64)
    _check(_load().oracle_dequant_gptq(_p(qw), _p(qz), _p(s), _p(gi), I64(K), I64(N), C.c_int(G), _p(out)),
           "dequant_gptq")
    return out


def qmm_gptq(x, qweight, qzeros, scales, g_idx, M: int, K: int, N: int, G: int) -> np.ndarray:
    xa = _c(x, np.uint16)
    qw, qz, s = _c(qweight, np.int32), _c(qzeros, np.int32), _c(scales, np.uint16)
    gi = None if g_idx is None else _c(g_idx, np.int32)
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_qmm_gptq(_p(xa), _p(qw), _p(qz), _p(s), _p(gi), I64(M), I64(K), I64(N), C.c_int(G),
                                   _p(y)), "qmm_gptq")
    return y


def gptq_to_affine_repack(qweight, qzeros, scales, g_idx, K: int, N: int, G: int, bias_dtype: str = "f32"):
    """Returns (packed [N, K/8] u32, scales [N, K/G] f16 bits, biases [N, K/G], k_perm [K] i32)."""
    qw, qz, s = _c(qweight, np.int32), _c(qzeros, np.int32), _c(scales, np.uint16)
    gi = None if g_idx is None else _c(g_idx, np.int32)
    packed = np.empty((N, K // 8), dtype=np.uint32)
    s_out = np.empty((N, K // G), dtype=np.uint16)
    b_out = np.empty((N, K // G), dtype=np.float32 if bias_dtype == "f32" else np.uint16)
    kp = np.empty((K,), dtype=np.int32)
    _check(_load().oracle_gptq_to_affine_repack(_p(qw), _p(qz), _p(s), _p(gi), I64(K), I64(N), C.c_int(G),
                                                C.c_int(_DT[bias_dtype]), _p(packed), _p(s_out), _p(b_out),
                                                _p(kp)), "gptq_to_affine_repack")
    return packed, s_out, b_out, kp


# ------------------------------------------------------------- W4A8

def w4a8_quantize_act(x, M: int, K: int):
    xa = _c(x, np.uint16)
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty((M,), dtype=np.float32)
    _check(_load().oracle_w4a8_quantize_act(_p(xa), I64(M), I64(K), _p(q), _p(s)), "w4a8_quantize_act")
    return q, s


def w4a8_acc(q, w_q4, M: int, N: int, K: int) -> np.ndarray:
    qa, w = _c(q, np.int8), _c(w_q4, np.uint32)
    acc = np.empty((M, N), dtype=np.int64)
    _check(_load().oracle_w4a8_acc(_p(qa), _p(w), I64(M), I64(N), I64(K), _p(acc)), "w4a8_acc")
    return acc


def w4a8(x, w_q4, s_w, M: int, N: int, K: int):
    """Returns (q_x int8 [M,K], s_x f32 [M], acc int64 [M,N], y f64 [M,N])."""
    xa, w, sw = _c(x, np.uint16), _c(w_q4, np.uint32), _c(s_w, np.uint16)
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty((M,), dtype=np.float32)
    acc = np.empty((M, N), dtype=np.int64)
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_w4a8(_p(xa), _p(w), _p(sw), I64(M), I64(N), I64(K), _p(q), _p(s), _p(acc), _p(y)),
           "w4a8")
    return q, s, acc, y


# ------------------------------------------------------------- quantize_pack

def quantize_pack_affine(w, w_dtype: str, N: int, K: int, G: int, bits: int, sb_dtype: str):
    """Returns (packed [N, K*bits/32] u32, scales [N, K/G], biases [N, K/G])."""
    wa = _sb(w, w_dtype)
    packed = np.empty((N, K * bits // 32), dtype=np.uint32)
    sdt = np.float32 if sb_dtype == "f32" else np.uint16
    s = np.empty((N, K // G), dtype=sdt)
    b = np.empty((N, K // G), dtype=sdt)
    _check(_load().oracle_quantize_pack_affine(_p(wa), C.c_int(_DT[w_dtype]), I64(N), I64(K), C.c_int(G),
                                               C.c_int(bits), C.c_int(_DT[sb_dtype]), _p(packed), _p(s), _p(b)),
           "quantize_pack_affine")
    return packed, s, b


# ------------------------------------------------------------- comparison

def affine_tolerance_report(y, ref) -> dict:
    """The float bar: max |y-ref|/(|ref|+1) <= 1e-2 and ||y-ref||_F/||ref||_F <= 5e-3."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(y - ref)
    elem = float((err / (np.abs(ref) + 1.0)).max()) if ref.size else 0.0
    nref = float(np.linalg.norm(ref))
    frob = float(np.linalg.norm(y - ref) / nref) if nref > 0 else float(np.linalg.norm(y - ref))
    return {"max_elem": elem, "rel_frob": frob, "ok": bool(elem <= 1e-2 and frob <= 5e-3 and np.isfinite(y).all())}


# ------------------------------------------------------------- dequant to a dtype

def f64_to_bf16(v) -> np.ndarray:
    a = _c(v, np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_f64_to_bf16(_p(a), I64(a.size), _p(out))
    return out


def dequant_affine_to(packed, scales, biases, sb_dtype: str, N: int, K: int, G: int, bits: int, out_dtype: str,
                      bias_dtype: str = None) -> np.ndarray:
    """Every weight exactly (fp64), rounded once to ``out_dtype`` (nearest even):
    uint16 patterns for bf16/f16, float32 for f32."""
    bias_dtype = bias_dtype or sb_dtype
    p, s, b = _c(packed, np.uint32), _sb(scales, sb_dtype), _sb(biases, bias_dtype)
    out = np.empty((N, K), dtype=np.float32 if out_dtype == "f32" else np.uint16)
    _check(_load().oracle_dequant_affine_to(_p(p), _p(s), C.c_int(_DT[sb_dtype]), _p(b), C.c_int(_DT[bias_dtype]),
                                            I64(N), I64(K), C.c_int(G), C.c_int(bits), C.c_int(_DT[out_dtype]),
                                            _p(out)), "dequant_affine_to")
    return out


# ------------------------------------------------------------- SiLU-gated GEMV

def silu(v) -> np.ndarray:
    a = _c(v, np.float64)
    out = np.empty(a.shape, dtype=np.float64)
    _load().oracle_silu(_p(a), I64(a.size), _p(out))
    return out


def qmm_affine_silu_gate(gate, up, resid, act_dtype: str, packed, scales, biases, sb_dtype: str, M: int, N: int,
                         K: int, G: int, bits: int, bias_dtype: str = None) -> np.ndarray:
    """y = W (silu(gate) * up) [+ resid], fp64; gate/up [M, K], resid [M, N] or None."""
    bias_dtype = bias_dtype or sb_dtype
    g, u = _c(gate, np.uint16), _c(up, np.uint16)
    r = None if resid is None else _c(resid, np.uint16)
    p, s, b = _c(packed, np.uint32), _sb(scales, sb_dtype), _sb(biases, bias_dtype)
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_qmm_affine_silu_gate(_p(g), _p(u), _p(r), C.c_int(_DT[act_dtype]), _p(p), _p(s),
                                               C.c_int(_DT[sb_dtype]), _p(b), C.c_int(_DT[bias_dtype]), I64(M),
                                               I64(N), I64(K), C.c_int(G), C.c_int(bits), _p(y)),
           "qmm_affine_silu_gate")
    return y


# ------------------------------------------------------------- decode chain

def qgemv_affine_chain(linears, buffers, act_dtype: str, G: int, bits: int = 4) -> dict:
    """A decode step's linears (one x row) in the order of their stages, each
    y = W h (+ resid) with h = x, or silu(gate) * x when a gate is given (the
    fused inputs of the mlx_int8.rs API page: gemv_gate_up, gemv_silu_gate,
    gemv_silu_gate_resid).  Every y is computed in fp64 from the stored
    values of its inputs (qmm_affine and qmm_affine_silu_gate above), then
    stored: rounded once to act_dtype, the value later linears read.

    buffers: {name: stored [K] or [N] patterns (np.uint16)}, the inputs; each
    linear: dict(name, x, gate, resid (names of buffers or of earlier
    linears, gate/resid may be None), packed, scales, biases (scales and
    biases in act_dtype), N, K).  Returns {name: fp64 y} and leaves the stored
    outputs in `buffers`."""
    rnd = f64_to_f16 if act_dtype == "f16" else f64_to_bf16
    out = {}
    for l in linears:
        N, K = l["N"], l["K"]
        x = buffers[l["x"]].reshape(1, K)
        if l.get("gate") is not None:
            r = None if l.get("resid") is None else buffers[l["resid"]].reshape(1, N)
            y = qmm_affine_silu_gate(buffers[l["gate"]].reshape(1, K), x, r, act_dtype, l["packed"], l["scales"],
                                     l["biases"], act_dtype, 1, N, K, G, bits)
        else:
            y = qmm_affine(x, act_dtype, l["packed"], l["scales"], l["biases"], act_dtype, 1, N, K, G, bits)
            if l.get("resid") is not None:
                y = y + to_f64(buffers[l["resid"]], act_dtype).reshape(1, N)
        out[l["name"]] = y.reshape(N)
        buffers[l["name"]] = rnd(y.reshape(N))
    return out


# ------------------------------------------------------------- SmoothQuant + W4A8

def smooth_factors(act_absmax, w, w_dtype: str, N: int, K: int, alpha: float) -> np.ndarray:
    a = _c(act_absmax, np.float32)
    wa = _sb(w, w_dtype)
    s = np.empty((K,), dtype=np.float32)
    _check(_load().oracle_smooth_factors(_p(a), _p(wa), C.c_int(_DT[w_dtype]), I64(N), I64(K), C.c_double(alpha),
                                         _p(s)), "smooth_factors")
    return s


def w4a8_quantize_weights(w, w_dtype: str, smooth, N: int, K: int):
    """Returns (w_q4 [N, K/8] u32, s_w [N] f16 bits)."""
    wa = _sb(w, w_dtype)
    sm = None if smooth is None else _c(smooth, np.float32)
    wq = np.empty((N, K // 8), dtype=np.uint32)
    sw = np.empty((N,), dtype=np.uint16)
    _check(_load().oracle_w4a8_quantize_weights(_p(wa), C.c_int(_DT[w_dtype]), _p(sm), I64(N), I64(K), _p(wq),
                                                _p(sw)), "w4a8_quantize_weights")
    return wq, sw


def w4a8_smooth(x, smooth, w_q4, s_w, M: int, N: int, K: int):
    """x / smooth per channel, then W4A8: (q_x, s_x, acc int64, y f64)."""
    xa, sm, w, sw = _c(x, np.uint16), _c(smooth, np.float32), _c(w_q4, np.uint32), _c(s_w, np.uint16)
    q = np.empty((M, K), dtype=np.int8)
    s = np.empty((M,), dtype=np.float32)
    acc = np.empty((M, N), dtype=np.int64)
    y = np.empty((M, N), dtype=np.float64)
    _check(_load().oracle_w4a8_smooth(_p(xa), _p(sm), _p(w), _p(sw), I64(M), I64(N), I64(K), _p(q), _p(s), _p(acc),
                                      _p(y)), "w4a8_smooth")
    return q, s, acc, y
