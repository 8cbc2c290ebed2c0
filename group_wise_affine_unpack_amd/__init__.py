"""Python binding of libqaff (group-wise affine quantized matmul, MI355X / gfx950).

Argument marshalling only: every computation runs in the HIP kernels of
libqaff.so, reached through its C ABI (include/qaff.h).  PyTorch supplies
device memory and the current HIP stream; nothing here computes.  There is no
CPU fallback: if the library is missing this module raises on first use.

Functions mirror the C entry points:
    qmm_affine, qgemv_affine, qgemv_affine_grouped, qmm_gptq, qgemm_w4a8,
    gptq_to_affine_repack, quantize_pack_affine
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

__all__ = ["QaffError", "qmm_affine", "qmm_affine_noalloc", "qgemv_affine", "qgemv_affine_grouped", "GroupedGemv", "qmm_gptq", "qgemm_w4a8", "qgemm_w4a8_tiled", "gptq_to_affine_repack",
           "quantize_pack_affine", "dequantize_affine", "qgemv_affine_silu_gate", "smoothquant_factors",
           "w4a8_quantize_weights", "qgemm_w4a8_smooth", "release_workspaces", "GemvChain", "library_path", "lib",
           "STATUS", "DTYPE"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqaff.so")

STATUS = {0: "QAFF_OK", 1: "QAFF_E_INVAL", 2: "QAFF_E_UNSUPPORTED", 3: "QAFF_E_ALIGN", 4: "QAFF_E_HIP"}
DTYPE = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}

_I64, _I32, _VP = C.c_int64, C.c_int32, C.c_void_p

# argument type lists of the exported symbols (include/qaff.h)
_SIGS = {
    "qmm_affine": [_VP] * 6 + [_I64] * 3 + [_I32] * 5 + [_VP],
    "qgemv_affine": [_VP] * 6 + [_I64] * 3 + [_I32] * 5 + [_VP],
    "qmm_affine_noalloc": [_VP] * 6 + [_I64] * 3 + [_I32] * 5 + [_VP],
    "qmm_gptq": [_VP] * 6 + [_I64] * 3 + [_I32, _VP],
    "qgemm_w4a8": [_VP] * 7 + [_I64] * 3 + [_VP],
    "qgemm_w4a8_tiled": [_VP] * 7 + [_I64] * 3 + [_I32] * 3 + [_VP],
    "gptq_to_affine_repack": [_VP] * 7 + [_I32, _VP] + [_I64] * 2 + [_I32, _VP],
    "quantize_pack_affine": [_VP, _I32, _VP, _VP, _VP, _I32, _I64, _I64, _I32, _I32, _VP],
    "qgemv_affine_grouped": [_VP, _I32, _I64] + [_I32] * 5 + [_VP],
    "dequantize_affine": [_VP] * 4 + [_I64] * 2 + [_I32] * 5 + [_VP],
    "qgemv_affine_silu_gate": [_VP] * 7 + [_I64] * 3 + [_I32] * 5 + [_VP],
    "smoothquant_factors": [_VP, _VP, _I32, C.c_double, _VP, _I64, _I64, _VP],
    "w4a8_quantize_weights": [_VP, _I32, _VP, _VP, _VP, _I64, _I64, _VP],
    "qgemm_w4a8_smooth": [_VP] * 8 + [_I64] * 3 + [_VP],
    "qaff_stream_read": [_VP, C.c_uint64, _VP, _I32, _VP],
    "qgemv_affine_chain_plan": [_VP, _I32, _I32, _I32, _I32, C.POINTER(_VP)],
    "qgemv_affine_chain_run": [_VP, _VP],
    "qgemv_affine_chain_status": [_VP, C.POINTER(_I32)],
    "qgemv_affine_chain_free": [_VP],
}


class GemvProblem(C.Structure):
    """qaff_gemv_problem (include/qaff.h)."""
    _fields_ = [("x", _VP), ("w_packed", _VP), ("scales", _VP), ("biases", _VP), ("k_perm", _VP), ("y", _VP),
                ("N", _I64), ("K", _I64)]


class ChainLinear(C.Structure):
    """qaff_chain_linear (include/qaff.h)."""
    _fields_ = [("x", _VP), ("gate", _VP), ("resid", _VP), ("w_packed", _VP), ("scales", _VP), ("biases", _VP),
                ("y", _VP), ("N", _I64), ("K", _I64), ("stage", _I32)]


class QaffError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libqaff.so (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        L = C.CDLL(_LIB_PATH)
        for name, argtypes in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = argtypes
            f.restype = C.c_int
        L.qaff_last_error.restype = C.c_char_p
        L.qaff_last_error.argtypes = []
        L.qaff_version.restype = C.c_int
        L.qaff_release_workspaces.restype = C.c_int
        L.qaff_release_workspaces.argtypes = [C.POINTER(C.c_uint64)]
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise QaffError(status, where, lib().qaff_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in DTYPE:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return DTYPE[t.dtype]


def _u32(t: torch.Tensor) -> torch.Tensor:
    # packed words travel as int32 or uint32 tensors; only the bits matter
    if t.dtype not in (torch.int32, torch.uint32):
        raise ValueError("packed words must be an int32/uint32 tensor")
    return t


def _affine(fn: str, x, w_packed, scales, biases, group_size, bits, k_perm, out):
    M, K = x.shape
    N = w_packed.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=x.dtype, device=x.device)
    st = getattr(lib(), fn)(_ptr(x), _ptr(_u32(w_packed)), _ptr(scales), _ptr(biases), _ptr(k_perm), _ptr(y), M, N, K,
                            group_size, bits, _dt(x), _dt(scales), _dt(biases), _stream(x.device))
    _check(st, fn)
    return y


def qmm_affine(x: torch.Tensor, w_packed: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
               group_size: int, bits: int, k_perm: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[M,N] = x[M,K] . W^T, W[n,k] = code*scale[n,k/G] + bias[n,k/G]."""
    return _affine("qmm_affine", x, w_packed, scales, biases, group_size, bits, k_perm, out)


def qmm_affine_noalloc(x: torch.Tensor, w_packed: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                       group_size: int, bits: int, k_perm: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """As qmm_affine, with the library's fixed scratch array (no device allocation)."""
    return _affine("qmm_affine_noalloc", x, w_packed, scales, biases, group_size, bits, k_perm, out)


def qgemv_affine(x, w_packed, scales, biases, group_size: int, bits: int, k_perm=None, out=None) -> torch.Tensor:
    """As qmm_affine, always on the GEMV kernel (M <= 16)."""
    return _affine("qgemv_affine", x, w_packed, scales, biases, group_size, bits, k_perm, out)


def qgemv_affine_silu_gate(gate, up, w_packed, scales, biases, group_size: int, bits: int, resid=None,
                           out=None) -> torch.Tensor:
    """y = W (silu(gate) * up) [+ resid] in one launch; gate/up [M, K], M <= 16."""
    M, K = gate.shape
    N = w_packed.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=gate.dtype, device=gate.device)
    st = lib().qgemv_affine_silu_gate(_ptr(gate), _ptr(up), _ptr(resid), _ptr(_u32(w_packed)), _ptr(scales),
                                      _ptr(biases), _ptr(y), M, N, K, group_size, bits, _dt(gate), _dt(scales),
                                      _dt(biases), _stream(gate.device))
    _check(st, "qgemv_affine_silu_gate")
    return y


def qgemv_affine_grouped(problems, group_size: int, bits: int, outs=None):
    """Independent GEMVs in as few launches as possible.

    problems: sequence of (x, w_packed, scales, biases) or (..., k_perm)
    tuples sharing M, dtypes, group_size and bits; returns the list of y.
    """
    n = len(problems)
    arr = (GemvProblem * max(n, 1))()
    ys = []
    for i, p in enumerate(problems):
        x, w, sc, bi = p[:4]
        kp = p[4] if len(p) > 4 else None
        M, K = x.shape
        N = w.shape[0]
        y = outs[i] if outs is not None else torch.empty((M, N), dtype=x.dtype, device=x.device)
        ys.append(y)
        arr[i] = GemvProblem(_ptr(x), _ptr(_u32(w)), _ptr(sc), _ptr(bi), _ptr(kp), _ptr(y), N, K)
    if n == 0:
        return ys
    x0, w0, s0, b0 = problems[0][:4]
    st = lib().qgemv_affine_grouped(C.cast(arr, _VP), n, x0.shape[0], group_size, bits, _dt(x0), _dt(s0), _dt(b0),
                                    _stream(x0.device))
    _check(st, "qgemv_affine_grouped")
    return ys


class GroupedGemv:
    """qgemv_affine_grouped with the descriptor array marshalled once.

    Holds references to every tensor it points at; calling it enqueues the
    GEMVs on the current stream of the device of the first x.
    """

    def __init__(self, problems, group_size: int, bits: int, outs=None):
        self.problems = [tuple(p) for p in problems]
        self.ys = []
        self.arr = (GemvProblem * max(len(problems), 1))()
        for i, p in enumerate(self.problems):
            x, w, sc, bi = p[:4]
            kp = p[4] if len(p) > 4 else None
            M, K = x.shape
            N = w.shape[0]
            y = outs[i] if outs is not None else torch.empty((M, N), dtype=x.dtype, device=x.device)
            self.ys.append(y)
            self.arr[i] = GemvProblem(_ptr(x), _ptr(_u32(w)), _ptr(sc), _ptr(bi), _ptr(kp), _ptr(y), N, K)
        x0, _, s0, b0 = self.problems[0][:4]
        self.args = (len(self.problems), x0.shape[0], group_size, bits, _dt(x0), _dt(s0), _dt(b0))
        self.device = x0.device

    def __call__(self):
        st = lib().qgemv_affine_grouped(C.cast(self.arr, _VP), *self.args, _stream(self.device))
        _check(st, "qgemv_affine_grouped")
        return self.ys


class GemvChain:
    """qgemv_affine_chain_plan / _run / _status / _free: linears of a decode
    step (one x row, 4-bit codes) in dependency stages, one launch per run.

    `linears`: dicts with x, w, s, b, y, stage and optionally gate, resid
    (tensors; x, gate [1, K] or [K], y and resid [1, N] or [N]).  Holds
    references to every tensor it points at; calling it enqueues the chain
    on the current stream of the device of the first x.
    """

    def __init__(self, linears, group_size: int, bits: int = 4):
        self.linears = [dict(l) for l in linears]
        arr = (ChainLinear * max(len(self.linears), 1))()
        for i, l in enumerate(self.linears):
            N, K = l["w"].shape[0], l["x"].shape[-1]
            arr[i] = ChainLinear(_ptr(l["x"]), _ptr(l.get("gate")), _ptr(l.get("resid")), _ptr(_u32(l["w"])),
                                 _ptr(l["s"]), _ptr(l["b"]), _ptr(l["y"]), N, K, int(l["stage"]))
        x0 = self.linears[0]["x"]
        self.device = x0.device
        self.plan = None
        h = _VP()
        with torch.cuda.device(self.device):
            st = lib().qgemv_affine_chain_plan(C.cast(arr, _VP), len(self.linears), group_size, bits, _dt(x0),
                                               C.byref(h))
        _check(st, "qgemv_affine_chain_plan")
        self.plan = h.value

    def __call__(self):
        st = lib().qgemv_affine_chain_run(self.plan, _stream(self.device))
        _check(st, "qgemv_affine_chain_run")

    def timed_out(self) -> bool:
        v = _I32(0)
        with torch.cuda.device(self.device):
            st = lib().qgemv_affine_chain_status(self.plan, C.byref(v))
        _check(st, "qgemv_affine_chain_status")
        return bool(v.value)

    def close(self):
        if self.plan is not None:
            with torch.cuda.device(self.device):
                st = lib().qgemv_affine_chain_free(self.plan)
            self.plan = None
            _check(st, "qgemv_affine_chain_free")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def qmm_gptq(x: torch.Tensor, qweight: torch.Tensor, qzeros: torch.Tensor, scales: torch.Tensor,
             g_idx: Optional[torch.Tensor], group_size: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x . W^T for a GPTQ layer (qweight [K/8,N], qzeros [K/G,N/8], scales f16 [K/G,N])."""
    M, K = x.shape
    N = qweight.shape[1]
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    st = lib().qmm_gptq(_ptr(x), _ptr(qweight), _ptr(qzeros), _ptr(scales), _ptr(g_idx), _ptr(y), M, N, K,
                        group_size, _stream(x.device))
    _check(st, "qmm_gptq")
    return y


def qgemm_w4a8(x: torch.Tensor, w_q4: torch.Tensor, s_w: torch.Tensor, want_acc: bool = False):
    """Returns (y f16 [M,N], x_q int8 [M,K], s_x f32 [M], acc int32 [M,N] or None)."""
    M, K = x.shape
    N = w_q4.shape[0]
    dev = x.device
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    x_q = torch.empty((M, K), dtype=torch.int8, device=dev)
    s_x = torch.empty((M,), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if want_acc else None
    st = lib().qgemm_w4a8(_ptr(x), _ptr(_u32(w_q4)), _ptr(s_w), _ptr(y), _ptr(x_q), _ptr(s_x), _ptr(acc), M, N, K,
                          _stream(dev))
    _check(st, "qgemm_w4a8")
    return y, x_q, s_x, acc


def qgemm_w4a8_tiled(x: torch.Tensor, w_q4: torch.Tensor, s_w: torch.Tensor, staged: bool, bm: int, bn: int,
                     want_acc: bool = False):
    """qgemm_w4a8 (M > 16) with the lowering (staged or full-K) and the bm x bn tile chosen."""
    M, K = x.shape
    N = w_q4.shape[0]
    dev = x.device
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    x_q = torch.empty((M, K), dtype=torch.int8, device=dev)
    s_x = torch.empty((M,), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if want_acc else None
    st = lib().qgemm_w4a8_tiled(_ptr(x), _ptr(_u32(w_q4)), _ptr(s_w), _ptr(y), _ptr(x_q), _ptr(s_x), _ptr(acc), M, N,
                                K, int(bool(staged)), bm, bn, _stream(dev))
    _check(st, "qgemm_w4a8_tiled")
    return y, x_q, s_x, acc


def smoothquant_factors(act_absmax: torch.Tensor, w: torch.Tensor, alpha: float = 0.5) -> torch.Tensor:
    """Per-input-channel smoothing factors s [K] f32 from calibration maxima of x and the dense weight w [N, K]."""
    N, K = w.shape
    s = torch.empty((K,), dtype=torch.float32, device=w.device)
    st = lib().smoothquant_factors(_ptr(act_absmax), _ptr(w), _dt(w), float(alpha), _ptr(s), N, K, _stream(w.device))
    _check(st, "smoothquant_factors")
    return s


def w4a8_quantize_weights(w: torch.Tensor, smooth: Optional[torch.Tensor] = None):
    """(w_q4 [N, K/8] int32, s_w [N] f16): the per-channel int4 weight, smoothing folded in when given."""
    N, K = w.shape
    wq = torch.empty((N, K // 8), dtype=torch.int32, device=w.device)
    sw = torch.empty((N,), dtype=torch.float16, device=w.device)
    st = lib().w4a8_quantize_weights(_ptr(w), _dt(w), _ptr(smooth), _ptr(wq), _ptr(sw), N, K, _stream(w.device))
    _check(st, "w4a8_quantize_weights")
    return wq, sw


def qgemm_w4a8_smooth(x: torch.Tensor, smooth: torch.Tensor, w_q4: torch.Tensor, s_w: torch.Tensor,
                      want_acc: bool = False):
    """qgemm_w4a8 on x / smooth: (y, x_q, s_x, acc or None)."""
    M, K = x.shape
    N = w_q4.shape[0]
    dev = x.device
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    x_q = torch.empty((M, K), dtype=torch.int8, device=dev)
    s_x = torch.empty((M,), dtype=torch.float32, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if want_acc else None
    st = lib().qgemm_w4a8_smooth(_ptr(x), _ptr(smooth), _ptr(_u32(w_q4)), _ptr(s_w), _ptr(y), _ptr(x_q), _ptr(s_x),
                                 _ptr(acc), M, N, K, _stream(dev))
    _check(st, "qgemm_w4a8_smooth")
    return y, x_q, s_x, acc


def gptq_to_affine_repack(qweight: torch.Tensor, qzeros: torch.Tensor, scales: torch.Tensor,
                          g_idx: Optional[torch.Tensor], group_size: int, bias_dtype=torch.float32):
    """Returns (w_packed [N,K/8] int32, scales [N,K/G] f16, biases [N,K/G] bias_dtype, k_perm [K] int32)."""
    K = qweight.shape[0] * 8
    N = qweight.shape[1]
    dev = qweight.device
    w = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    s = torch.empty((N, K // group_size), dtype=torch.float16, device=dev)
    b = torch.empty((N, K // group_size), dtype=bias_dtype, device=dev)
    kp = torch.empty((K,), dtype=torch.int32, device=dev)
    st = lib().gptq_to_affine_repack(_ptr(qweight), _ptr(qzeros), _ptr(scales), _ptr(g_idx), _ptr(w), _ptr(s),
                                     _ptr(b), DTYPE[bias_dtype], _ptr(kp), K, N, group_size, _stream(dev))
    _check(st, "gptq_to_affine_repack")
    return w, s, b, kp


def dequantize_affine(w_packed: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, K: int, group_size: int,
                      bits: int, out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The dense weight [N, K] in out_dtype: code*scale + bias, rounded once."""
    N = w_packed.shape[0]
    o = out if out is not None else torch.empty((N, K), dtype=out_dtype, device=w_packed.device)
    st = lib().dequantize_affine(_ptr(_u32(w_packed)), _ptr(scales), _ptr(biases), _ptr(o), N, K, group_size, bits,
                                 _dt(scales), _dt(biases), _dt(o), _stream(w_packed.device))
    _check(st, "dequantize_affine")
    return o


def stream_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int) -> None:
    """Measurement helper: read all of `buf` once (qaff_stream_read)."""
    st = lib().qaff_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), blocks, _stream(buf.device))
    _check(st, "qaff_stream_read")


def release_workspaces() -> int:
    """Free the scratch the library holds (qaff_release_workspaces).  Call it
    only with no library work pending on any stream and no captured graph
    that will replay a library call.  Returns the bytes of the per-stream
    buffers that were cached."""
    freed = C.c_uint64(0)
    _check(lib().qaff_release_workspaces(C.byref(freed)), "qaff_release_workspaces")
    return int(freed.value)


def quantize_pack_affine(w: torch.Tensor, group_size: int, bits: int, sb_dtype=torch.bfloat16):
    """Returns (w_packed [N, K*bits/32] int32, scales [N,K/G], biases [N,K/G])."""
    N, K = w.shape
    dev = w.device
    packed = torch.empty((N, K * bits // 32), dtype=torch.int32, device=dev)
    s = torch.empty((N, K // group_size), dtype=sb_dtype, device=dev)
    b = torch.empty((N, K // group_size), dtype=sb_dtype, device=dev)
    st = lib().quantize_pack_affine(_ptr(w), _dt(w), _ptr(packed), _ptr(s), _ptr(b), DTYPE[sb_dtype], N, K,
                                    group_size, bits, _stream(dev))
    _check(st, "quantize_pack_affine")
    return packed, s, b
