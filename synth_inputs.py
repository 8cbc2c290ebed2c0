"""Seeded synthetic inputs for the fused dequant + matmul path.

This module is shared by the CPU oracle tests, the GPU parity tests, the smoke
check and the benchmark. It holds none of the method's arithmetic: it draws
random numbers, rounds them to their storage dtype with torch's own converters,
and lays integer codes out in 32-bit words. Decoding those words, dequantizing
and multiplying is done separately by the oracle and by the HIP kernels.

Arrays are numpy. Half-precision tensors are carried as their raw 16-bit
patterns (``np.uint16``) together with a dtype tag ("bf16" or "f16"), so the
same bytes reach both sides.

Recipes follow the workloads on the pages:
  * affine 2/4/8-bit weights with per-group scales and biases, uint32 words
    with the lowest column in the low bits (metrale_gpu_runtime mlx_int8.rs,
    module docs "Layout"; Transformers "Metal" quantization page, intro);
  * GPTQ quartets qweight/qzeros/scales/g_idx (TinyGPT "Quantization
    Expansion", section 1 "GPTQReader", "Format");
  * W4A8 int8-activation x int4-weight GEMM inputs (executorch PR #24467,
    "What this adds").
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# --------------------------------------------------------------------------
# storage-dtype helpers (torch's converters; round-to-nearest-even)


def bf16_bits(a) -> np.ndarray:
    """Round float values to bfloat16 and return the raw 16-bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def f16_bits(a) -> np.ndarray:
    """Round float values to IEEE half and return the raw 16-bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored 16-bit patterns (or f32 values) to float32 (exact)."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.to(torch.float32).numpy()


def store(values_f32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to a storage dtype ("bf16", "f16" or "f32")."""
    if dtype == "bf16":
        return bf16_bits(values_f32)
    if dtype == "f16":
        return f16_bits(values_f32)
    if dtype == "f32":
        return np.ascontiguousarray(values_f32, dtype=np.float32)
    raise ValueError(dtype)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def pack_nibbles_along_last(nib: np.ndarray) -> np.ndarray:
    """Lay 4-bit values out 8 per uint32 word along the last axis, the first
    value of each run of 8 in the low nibble (the layout the GPTQ qzeros
    tensor and the W4A8 weight use)."""
    nib = np.asarray(nib, dtype=np.uint32) & np.uint32(0xF)
    *lead, L = nib.shape
    assert L % 8 == 0
    v = nib.reshape(*lead, L // 8, 8)
    word = np.zeros((*lead, L // 8), dtype=np.uint32)
    for j in range(8):
        word |= v[..., j] << np.uint32(4 * j)
    return word


# --------------------------------------------------------------------------
# affine (MLX-layout) weights


@dataclass
class AffineCase:
    M: int
    N: int
    K: int
    G: int
    bits: int
    x: np.ndarray            # [M, K] uint16 patterns, act_dtype
    packed: np.ndarray       # [N, K*bits/32] uint32
    scales: np.ndarray       # [N, K/G] uint16 patterns or float32
    biases: np.ndarray       # [N, K/G]
    act_dtype: str = "bf16"
    sb_dtype: str = "bf16"
    k_perm: Optional[np.ndarray] = None   # [K] int32 or None
    name: str = ""
    bias_dtype: Optional[str] = None      # defaults to sb_dtype

    def __post_init__(self):
        if self.bias_dtype is None:
            self.bias_dtype = self.sb_dtype


def affine_weights(N: int, K: int, G: int, bits: int, *, seed, scale_range,
                   bias_mode: str, sb_dtype: str = "bf16"):
    """Packed codes plus per-group scales and biases.

    Codes are independent and uniform over 0..2^bits-1, so every bit of every
    word is an independent fair coin: the words are drawn directly as uniform
    uint32.  Scales are uniform in ``scale_range``.  ``bias_mode``:
      * "noise":  bias = -2^(bits-1) * scale_stored + U(-0.002, 0.002)
      * "exact":  bias = -2^(bits-1) * scale_stored  (exact in the dtype)
    """
    r = _rng(*seed)
    words_per_row = K * bits // 32
    packed = r.integers(0, 2**32, size=(N, words_per_row), dtype=np.uint64).astype(np.uint32)
    lo, hi = scale_range
    s32 = r.uniform(lo, hi, size=(N, K // G)).astype(np.float32)
    scales = store(s32, sb_dtype)
    s_stored = bits_to_f32(scales, sb_dtype) if sb_dtype != "f32" else scales
    half = np.float32(2 ** (bits - 1))
    if bias_mode == "noise":
        noise = r.uniform(-0.002, 0.002, size=(N, K // G)).astype(np.float32)
        b32 = (-half * s_stored + noise).astype(np.float32)
    elif bias_mode == "exact":
        b32 = (-half * s_stored).astype(np.float32)
    else:
        raise ValueError(bias_mode)
    biases = store(b32, sb_dtype)
    return packed, scales, biases


def activations(M: int, K: int, *, seed, dtype: str = "bf16", outlier_frac: float = 0.0,
                outlier_mult: float = 20.0) -> np.ndarray:
    """x ~ N(0, 1), optionally with a Bernoulli(outlier_frac) fraction of
    elements multiplied by ``outlier_mult`` before rounding."""
    r = _rng(*seed)
    x = r.standard_normal(size=(M, K)).astype(np.float32)
    if outlier_frac > 0:
        mask = r.random(size=(M, K)) < outlier_frac
        x = np.where(mask, x * np.float32(outlier_mult), x).astype(np.float32)
    return store(x, dtype)


def affine_case(M: int, N: int, K: int, G: int = 64, bits: int = 4, *, seed=(0,),
                scale_range=(0.005, 0.02), bias_mode: str = "noise",
                act_dtype: str = "bf16", sb_dtype: str = "bf16", name: str = "") -> AffineCase:
    packed, scales, biases = affine_weights(N, K, G, bits, seed=(*seed, 1), scale_range=scale_range,
                                            bias_mode=bias_mode, sb_dtype=sb_dtype)
    x = activations(M, K, seed=(*seed, 2), dtype=act_dtype)
    return AffineCase(M, N, K, G, bits, x, packed, scales, biases, act_dtype, sb_dtype, None, name)


# The workloads -----------------------------------------------------------

# Single 4-bit affine linear (decode, one token)
CFG0 = dict(M=1, N=2048, K=2048, G=64, bits=4)

# Decode GEMV set shaped like a 1B-parameter decoder (hidden 2048, FFN 8192):
# (name, N, K); gate and up are two distinct 8192x2048 matrices.
CFG1_LINEARS = [
    ("q", 2048, 2048), ("k", 512, 2048), ("v", 512, 2048), ("o", 2048, 2048),
    ("gate", 8192, 2048), ("up", 8192, 2048), ("down", 2048, 8192),
]
CFG1_M = (1, 4, 16)

# Prefill GEMM shaped like an 8B-parameter decoder: (N, K) at M=2048
CFG2_SHAPES = [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)]
CFG2_M = 2048
CFG2_BITS = (4, 8)

# GPTQ act-order layer
CFG3 = dict(K=4096, N=11008, G=128)
CFG3_M = (1, 32)

# W4A8 speech-encoder-like shapes: (N, K)
CFG4_SHAPES = [(1024, 1024), (4096, 1024), (1024, 4096)]
CFG4_M = (8, 128, 2048)


def cfg0_case(seed=(0, 0, 0)) -> AffineCase:
    return affine_case(**CFG0, seed=seed, scale_range=(0.005, 0.02), bias_mode="noise", name="cfg0")


def cfg1_case(N: int, K: int, M: int, seed) -> AffineCase:
    return affine_case(M, N, K, 64, 4, seed=seed, scale_range=(0.005, 0.02), bias_mode="noise",
                       name=f"cfg1_{N}x{K}_M{M}")


def cfg2_case(N: int, K: int, bits: int, M: int = CFG2_M, seed=(2, 0, 0)) -> AffineCase:
    return affine_case(M, N, K, 64, bits, seed=seed, scale_range=(0.002, 0.01), bias_mode="exact",
                       name=f"cfg2_{N}x{K}_b{bits}_M{M}")


# --------------------------------------------------------------------------
# GPTQ quartet


@dataclass
class GptqCase:
    M: int
    K: int
    N: int
    G: int
    x: np.ndarray         # [M, K] f16 patterns
    qweight: np.ndarray   # [K/8, N] int32
    qzeros: np.ndarray    # [K/G, N/8] int32, stores zero-1
    scales: np.ndarray    # [K/G, N] f16 patterns
    g_idx: Optional[np.ndarray]   # [K] int32 or None
    name: str = ""
    zeros: np.ndarray = field(default=None, repr=False)  # [K/G, N] drawn zero points (1..16 range)


def gptq_case(M: int, K: int, N: int, G: int = 128, *, seed=(3, 0, 0), act_order: bool = True,
              zero_range=(6, 10), scale_range=(0.005, 0.02), name: str = "") -> GptqCase:
    """qweight codes uniform 0..15 (uniform words); zero points uniform in
    ``zero_range`` stored as zero-1; scales fp16 uniform; g_idx = pi(i) // G
    for a seeded permutation pi of 0..K-1 (act-order), else i // G."""
    r = _rng(*seed)
    qweight = r.integers(0, 2**32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32).view(np.int32)
    s32 = r.uniform(*scale_range, size=(K // G, N)).astype(np.float32)
    scales = f16_bits(s32)
    zeros = r.integers(zero_range[0], zero_range[1] + 1, size=(K // G, N)).astype(np.uint32)
    qzeros = pack_nibbles_along_last(zeros - 1).view(np.int32)
    if act_order:
        pi = r.permutation(K)
        g_idx = (pi // G).astype(np.int32)
    else:
        g_idx = (np.arange(K) // G).astype(np.int32)
    x = activations(M, K, seed=(*seed, 9), dtype="f16")
    return GptqCase(M, K, N, G, x, qweight, qzeros, scales, g_idx, name, zeros)


def cfg3_case(M: int, seed=(3, 0, 0)) -> GptqCase:
    return gptq_case(M, CFG3["K"], CFG3["N"], CFG3["G"], seed=(*seed[:2], M), act_order=True,
                     name=f"cfg3_M{M}")


# --------------------------------------------------------------------------
# W4A8


@dataclass
class W4A8Case:
    M: int
    N: int
    K: int
    x: np.ndarray      # [M, K] f16 patterns
    w_q4: np.ndarray   # [N, K/8] uint32, two's-complement nibbles, low nibble = lowest k
    s_w: np.ndarray    # [N] f16 patterns
    name: str = ""
    codes: np.ndarray = field(default=None, repr=False)  # [N, K] int8 drawn weight codes


def w4a8_case(M: int, N: int, K: int, *, seed=(4, 0, 0), outlier_frac: float = 0.01,
              name: str = "") -> W4A8Case:
    """Weights w ~ N(0, 0.02) [N, K]; per-row s_w = fp16(max|w| / 7);
    codes = clamp(rint(w / s_w), -8, 7) stored as two's-complement nibbles.
    Activations x ~ N(0, 1) in fp16 with ``outlier_frac`` of elements x20."""
    r = _rng(*seed)
    w = (r.standard_normal(size=(N, K)) * 0.02).astype(np.float32)
    amax = np.abs(w).max(axis=1)
    s_w = f16_bits(amax / np.float32(7.0))
    s_f = bits_to_f32(s_w, "f16")
    codes = np.clip(np.rint(w / s_f[:, None]), -8, 7).astype(np.int8)
    w_q4 = pack_nibbles_along_last(codes.astype(np.int32) & 0xF)
    x = activations(M, K, seed=(*seed, 9), dtype="f16", outlier_frac=outlier_frac)
    return W4A8Case(M, N, K, x, w_q4, s_w, name, codes)


def cfg4_case(N: int, K: int, M: int, seed=(4, 0, 0)) -> W4A8Case:
    return w4a8_case(M, N, K, seed=seed, name=f"cfg4_{N}x{K}_M{M}")


# --------------------------------------------------------------------------
# dense weights for quantize_pack_affine


def dense_weights(N: int, K: int, *, seed, dtype: str = "bf16", std: float = 0.02) -> np.ndarray:
    r = _rng(*seed)
    w = (r.standard_normal(size=(N, K)) * std).astype(np.float32)
    return store(w, dtype)


def sample_indices(total: int, count: int, *, seed, include_edges: bool = True) -> np.ndarray:
    """Sorted distinct indices in [0, total): ``count`` of them, always including
    the first and last (ragged tails are where indexing mistakes show)."""
    count = min(count, total)
    r = _rng(*seed)
    idx = set(r.choice(total, size=count, replace=False).tolist())
    if include_edges:
        idx |= {0, total - 1}
    return np.array(sorted(idx), dtype=np.int64)
