// Standalone dequantization of group-wise affine weights into a dense
// array: out[n, k] = q(n,k) * scale[n, k/G] + bias[n, k/G], rounded once to
// the output type (the mlx_int8.rs API page, `dequantize_to`, writes the
// whole weight as BF16; the Transformers "Metal" page, "Dequantize" section,
// gives the packed -> float direction).
//
// Each weight is evaluated exactly in fp64 (the code times a 16-bit or fp32
// scale needs at most 32 significant bits; the bias is added with one
// fp64 rounding, which for 16-bit parameters is exact), then rounded to the
// output type with round-to-nearest-even:
//   f32:      one conversion (v_cvt_f32_f64 rounds to nearest even);
//   bf16/f16: round-to-odd into fp32, then the nearest-even conversion.
//             fp32 carries at least two more bits than either target, so
//             the pair of roundings equals a single rounding of the exact
//             value (rounding to odd first removes the double-rounding
//             error at ties).
// Memory-bound: one thread per packed word, P = 32/bits outputs per thread,
// written with 8..64-byte stores; consecutive threads take consecutive
// words, so loads and stores are coalesced.
#include "common.h"

namespace qaff {
namespace {

// fp64 -> fp32, rounding to odd: truncate toward zero, and set the last bit
// when anything was dropped
__device__ __forceinline__ float f64_to_f32_odd(double d) {
  const float f = (float)d;  // nearest even
  const double back = (double)f;
  if (back == d) return f;
  uint32_t u = __float_as_uint(f);
  if (fabs(back) > fabs(d)) u -= 1u;  // rounded away from zero: one step back toward it
  return __uint_as_float(u | 1u);
}

__device__ __forceinline__ double load_f64(const void* base, long i, int dt) {
  if (dt == BF16) return (double)bf16_bits_to_f32(((const uint16_t*)base)[i]);
  if (dt == F16) return (double)f16_bits_to_f32(((const uint16_t*)base)[i]);
  return (double)((const float*)base)[i];
}

template <int BITS, int OUT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ w, const void* __restrict__ sc,
                                                      const void* __restrict__ bi, void* __restrict__ out,
                                                      long words, int wpr, int ng, int gsh, int sdt, int bdt) {
  constexpr int P = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= words) return;
  const long n = i / wpr;
  const int k0 = (int)(i % wpr) * P;  // first column of this word
  const long gi = n * ng + (k0 >> gsh);  // a word never spans two groups (P <= 16 <= G)
  const double s = load_f64(sc, gi, sdt), b = load_f64(bi, gi, bdt);
  const uint32_t word = w[i];
  if constexpr (OUT == F32) {
    float v[P];
#pragma unroll
    for (int j = 0; j < P; ++j) v[j] = (float)fma((double)((word >> (BITS * j)) & MASK), s, b);
    float* o = static_cast<float*>(out) + i * P;
#pragma unroll
    for (int j = 0; j < P; j += 4) *reinterpret_cast<f32x4_t*>(o + j) = f32x4_t{v[j], v[j + 1], v[j + 2], v[j + 3]};
  } else {
    uint32_t h[P / 2];
#pragma unroll
    for (int j = 0; j < P; j += 2) {
      // q*s is exact in fp64, so the fused form rounds exactly as q*s + b
      const float a0 = f64_to_f32_odd(fma((double)((word >> (BITS * j)) & MASK), s, b));
      const float a1 = f64_to_f32_odd(fma((double)((word >> (BITS * (j + 1))) & MASK), s, b));
      const uint32_t lo = OUT == BF16 ? f32_to_bf16_bits(a0) : f32_to_f16_bits(a0);
      const uint32_t hi = OUT == BF16 ? f32_to_bf16_bits(a1) : f32_to_f16_bits(a1);
      h[j / 2] = lo | (hi << 16);
    }
    uint16_t* o = static_cast<uint16_t*>(out) + i * P;
    if constexpr (P == 4) {
      *reinterpret_cast<u32x2_t*>(o) = u32x2_t{h[0], h[1]};
    } else {
#pragma unroll
      for (int j = 0; j < P / 2; j += 4) *reinterpret_cast<u32x4_t*>(o + 2 * j) = u32x4_t{h[j], h[j + 1], h[j + 2], h[j + 3]};
    }
  }
}

template <int BITS>
hipError_t run_dequant(const uint32_t* w, const void* s, const void* b, void* out, int64_t N, int64_t K, int G,
                       int sdt, int bdt, int odt, hipStream_t st) {
  const int wpr = (int)(K * BITS / 32);
  const long words = (long)N * wpr;
  const int ng = (int)(K / G);
  const int gsh = G == 32 ? 5 : (G == 64 ? 6 : 7);
  const dim3 grid((unsigned)((words + 255) / 256));
  if (odt == F32)
    hipLaunchKernelGGL((dequant_kernel<BITS, F32>), grid, dim3(256), 0, st, w, s, b, out, words, wpr, ng, gsh, sdt, bdt);
  else if (odt == F16)
    hipLaunchKernelGGL((dequant_kernel<BITS, F16>), grid, dim3(256), 0, st, w, s, b, out, words, wpr, ng, gsh, sdt, bdt);
  else
    hipLaunchKernelGGL((dequant_kernel<BITS, BF16>), grid, dim3(256), 0, st, w, s, b, out, words, wpr, ng, gsh, sdt, bdt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const uint32_t* w, const void* s, const void* b, void* out, int64_t N, int64_t K, int G,
                          int bits, int sdt, int bdt, int odt, hipStream_t st) {
  if (N * (K * bits / 32) >= (int64_t(1) << 40)) return hipErrorNotSupported;
  switch (bits) {
    case 2: return run_dequant<2>(w, s, b, out, N, K, G, sdt, bdt, odt, st);
    case 4: return run_dequant<4>(w, s, b, out, N, K, G, sdt, bdt, odt, st);
    default: return run_dequant<8>(w, s, b, out, N, K, G, sdt, bdt, odt, st);
  }
}

}  // namespace qaff
