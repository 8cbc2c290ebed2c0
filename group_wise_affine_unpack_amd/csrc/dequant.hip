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
// words, so loads and stores are coalesced.  A workgroup finds the row of
// its first word with one scalar division; a lane's row is then that row or
// a few after it (rows of 256 or more words: at most one after, by a
// compare; shorter rows: by a multiplication with a 20-bit reciprocal,
// exact for the 511 words a workgroup can span).
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
                                                      long words, int wpr, uint32_t inv20, int ng, int gsh, int sdt,
                                                      int bdt) {
  constexpr int P = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const long base = (long)blockIdx.x * 256;  // the workgroup's first word
  const long i = base + threadIdx.x;
  if (i >= words) return;
  const long n0 = base / wpr;                // (uniform: scalar)
  int j = (int)(base - n0 * wpr) + (int)threadIdx.x;
  long n = n0;
  if (wpr >= 256) {  // uniform
    if (j >= wpr) {
      j -= wpr;
      ++n;
    }
  } else {
    const int q = (int)(((uint32_t)j * inv20) >> 20);  // j / wpr: j < 512, wpr < 256
    n += q;
    j -= q * wpr;
  }
  const int k0 = j * P;  // first column of this word
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

// 2- and 4-bit codes into bf16/f16: a group's 2^BITS possible outputs are
// computed once (the same exact fp64 evaluation and round-to-odd as above),
// by the group's own lanes, into an LDS table; each output is then a table
// read.  A lane takes two adjacent words (one group: G*BITS/32 = GW words
// is even) and stores their 2P outputs with 32-byte stores; the GW/2 lanes
// of one group are neighbours in one wave, so the table needs no barrier
// (one wave's LDS accesses execute in order).  Rows are an even number of
// words (K % G == 0), so a lane's words share a row.
template <int BITS, int OUT, int GW>
__global__ __launch_bounds__(256) void dequant_table_kernel(const uint32_t* __restrict__ w, const void* __restrict__ sc,
                                                            const void* __restrict__ bi, void* __restrict__ out,
                                                            long words, int wpr, uint32_t inv20, int ng, int gsh,
                                                            int sdt, int bdt) {
  constexpr int P = 32 / BITS, E = 1 << BITS, GL = GW / 2;  // GL lanes per group
  __shared__ uint16_t tab[256 / GL * E];
  const long base = (long)blockIdx.x * 512;  // the workgroup's first word
  const long i = base + 2 * threadIdx.x;     // this lane's first word
  if (i >= words) return;  // (a whole group past the end: words is a multiple of GW)
  const long n0 = base / wpr;
  int j = (int)(base - n0 * wpr) + 2 * (int)threadIdx.x;
  long n = n0;
  if (wpr >= 512) {  // uniform
    if (j >= wpr) {
      j -= wpr;
      ++n;
    }
  } else {
    const int q = (int)(((uint32_t)j * inv20) >> 20);  // j / wpr: j < 1024, wpr < 512
    n += q;
    j -= q * wpr;
  }
  const long gi = n * ng + ((j * P) >> gsh);
  const double s = load_f64(sc, gi, sdt), b = load_f64(bi, gi, bdt);
  const u32x2_t word = *reinterpret_cast<const u32x2_t*>(w + i);
  // this lane's share of the group's table
  const int lt = (int)threadIdx.x % GL, row = ((int)threadIdx.x / GL) * E;
#pragma unroll
  for (int e0 = 0; e0 < E; e0 += GL) {
    const int e = e0 + lt;
    if (e < E) {
      const float a = f64_to_f32_odd(fma((double)e, s, b));
      tab[row + e] = OUT == BF16 ? f32_to_bf16_bits(a) : f32_to_f16_bits(a);
    }
  }
  const uint16_t* tr = tab + row;
  uint32_t h[P];
#pragma unroll
  for (int k = 0; k < 2 * P; k += 2) {
    const uint32_t wd = word[k / P];
    const int c = k % P;
    h[k / 2] = (uint32_t)tr[__builtin_amdgcn_ubfe(wd, BITS * c, BITS)] |
               ((uint32_t)tr[__builtin_amdgcn_ubfe(wd, BITS * (c + 1), BITS)] << 16);
  }
  uint16_t* o = static_cast<uint16_t*>(out) + i * P;
#pragma unroll
  for (int k = 0; k < P; k += 4) *reinterpret_cast<u32x4_t*>(o + 2 * k) = u32x4_t{h[k], h[k + 1], h[k + 2], h[k + 3]};
}

template <int BITS, int GW>
void launch_table(int odt, dim3 grid, hipStream_t st, const uint32_t* w, const void* s, const void* b, void* out, long words,
                  int wpr, uint32_t inv20, int ng, int gsh, int sdt, int bdt) {
  if (odt == F16)
    hipLaunchKernelGGL((dequant_table_kernel<BITS, F16, GW>), grid, dim3(256), 0, st, w, s, b, out, words, wpr, inv20, ng,
                       gsh, sdt, bdt);
  else
    hipLaunchKernelGGL((dequant_table_kernel<BITS, BF16, GW>), grid, dim3(256), 0, st, w, s, b, out, words, wpr, inv20, ng,
                       gsh, sdt, bdt);
}

template <int BITS>
hipError_t run_dequant(const uint32_t* w, const void* s, const void* b, void* out, int64_t N, int64_t K, int G,
                       int sdt, int bdt, int odt, hipStream_t st) {
  const int wpr = (int)(K * BITS / 32);
  const long words = (long)N * wpr;
  const uint32_t inv20 = (uint32_t)(((1u << 20) + wpr - 1) / wpr);  // ceil(2^20 / wpr)
  const int ng = (int)(K / G);
  const int gsh = G == 32 ? 5 : (G == 64 ? 6 : 7);
  const dim3 grid((unsigned)((words + 255) / 256));
  if constexpr (BITS <= 4) {
    // a group's lanes: G*BITS/32 words (2..16) two per lane, all in one wave
    if (odt != F32) {
      const dim3 grid2((unsigned)((words + 511) / 512));
      const int gw = G * BITS / 32;
      if (gw == 32 * BITS / 32) launch_table<BITS, 32 * BITS / 32>(odt, grid2, st, w, s, b, out, words, wpr, inv20, ng, gsh, sdt, bdt);
      else if (gw == 64 * BITS / 32) launch_table<BITS, 64 * BITS / 32>(odt, grid2, st, w, s, b, out, words, wpr, inv20, ng, gsh, sdt, bdt);
      else launch_table<BITS, 128 * BITS / 32>(odt, grid2, st, w, s, b, out, words, wpr, inv20, ng, gsh, sdt, bdt);
      return hipGetLastError();
    }
  }
  if (odt == F32)
    hipLaunchKernelGGL((dequant_kernel<BITS, F32>), grid, dim3(256), 0, st, w, s, b, out, words, wpr, inv20, ng, gsh, sdt, bdt);
  else if (odt == F16)
    hipLaunchKernelGGL((dequant_kernel<BITS, F16>), grid, dim3(256), 0, st, w, s, b, out, words, wpr, inv20, ng, gsh, sdt, bdt);
  else
    hipLaunchKernelGGL((dequant_kernel<BITS, BF16>), grid, dim3(256), 0, st, w, s, b, out, words, wpr, inv20, ng, gsh, sdt, bdt);
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
