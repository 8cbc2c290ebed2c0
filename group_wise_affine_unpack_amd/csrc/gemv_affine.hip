// Decode GEMV for group-wise affine weights, M <= 16 (memory-bound path).
//
//   y[m, n] = sum_k x[m, k] * (q(n,k) * scale[n, k/G] + bias[n, k/G])
//
// The weight layout (uint32 words, lowest column in the low bits, per-group
// scale and bias) is the one of the mlx_int8.rs API page ("Layout") and of
// the Transformers "Metal" quantization page (bits 2/4/8).
//
// Design for CDNA4:
//  * one 16-byte (dwordx4) load per lane per weight chunk; 64 lanes of a wave
//    read 1 KiB of one row, fully coalesced;
//  * the lane's slice of x is decoded once into registers and reused for R
//    rows; codes are turned into exact half-precision values with the
//    exponent-bias trick (code | 0x4300 is 128+code in bf16, code | 0x6400 is
//    1024+code in f16) and fed to v_dot2c_f32_{bf16,f16}, two products per
//    instruction, fp32 accumulate;
//  * per group segment the lane applies its scale and bias to its own partial
//    sum:  s*sum(c*x) + (b - off*s)*sum(x), which keeps every weight exact;
//  * split-K across the 4 waves of a workgroup for long rows, DPP row
//    rotations + two cross-row swaps to reduce a wave, LDS to combine waves.
#include "common.h"

namespace qaff {
namespace {

template <typename T>
__device__ __forceinline__ T bc(uint32_t v) { return __builtin_bit_cast(T, v); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(bc<bf16x2_t>(a), bc<bf16x2_t>(b), c, false);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(bc<f16x2_t>(a), bc<f16x2_t>(b), c, false);
}
__device__ __forceinline__ float half_to_f32(uint32_t h, bool f16) {
  return f16 ? f16_bits_to_f32(h & 0xffffu) : bf16_bits_to_f32(h & 0xffffu);
}

// Natural pairs p[i] = (x[k0 + 2i], x[k0 + 2i + 1]) for NP pairs, direct or
// through the column permutation.
template <int NP>
__device__ __forceinline__ void load_pairs(const uint16_t* __restrict__ xrow, const int32_t* __restrict__ kp, int k0,
                                           uint32_t (&p)[NP]) {
  if (kp == nullptr) {
    const uint4* src = reinterpret_cast<const uint4*>(xrow + k0);
#pragma unroll
    for (int i = 0; i < NP / 4; ++i) {
      uint4 v = src[i];
      p[4 * i + 0] = v.x;
      p[4 * i + 1] = v.y;
      p[4 * i + 2] = v.z;
      p[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      uint32_t lo = xrow[kp[k0 + 2 * i]], hi = xrow[kp[k0 + 2 * i + 1]];
      p[i] = lo | (hi << 16);
    }
  }
}

// (lo half of a, lo half of b) or (hi half of a, hi half of b)
__device__ __forceinline__ uint32_t pick(uint32_t a, uint32_t b, int hi) {
  return hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

// One codec per (bits, activation dtype): how a lane's x slice is held, and
// how a 16-byte weight chunk is dotted with it.
template <int BITS, bool F16>
struct Codec;

// 4-bit codes: word w holds codes 8w..8w+7; ((w >> 4i) & 0x000F000F) gives the
// pair (code i, code i+4) in the two halves.  x is held as the matching pairs.
template <bool F16>
struct Codec<4, F16> {
  static constexpr int CPL = 32, NSEG = 1, SEGK = 32;
  static constexpr float OFF = F16 ? 1024.f : 128.f;
  static constexpr uint32_t MAGIC = F16 ? 0x64006400u : 0x43004300u;
  struct XSlice {
    uint32_t q[16];
    float sum[NSEG];
  };
  static __device__ __forceinline__ void load(const uint16_t* xrow, const int32_t* kp, int k0, XSlice& s) {
    uint32_t p[16];
    load_pairs<16>(xrow, kp, k0, p);
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += half_to_f32(p[i], F16) + half_to_f32(p[i] >> 16, F16);
    s.sum[0] = t;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) s.q[4 * w + i] = pick(p[4 * w + i / 2], p[4 * w + 2 + i / 2], i & 1);
  }
  static __device__ __forceinline__ void zero(XSlice& s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s.q[i] = 0;
    s.sum[0] = 0.f;
  }
  static __device__ __forceinline__ float dot(const uint4& c, const XSlice& s, int) {
    const uint32_t ww[4] = {c.x, c.y, c.z, c.w};
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t pr = ((ww[w] >> (4 * i)) & 0x000F000Fu) | MAGIC;
        acc = F16 ? dot2_f16(pr, s.q[4 * w + i], acc) : dot2_bf16(pr, s.q[4 * w + i], acc);
      }
    return acc;
  }
};

// 2-bit codes: word w holds codes 16w..16w+15; ((w >> 2i) & 0x00030003) is
// the pair (code i, code i+8).  A chunk is 64 codes = two 32-code segments,
// each inside one group (G >= 32).
template <bool F16>
struct Codec<2, F16> {
  static constexpr int CPL = 64, NSEG = 2, SEGK = 32;
  static constexpr float OFF = F16 ? 1024.f : 128.f;
  static constexpr uint32_t MAGIC = F16 ? 0x64006400u : 0x43004300u;
  struct XSlice {
    uint32_t q[32];
    float sum[NSEG];
  };
  static __device__ __forceinline__ void load(const uint16_t* xrow, const int32_t* kp, int k0, XSlice& s) {
    uint32_t p[32];
    load_pairs<32>(xrow, kp, k0, p);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float t = 0.f;
#pragma unroll
      for (int i = 16 * h; i < 16 * h + 16; ++i) t += half_to_f32(p[i], F16) + half_to_f32(p[i] >> 16, F16);
      s.sum[h] = t;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int i = 0; i < 8; ++i) s.q[8 * w + i] = pick(p[8 * w + i / 2], p[8 * w + 4 + i / 2], i & 1);
  }
  static __device__ __forceinline__ void zero(XSlice& s) {
#pragma unroll
    for (int i = 0; i < 32; ++i) s.q[i] = 0;
    s.sum[0] = s.sum[1] = 0.f;
  }
  static __device__ __forceinline__ float dot(const uint4& c, const XSlice& s, int seg) {
    const uint32_t ww[4] = {c.x, c.y, c.z, c.w};
    float acc = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 2; ++w2) {
      const int w = 2 * seg + w2;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t pr = ((ww[w] >> (2 * i)) & 0x00030003u) | MAGIC;
        acc = F16 ? dot2_f16(pr, s.q[8 * w + i], acc) : dot2_bf16(pr, s.q[8 * w + i], acc);
      }
    }
    return acc;
  }
};

// 8-bit codes with bf16 activations: bytes to fp32 (v_cvt_f32_ubyte*) and
// fp32 FMA; 128+code does not fit a bf16 significand.
template <>
struct Codec<8, false> {
  static constexpr int CPL = 16, NSEG = 1, SEGK = 16;
  static constexpr float OFF = 0.f;
  struct XSlice {
    float f[16];
    float sum[NSEG];
  };
  static __device__ __forceinline__ void load(const uint16_t* xrow, const int32_t* kp, int k0, XSlice& s) {
    uint32_t p[8];
    load_pairs<8>(xrow, kp, k0, p);
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s.f[2 * i] = bf16_bits_to_f32(p[i] & 0xffffu);
      s.f[2 * i + 1] = bf16_bits_to_f32(p[i] >> 16);
      t += s.f[2 * i] + s.f[2 * i + 1];
    }
    s.sum[0] = t;
  }
  static __device__ __forceinline__ void zero(XSlice& s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s.f[i] = 0.f;
    s.sum[0] = 0.f;
  }
  static __device__ __forceinline__ float dot(const uint4& c, const XSlice& s, int) {
    const uint32_t ww[4] = {c.x, c.y, c.z, c.w};
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf((float)((ww[w] >> (8 * e)) & 0xffu), s.f[4 * w + e], acc);
    return acc;
  }
};

// 8-bit codes with f16 activations: v_perm_b32 builds (0x6400|b0, 0x6400|b2)
// and (0x6400|b1, 0x6400|b3) = 1024+code, exact in f16.
template <>
struct Codec<8, true> {
  static constexpr int CPL = 16, NSEG = 1, SEGK = 16;
  static constexpr float OFF = 1024.f;
  struct XSlice {
    uint32_t q[8];
    float sum[NSEG];
  };
  static __device__ __forceinline__ void load(const uint16_t* xrow, const int32_t* kp, int k0, XSlice& s) {
    uint32_t p[8];
    load_pairs<8>(xrow, kp, k0, p);
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += half_to_f32(p[i], true) + half_to_f32(p[i] >> 16, true);
    s.sum[0] = t;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s.q[2 * w] = pick(p[2 * w], p[2 * w + 1], 0);      // (x[4w], x[4w+2])
      s.q[2 * w + 1] = pick(p[2 * w], p[2 * w + 1], 1);  // (x[4w+1], x[4w+3])
    }
  }
  static __device__ __forceinline__ void zero(XSlice& s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s.q[i] = 0;
    s.sum[0] = 0.f;
  }
  static __device__ __forceinline__ float dot(const uint4& c, const XSlice& s, int) {
    const uint32_t ww[4] = {c.x, c.y, c.z, c.w};
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t p02 = __builtin_amdgcn_perm(0x64646464u, ww[w], 0x04020400u);
      uint32_t p13 = __builtin_amdgcn_perm(0x64646464u, ww[w], 0x04030401u);
      acc = dot2_f16(p02, s.q[2 * w], acc);
      acc = dot2_f16(p13, s.q[2 * w + 1], acc);
    }
    return acc;
  }
};

// Grid: blockIdx.x covers (4/KS)*R rows.  Wave w works on row group w/KS and
// on the K chunks c = w%KS, w%KS + KS, ...; a chunk is 64 lanes x 16 bytes.
template <int BITS, bool F16, int MT, int R>
__global__ __launch_bounds__(256) void gemv_affine_kernel(const uint16_t* __restrict__ x, const uint4* __restrict__ w,
                                                          const void* __restrict__ scales,
                                                          const void* __restrict__ biases,
                                                          const int32_t* __restrict__ k_perm,
                                                          uint16_t* __restrict__ y, int M, int N, int K, int G,
                                                          int sdt, int bdt, int KS) {
  using C = Codec<BITS, F16>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rg = wave / KS, kpart = wave % KS;
  const int row0 = blockIdx.x * ((4 / KS) * R) + rg * R;
  const int L = K * BITS / 128;  // 16-byte chunks per row
  const int nch = (L + 63) / 64;
  const int ng = K / G;

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

  for (int c = kpart; c < nch; c += KS) {
    const int j = c * 64 + lane;
    const bool live = j < L;
    const int k0 = j * C::CPL;

    // every load of this chunk is issued before any arithmetic: the weight
    // words, the group scales and biases of all R rows, and the x slices
    uint4 wv[R];
    float sv[R][C::NSEG], bv[R][C::NSEG];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = row0 + r;
      const bool ok = live && row < N;
      const int rowc = ok ? row : 0;
      wv[r] = ok ? w[(long)rowc * L + j] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int seg = 0; seg < C::NSEG; ++seg) {
        const long gi = (long)rowc * ng + (ok ? (k0 + seg * C::SEGK) / G : 0);
        sv[r][seg] = ok ? load_as_f32(scales, gi, sdt) : 0.f;
        bv[r][seg] = ok ? load_as_f32(biases, gi, bdt) : 0.f;
      }
    }
    typename C::XSlice xs[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (live && m < M)
        C::load(x + (long)m * K, k_perm, k0, xs[m]);
      else
        C::zero(xs[m]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int seg = 0; seg < C::NSEG; ++seg) {
        const float s = sv[r][seg];
        const float b = bv[r][seg] - C::OFF * s;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float d = C::dot(wv[r], xs[m], seg);
          acc[r][m] = fmaf(s, d, fmaf(b, xs[m].sum[seg], acc[r][m]));
        }
      }
    }
  }

  __shared__ float red[4][R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = wave_sum(acc[r][m]);
      if (lane == 0) red[wave][r][m] = v;
    }
  __syncthreads();
  if (kpart == 0 && lane < R * MT) {
    const int r = lane / MT, m = lane % MT;
    float v = 0.f;
    for (int q = 0; q < KS; ++q) v += red[rg * KS + q][r][m];
    const int row = row0 + r;
    if (row < N && m < M) y[(long)m * N + row] = f32_to_act_bits(v, F16);
  }
}

template <int BITS, bool F16, int MT>
hipError_t launch_r(const AffineArgs& a, const uint16_t* x, uint16_t* y, int M, int R, int KS, hipStream_t s) {
  const int rows_per_wg = (4 / KS) * R;
  const dim3 grid((unsigned)((a.N + rows_per_wg - 1) / rows_per_wg));
  const uint4* w = reinterpret_cast<const uint4*>(a.w);
  const int N = (int)a.N, K = (int)a.K;
  switch (R) {
    case 1:
      hipLaunchKernelGGL((gemv_affine_kernel<BITS, F16, MT, 1>), grid, dim3(256), 0, s, x, w, a.scales, a.biases,
                         a.k_perm, y, M, N, K, a.G, a.s_dt, a.b_dt, KS);
      break;
    case 2:
      hipLaunchKernelGGL((gemv_affine_kernel<BITS, F16, MT, 2>), grid, dim3(256), 0, s, x, w, a.scales, a.biases,
                         a.k_perm, y, M, N, K, a.G, a.s_dt, a.b_dt, KS);
      break;
    default:
      hipLaunchKernelGGL((gemv_affine_kernel<BITS, F16, MT, 4>), grid, dim3(256), 0, s, x, w, a.scales, a.biases,
                         a.k_perm, y, M, N, K, a.G, a.s_dt, a.b_dt, KS);
      break;
  }
  return hipGetLastError();
}

template <int BITS, bool F16>
hipError_t launch_bits(const AffineArgs& a, hipStream_t s) {
  const int64_t L = a.K * BITS / 128;
  const int64_t nch = (L + 63) / 64;
  const int KS = nch >= 4 ? 4 : (nch >= 2 ? 2 : 1);
  // rows per thread: enough workgroups to cover the chip twice when possible
  int R = 4;
  while (R > 1 && a.N / ((4 / KS) * R) < 512) R /= 2;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  uint16_t* y = static_cast<uint16_t*>(a.y);
  if (a.M == 1) return launch_r<BITS, F16, 1>(a, x, y, 1, R, KS, s);
  // x rows in chunks of 4; each chunk is one launch over the whole weight
  for (int64_t m0 = 0; m0 < a.M; m0 += 4) {
    const int mc = (int)((a.M - m0) < 4 ? (a.M - m0) : 4);
    hipError_t e = launch_r<BITS, F16, 4>(a, x + m0 * a.K, y + m0 * a.N, mc, R, KS, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemv_affine(const AffineArgs& a, hipStream_t s) {
  const bool f16 = a.act_dt == F16;
  switch (a.bits) {
    case 2: return f16 ? launch_bits<2, true>(a, s) : launch_bits<2, false>(a, s);
    case 4: return f16 ? launch_bits<4, true>(a, s) : launch_bits<4, false>(a, s);
    default: return f16 ? launch_bits<8, true>(a, s) : launch_bits<8, false>(a, s);
  }
}

}  // namespace qaff
