// GPTQ layout (TinyGPT "Quantization Expansion", section 1 "GPTQReader",
// "Format" and the dequant recipe):
//   qweight [K/8, N] int32: 8 codes along K per word, code i in nibble i%8
//   qzeros  [K/G, N/8] int32: 8 zero points along N per word, stored as zero-1
//   scales  [K/G, N] f16;  g_idx [K] int32 (act-order) or NULL (i/G)
//   W[n,i] = scale[g,n] * (q - (z_stored + 1)),  g = g_idx[i]
//
// qmm_gptq (direct kernel): one thread per output column n; consecutive
// threads read consecutive words of a qweight row (coalesced).  A block
// covers 64 columns; its 4 waves split K.  The block first builds an LDS
// table of (scale, -scale*(z+1)) in fp32 for every group and column, so the
// act-order gather g_idx[i] -> table row costs one LDS read per code, and
// the weight is exact in fp32: W = scale*q + bias.  x values are uniform
// across the wave and arrive through scalar loads.
//
// gptq_to_affine_repack (kernel part): gathers codes through the permutation
// (computed on the host) into the affine [N, K/8] layout and writes the
// transposed scales and the biases -scale*(z+1).
#include "common.h"

namespace qaff {
namespace {

constexpr int COLS = 64;  // columns per block
constexpr int MT = 4;     // rows of x per pass

__device__ __forceinline__ uint32_t nib(uint32_t w, int j) { return (w >> (4 * j)) & 0xFu; }

__global__ __launch_bounds__(256) void gptq_direct_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
                                                          const uint32_t* __restrict__ qz,
                                                          const uint16_t* __restrict__ sc,
                                                          const int32_t* __restrict__ g_idx,
                                                          uint16_t* __restrict__ y, int M, int N, int K, int G) {
  extern __shared__ float2 tab[];  // [ng][COLS] (scale, bias)
  const int ng = K / G;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n0 = blockIdx.x * COLS;
  const int n = n0 + lane;
  const bool live = n < N;

  for (int i = t; i < ng * COLS; i += 256) {
    const int g = i / COLS, c = i % COLS, nn = n0 + c;
    float2 e = make_float2(0.f, 0.f);
    if (nn < N) {
      const float s = f16_bits_to_f32(sc[(long)g * N + nn]);
      const float z = (float)nib(qz[(long)g * (N / 8) + nn / 8], nn % 8) + 1.f;
      e = make_float2(s, -s * z);  // exact: 11-bit scale times a 5-bit integer
    }
    tab[i] = e;
  }
  __syncthreads();

  // this wave's K range, in whole words
  const int nw = K / 8;
  const int w_per_wave = (nw + 3) / 4;
  const int kw0 = wave * w_per_wave, kw1 = min(nw, kw0 + w_per_wave);
  const int ncol = live ? n : 0;

  for (int mc = 0; mc < M; mc += MT) {
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
    for (int kw = kw0; kw < kw1; ++kw) {
      const uint32_t word = qw[(long)kw * N + ncol];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k = kw * 8 + e;
        const int g = g_idx ? g_idx[k] : k / G;
        const float2 sb = tab[g * COLS + lane];
        const float wv = fmaf(sb.x, (float)nib(word, e), sb.y);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int mm = mc + m < M ? mc + m : M - 1;
          acc[m] = fmaf(f16_bits_to_f32(x[(long)mm * K + k]), wv, acc[m]);
        }
      }
    }
    __shared__ float red[4][MT][64];
#pragma unroll
    for (int m = 0; m < MT; ++m) red[wave][m][lane] = acc[m];
    __syncthreads();
    if (wave == 0 && live) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (mc + m < M) {
          const float v = red[0][m][lane] + red[1][m][lane] + red[2][m][lane] + red[3][m][lane];
          y[(long)(mc + m) * N + n] = f32_to_f16_bits(v);
        }
      }
    }
    __syncthreads();
  }
}

// one thread per output word (n, jw): 8 codes gathered through k_perm
__global__ __launch_bounds__(256) void gptq_repack_codes_kernel(const uint32_t* __restrict__ qw,
                                                                const int32_t* __restrict__ kp,
                                                                uint32_t* __restrict__ out, int N, int K) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long nw = K / 8;
  if (idx >= (long)N * nw) return;
  const int n = (int)(idx % N), jw = (int)(idx / N);
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = kp[jw * 8 + e];
    word |= nib(qw[(long)(i / 8) * N + n], i % 8) << (4 * e);
  }
  out[(long)n * nw + jw] = word;
}

// one thread per (g, n): transposed scale and bias -scale*(z+1)
__global__ __launch_bounds__(256) void gptq_repack_params_kernel(const uint32_t* __restrict__ qz,
                                                                 const uint16_t* __restrict__ sc,
                                                                 uint16_t* __restrict__ s_out, void* __restrict__ b_out,
                                                                 int bias_f32, int N, int ng) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)N * ng) return;
  const int n = (int)(idx % N), g = (int)(idx / N);
  const uint16_t sbits = sc[(long)g * N + n];
  const float s = f16_bits_to_f32(sbits);
  const float z = (float)nib(qz[(long)g * (N / 8) + n / 8], n % 8) + 1.f;
  const float b = -s * z;  // exact in fp32
  s_out[(long)n * ng + g] = sbits;
  if (bias_f32)
    ((float*)b_out)[(long)n * ng + g] = b;
  else
    ((uint16_t*)b_out)[(long)n * ng + g] = f32_to_f16_bits(b);
}

}  // namespace

hipError_t launch_gptq_direct(const GptqArgs& a, hipStream_t s) {
  const int ng = (int)(a.K / a.G);
  const size_t lds = (size_t)ng * COLS * sizeof(float2);
  if (lds > 150 * 1024) return hipErrorNotSupported;  // group table must fit in LDS
  const dim3 grid((unsigned)((a.N + COLS - 1) / COLS));
  hipLaunchKernelGGL(gptq_direct_kernel, grid, dim3(256), lds, s, (const uint16_t*)a.x, (const uint32_t*)a.qweight,
                     (const uint32_t*)a.qzeros, (const uint16_t*)a.scales, a.g_idx, (uint16_t*)a.y, (int)a.M,
                     (int)a.N, (int)a.K, a.G);
  return hipGetLastError();
}

hipError_t launch_gptq_repack(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                              const int32_t* k_perm_dev, uint32_t* w_out, void* s_out, void* b_out, int bias_dt,
                              int64_t K, int64_t N, int G, hipStream_t s) {
  const long words = N * (K / 8);
  hipLaunchKernelGGL(gptq_repack_codes_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                     (const uint32_t*)qweight, k_perm_dev, w_out, (int)N, (int)K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long np = N * (K / G);
  hipLaunchKernelGGL(gptq_repack_params_kernel, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, s,
                     (const uint32_t*)qzeros, (const uint16_t*)scales, (uint16_t*)s_out, b_out, bias_dt == F32 ? 1 : 0,
                     (int)N, (int)(K / G));
  return hipGetLastError();
}

}  // namespace qaff
