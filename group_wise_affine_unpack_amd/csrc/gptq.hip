// GPTQ layout (TinyGPT "Quantization Expansion", section 1 "GPTQReader",
// "Format" and the dequant recipe):
//   qweight [K/8, N] int32: 8 codes along K per word, code i in nibble i%8
//   qzeros  [K/G, N/8] int32: 8 zero points along N per word, stored as zero-1
//   scales  [K/G, N] f16;  g_idx [K] int32 (act-order) or NULL (i/G)
//   W[n,i] = scale[g,n] * (q - (z_stored + 1)),  g = g_idx[i]
//
// qmm_gptq (direct kernel): split-K over workgroups and waves, one lane per
// output column, an LDS table for the act-order group lookup; described at
// the kernel below.
//
// gptq_to_affine_repack (kernel part): gathers codes through the permutation
// (computed on the host) into the affine [N, K/8] layout and writes the
// transposed scales and the biases -scale*(z+1).
#include <algorithm>

#include "common.h"

namespace qaff {
namespace {

constexpr int COLS = 64;   // columns per workgroup: one per lane
constexpr int WAVES = 8;   // waves per workgroup, each on its own slice of K
constexpr int KW_MAX = 16; // word rows a wave loads at once

__device__ __forceinline__ uint32_t nib(uint32_t w, int j) { return (w >> (4 * j)) & 0xFu; }

// Direct GPTQ GEMV/GEMM for small M.  Workgroup (cg, sp): columns
// [64cg, 64cg+64) (lane = column; consecutive lanes read consecutive words of
// a qweight row, so every load is one coalesced 256-byte row piece) and K
// slice sp of S.  Its 8 waves split the slice again.  Each wave loads all its
// weight words first; meanwhile the workgroup builds an LDS table of
// (scale, -scale*(z+1)) in fp32 for every group and column, so the
// act-order lookup g_idx[k] -> table row is one LDS read per code and the
// weight is exact in fp32: W = scale*q + bias.  x and g_idx values are
// uniform across the wave and arrive through scalar loads.  The waves meet
// in LDS; the slice's sum goes to an fp32 partial buffer [S][M][N], and a
// second kernel adds the S partials into y.
template <int MT>  // rows of x per pass
__global__ __launch_bounds__(COLS * WAVES) void gptq_direct_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint32_t* __restrict__ qz,
    const uint16_t* __restrict__ sc, const int32_t* __restrict__ g_idx, float* __restrict__ part, int M, int N,
    int K, int G, int S) {
  extern __shared__ float2 tab[];  // [ng][COLS] (scale, bias)
  __shared__ float red[WAVES][MT][COLS];
  const int ng = K / G;
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int ncg = (N + COLS - 1) / COLS;
  const int cg = blockIdx.x % ncg, sp = blockIdx.x / ncg;
  const int n0 = cg * COLS, n = n0 + lane;
  const bool live = n < N;
  const int ncol = live ? n : N - 1;

  // this wave's word rows: slice sp of S, part `wave` of WAVES
  const int nw = K / 8;
  const int per_sp = (nw + S - 1) / S;
  const int sp0 = sp * per_sp, sp1 = min(nw, sp0 + per_sp);
  const int per_w = (sp1 - sp0 + WAVES - 1) / WAVES;
  const int kw0 = min(sp1, sp0 + wave * per_w), kw1 = min(sp1, kw0 + per_w);

  // the first batch of this wave's weight words, in flight during the table build
  uint32_t wv[KW_MAX];
#pragma unroll
  for (int j = 0; j < KW_MAX; ++j) wv[j] = j < kw1 - kw0 ? qw[(long)(kw0 + j) * N + ncol] : 0u;

  for (int i = t; i < ng * COLS; i += COLS * WAVES) {
    const int g = i / COLS, c = i % COLS, nn = n0 + c;
    float2 e = make_float2(0.f, 0.f);
    if (nn < N) {
      const float sv = f16_bits_to_f32(sc[(long)g * N + nn]);
      const float z = (float)nib(qz[(long)g * (N / 8) + nn / 8], nn % 8) + 1.f;
      e = make_float2(sv, -sv * z);  // exact: an 11-bit scale times a 5-bit integer
    }
    tab[i] = e;
  }
  __syncthreads();

  for (int m0 = 0; m0 < M; m0 += MT) {
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
    for (int kb = kw0; kb < kw1; kb += KW_MAX) {
      const int cnt = min(KW_MAX, kw1 - kb);
      if (kb != kw0 || m0 != 0) {
#pragma unroll
        for (int j = 0; j < KW_MAX; ++j) wv[j] = j < cnt ? qw[(long)(kb + j) * N + ncol] : 0u;
      }
#pragma unroll
      for (int j = 0; j < KW_MAX; ++j) {
        if (j < cnt) {  // uniform
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = (kb + j) * 8 + e;
          const int g = g_idx ? g_idx[k] : k / G;
          const float2 sb = tab[g * COLS + lane];
          const float wk = fmaf(sb.x, (float)nib(wv[j], e), sb.y);
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const int mm = m0 + m < M ? m0 + m : M - 1;
            acc[m] = fmaf(f16_bits_to_f32(x[(long)mm * K + k]), wk, acc[m]);
          }
        }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) red[wave][m][lane] = acc[m];
    __syncthreads();
    if (wave == 0 && live) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m0 + m < M) {
          float v = 0.f;
#pragma unroll
          for (int q = 0; q < WAVES; ++q) v += red[q][m][lane];
          part[((long)sp * M + m0 + m) * N + n] = v;
        }
      }
    }
    __syncthreads();
  }
}

// y[m, n] = f16(sum over the S slices)
__global__ __launch_bounds__(256) void gptq_finalize_kernel(const float* __restrict__ part, uint16_t* __restrict__ y,
                                                            long MN, int S) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[(long)s * MN + i];
  y[i] = f32_to_f16_bits(v);
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
  if (lds > 96 * 1024) return hipErrorNotSupported;  // group table must fit in LDS
  const int64_t ncg = (a.N + COLS - 1) / COLS;
  const int64_t nw = a.K / 8;
  // K slices: enough workgroups to fill the chip twice, each wave keeping
  // at least 4 word rows
  int S = (int)std::min<int64_t>((512 + ncg - 1) / ncg, std::max<int64_t>(1, nw / (4 * WAVES)));
  if (S < 1) S = 1;
  const int64_t MN = a.M * a.N;
  keep_pool_memory(s);
  float* part = nullptr;
  hipError_t e = hipMallocAsync((void**)&part, (size_t)S * MN * sizeof(float), s);
  if (e != hipSuccess) return e;
  if (a.M == 1)
    hipLaunchKernelGGL((gptq_direct_kernel<1>), dim3((unsigned)(ncg * S)), dim3(COLS * WAVES), lds, s,
                       (const uint16_t*)a.x, (const uint32_t*)a.qweight, (const uint32_t*)a.qzeros,
                       (const uint16_t*)a.scales, a.g_idx, part, (int)a.M, (int)a.N, (int)a.K, a.G, S);
  else
    hipLaunchKernelGGL((gptq_direct_kernel<8>), dim3((unsigned)(ncg * S)), dim3(COLS * WAVES), lds, s,
                       (const uint16_t*)a.x, (const uint32_t*)a.qweight, (const uint32_t*)a.qzeros,
                       (const uint16_t*)a.scales, a.g_idx, part, (int)a.M, (int)a.N, (int)a.K, a.G, S);
  e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL(gptq_finalize_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, part,
                       (uint16_t*)a.y, (long)MN, S);
    e = hipGetLastError();
  }
  const hipError_t f = hipFreeAsync(part, s);
  return e != hipSuccess ? e : f;
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
