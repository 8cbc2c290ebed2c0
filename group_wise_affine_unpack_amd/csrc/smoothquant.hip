// SmoothQuant ahead of W4A8 (TinyGPT "Quantization Expansion", section 3
// "SmoothQuant": per input channel, y = (x / s) . (s W), with Xiao et al.'s
// s = max|x|^alpha / max|W|^(1 - alpha)), and the per-channel int4 weight
// quantization of W4A8 (executorch PR #24467, "What this adds").
//
//   smooth_factors_kernel   s[k] from the calibration maxima of x and the
//                           column maxima of W (one thread per column, the
//                           column walked with n fastest across threads)
//   w4a8_weights_kernel     per row: W'[n,k] = W[n,k] * s[k] (fp32), s_w =
//                           f16(max|W'| / 7), codes clamp(rint(W'/s_w),
//                           -8, 7) packed as two's complement nibbles
//   smooth_quant_kernel     per token: xs = fp32(x) / s[k], s_x = max|xs|/127,
//                           codes clamp(rint(xs / s_x), -127, 127)
// Every division is the IEEE one (__fdiv_rn), so codes and scales are the
// same bits as the plain C definition; rint rounds half to even.
#include "common.h"

namespace qaff {
namespace {

__global__ __launch_bounds__(256) void smooth_factors_kernel(const float* __restrict__ amax, const void* __restrict__ w,
                                                             int w_dt, int N, int K, double alpha,
                                                             float* __restrict__ s) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  float wmax = 0.f;
  for (int n = 0; n < N; ++n) wmax = fmaxf(wmax, fabsf(load_as_f32(w, (long)n * K + k, w_dt)));
  const double a = (double)amax[k], m = (double)wmax;
  // a channel with a zero maximum (or a non-finite one) is left as it is
  s[k] = (a > 0.0 && m > 0.0) ? (float)(pow(a, alpha) / pow(m, 1.0 - alpha)) : 1.f;
}

// one block (256 threads) per row n
__global__ __launch_bounds__(256) void w4a8_weights_kernel(const void* __restrict__ w, int w_dt,
                                                           const float* __restrict__ smooth, int K,
                                                           uint32_t* __restrict__ w_q4, uint16_t* __restrict__ s_w) {
  const int n = blockIdx.x, t = threadIdx.x;
  __shared__ float red[4];
  auto val = [&](int k) {
    const float v = load_as_f32(w, (long)n * K + k, w_dt);
    return smooth ? __fmul_rn(v, smooth[k]) : v;
  };
  float amax = 0.f;
  for (int k = t; k < K; k += 256) amax = fmaxf(amax, fabsf(val(k)));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const uint16_t h = f32_to_f16_bits(__fdiv_rn(amax, 7.f));
  if (t == 0) s_w[n] = h;
  const float sr = f16_bits_to_f32(h);
  for (int c = t; c < K / 8; c += 256) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float q = 0.f;
      if (sr != 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(val(8 * c + j), sr)), -8.f), 7.f);
      word |= ((uint32_t)(int)q & 0xFu) << (4 * j);
    }
    w_q4[(long)n * (K / 8) + c] = word;
  }
}

// one block (256 threads) per token m
__global__ __launch_bounds__(256) void smooth_quant_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ smooth, int K,
                                                           int8_t* __restrict__ x_q, float* __restrict__ s_x) {
  const int m = blockIdx.x, t = threadIdx.x;
  __shared__ float red[4];
  const uint16_t* xr = x + (long)m * K;
  float amax = 0.f;
  for (int k = t; k < K; k += 256) amax = fmaxf(amax, fabsf(__fdiv_rn(f16_bits_to_f32(xr[k]), smooth[k])));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = __fdiv_rn(amax, 127.f);
  if (t == 0) s_x[m] = sc;
  for (int k = t; k < K; k += 256) {
    float q = 0.f;
    if (sc != 0.f)
      q = fminf(fmaxf(rintf(__fdiv_rn(__fdiv_rn(f16_bits_to_f32(xr[k]), smooth[k]), sc)), -127.f), 127.f);
    x_q[(long)m * K + k] = (int8_t)q;
  }
}

}  // namespace

hipError_t launch_smooth_factors(const float* amax, const void* w, int w_dt, int64_t N, int64_t K, double alpha,
                                 float* s, hipStream_t st) {
  hipLaunchKernelGGL(smooth_factors_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, amax, w, w_dt,
                     (int)N, (int)K, alpha, s);
  return hipGetLastError();
}

hipError_t launch_w4a8_weights(const void* w, int w_dt, const float* smooth, int64_t N, int64_t K, uint32_t* w_q4,
                               uint16_t* s_w, hipStream_t st) {
  hipLaunchKernelGGL(w4a8_weights_kernel, dim3((unsigned)N), dim3(256), 0, st, w, w_dt, smooth, (int)K, w_q4, s_w);
  return hipGetLastError();
}

hipError_t launch_smooth_quant(const void* x, const float* smooth, int64_t M, int64_t K, int8_t* x_q, float* s_x,
                               hipStream_t st) {
  hipLaunchKernelGGL(smooth_quant_kernel, dim3((unsigned)M), dim3(256), 0, st, (const uint16_t*)x, smooth, (int)K, x_q,
                     s_x);
  return hipGetLastError();
}

}  // namespace qaff
