// quantize_pack_affine: dense weights -> packed codes + per-group scale/bias.
// The Transformers "Metal" quantization page quantizes nn.Linear weights on
// load into this layout but gives no formula; the rule here is plain min/max
// affine quantization, in IEEE fp32 exactly as written (no contraction):
//   scale = (max - min) / (2^bits - 1)  -> stored in sb_dtype (nearest even)
//   bias  = min                         -> stored in sb_dtype
//   q     = clamp(rint((w - bias_stored) / scale_stored), 0, 2^bits - 1)
//           (0 when scale_stored == 0)
// packed with the lowest column in the low bits of each uint32 word.
// One thread per (row, group): a setup call, not on the hot path.
#include "common.h"

namespace qaff {
namespace {

__device__ __forceinline__ float round_to(float v, int dt) {
  if (dt == BF16) return bf16_bits_to_f32(f32_to_bf16_bits(v));
  if (dt == F16) return f16_bits_to_f32(f32_to_f16_bits(v));
  return v;
}

__device__ __forceinline__ void store_as(void* base, long i, int dt, float v) {
  if (dt == BF16)
    ((uint16_t*)base)[i] = f32_to_bf16_bits(v);
  else if (dt == F16)
    ((uint16_t*)base)[i] = f32_to_f16_bits(v);
  else
    ((float*)base)[i] = v;
}

template <int BITS>
__global__ __launch_bounds__(256) void quantize_pack_kernel(const void* __restrict__ w, int w_dt,
                                                            uint32_t* __restrict__ packed, void* __restrict__ scales,
                                                            void* __restrict__ biases, int sb_dt, int N, int K,
                                                            int G) {
  const int ng = K / G;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)N * ng) return;
  const int n = (int)(idx / ng), g = (int)(idx % ng);
  const long base = (long)n * K + (long)g * G;
  float lo = __builtin_inff(), hi = -__builtin_inff();
  for (int k = 0; k < G; ++k) {
    const float v = load_as_f32(w, base + k, w_dt);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  const float qmax = (float)((1 << BITS) - 1);
  const float range = __fsub_rn(hi, lo);
  const float s = __fdiv_rn(range, qmax);
  const float s_r = round_to(s, sb_dt);
  const float b_r = round_to(lo, sb_dt);
  store_as(scales, idx, sb_dt, s);
  store_as(biases, idx, sb_dt, lo);
  constexpr int PER = 32 / BITS;
  const long wbase = ((long)n * K + (long)g * G) / PER;
  for (int wi = 0; wi < G / PER; ++wi) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float v = load_as_f32(w, base + wi * PER + e, w_dt);
      float q = 0.f;
      if (s_r != 0.f) {
        q = rintf(__fdiv_rn(__fsub_rn(v, b_r), s_r));
        q = fminf(fmaxf(q, 0.f), qmax);
      }
      word |= (uint32_t)q << (BITS * e);
    }
    packed[wbase + wi] = word;
  }
}

}  // namespace

hipError_t launch_quantize_pack(const void* w, int w_dt, uint32_t* packed, void* scales, void* biases, int sb_dt,
                                int64_t N, int64_t K, int G, int bits, hipStream_t s) {
  const long total = N * (K / G);
  const dim3 grid((unsigned)((total + 255) / 256));
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(quantize_pack_kernel<2>, grid, dim3(256), 0, s, w, w_dt, packed, scales, biases, sb_dt,
                         (int)N, (int)K, G);
      break;
    case 4:
      hipLaunchKernelGGL(quantize_pack_kernel<4>, grid, dim3(256), 0, s, w, w_dt, packed, scales, biases, sb_dt,
                         (int)N, (int)K, G);
      break;
    default:
      hipLaunchKernelGGL(quantize_pack_kernel<8>, grid, dim3(256), 0, s, w, w_dt, packed, scales, biases, sb_dt,
                         (int)N, (int)K, G);
      break;
  }
  return hipGetLastError();
}

}  // namespace qaff
