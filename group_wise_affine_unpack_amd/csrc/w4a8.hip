// W4A8: dynamic per-token int8 activations x symmetric per-channel int4
// weights, int32 accumulation (executorch PR #24467, mlx::int8_int4_gemm,
// "What this adds"; the symmetric per-row scale rule max|.|/qMax is the one of
// TinyGPT "Quantization Expansion", section 4 "Fake-quant + STE").
//
//   s_x[m]   = max_k |x[m,k]| / 127                      IEEE fp32 division
//   x_q[m,k] = clamp(rint(x[m,k] / s_x[m]), -127, 127)     round half to even
//   acc[m,n] = sum_k x_q[m,k] * v[n,k]                    exact int32
//   y[m,n]   = f16((float(acc) * s_x[m]) * s_w[n])
//
// Kernels:
//   quant : one block per row; bit-exact codes and scale.
//   gemm  : v_mfma_i32_32x32x32_i8, tile BM x BN (4 waves along N, each
//           BM x NB*32), x_q tile double-buffered in LDS, int4 words decoded in
//           registers; the tile shrinks until the grid covers the chip.  A nibble
//           is placed in the HIGH half of its byte, which makes the byte the
//           int8 value 16*v with no sign extension step; the accumulator is
//           shifted right by 4 at the end (exact: every product is a multiple
//           of 16, and |acc| * 16 < 2^31 for K <= 2^17).
#include "common.h"

namespace qaff {
namespace {

__global__ __launch_bounds__(256) void w4a8_quant_kernel(const uint16_t* __restrict__ x, int K,
                                                         int8_t* __restrict__ xq, float* __restrict__ sx) {
  const int m = blockIdx.x, t = threadIdx.x;
  const uint16_t* row = x + (long)m * K;
  __shared__ float red[4];
  float amax = 0.f;
  for (int k = t; k < K; k += 256) amax = fmaxf(amax, fabsf(f16_bits_to_f32(row[k])));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax / 127.0f;  // correctly rounded division (HIP default)
  if (t == 0) sx[m] = s;
  int8_t* qrow = xq + (long)m * K;
  for (int k = t; k < K; k += 256) {
    float q = 0.f;
    if (s != 0.f) {
      q = rintf(f16_bits_to_f32(row[k]) / s);
      q = fminf(fmaxf(q, -127.f), 127.f);
    }
    qrow[k] = (int8_t)(int)q;
  }
}

constexpr int BK = 64;       // int8 codes per K tile
constexpr int LDS_ROW = 80;  // 64 bytes + 16 bytes padding (conflict-free 16-byte reads)

struct Params {
  const int8_t* xq;
  const float* sx;
  const uint32_t* w;
  const uint16_t* sw;
  uint16_t* y;
  int32_t* acc_out;
  int M, N, K;
  int Tm, Tn, per_xcd;
};

// 8 nibbles of one word -> 8 int8 (16*v) in natural k order (2 dwords)
__device__ __forceinline__ void decode_word(uint32_t w, uint32_t& d0, uint32_t& d1) {
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u;  // nibbles 0,2,4,6 in the byte high halves
  const uint32_t hi = w & 0xF0F0F0F0u;         // nibbles 1,3,5,7
  d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // (n0, n1, n2, n3)
  d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // (n4, n5, n6, n7)
}

template <int MB, int NB>
__global__ __launch_bounds__(256) void w4a8_gemm_kernel(Params p) {
  constexpr int BM = MB * 32;
  constexpr int BN = NB * 128;
  constexpr int A_CHUNKS = BM * 4 / 256;  // 16-byte chunks of the x_q tile per thread (>= 1)
  const int b = blockIdx.x;
  const int v = (b & 7) * p.per_xcd + (b >> 3);
  if (v >= p.Tm * p.Tn) return;
  const int tm = v / p.Tn, tn = v % p.Tn;
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l32 = lane & 31, half = lane >> 5;

  __shared__ __attribute__((aligned(16))) unsigned char lds[2][BM * LDS_ROW];

  i32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  int nrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n0 + wave * NB * 32 + nb * 32 + l32;
    nrow[nb] = n < p.N ? n : p.N - 1;
  }
  const long wrow = p.K / 8;
  const int nkt = p.K / BK;
  u32x4_t wcur[NB], wnxt[NB];
  u32x4_t areg[A_CHUNKS];

  // x_q rows past M are read clamped to M-1; their results are not stored
  auto a_src = [&](int kt, int c) {
    const int ch = t + 256 * c, row = ch >> 2, col = ch & 3;
    const int m = m0 + row < p.M ? m0 + row : p.M - 1;
    return reinterpret_cast<const u32x4_t*>(p.xq + (long)m * p.K + kt * BK) + col;
  };
#pragma unroll
  for (int c = 0; c < A_CHUNKS; ++c) areg[c] = *a_src(0, c);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wcur[nb] = *reinterpret_cast<const u32x4_t*>(p.w + nrow[nb] * wrow + half * 4);
#pragma unroll
  for (int c = 0; c < A_CHUNKS; ++c) {
    const int ch = t + 256 * c;
    *reinterpret_cast<u32x4_t*>(&lds[0][(ch >> 2) * LDS_ROW + (ch & 3) * 16]) = areg[c];
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) {
#pragma unroll
      for (int c = 0; c < A_CHUNKS; ++c) areg[c] = *a_src(kt + 1, c);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        wnxt[nb] = *reinterpret_cast<const u32x4_t*>(p.w + nrow[nb] * wrow + (kt + 1) * 8 + half * 4);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      i32x4_t af[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[mb] = *reinterpret_cast<const i32x4_t*>(&lds[buf][(mb * 32 + l32) * LDS_ROW + 32 * half + 16 * s]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t w0 = s == 0 ? wcur[nb].x : wcur[nb].z;
        const uint32_t w1 = s == 0 ? wcur[nb].y : wcur[nb].w;
        uint32_t d0, d1, d2, d3;
        decode_word(w0, d0, d1);
        decode_word(w1, d2, d3);
        const i32x4_t bf = {(int)d0, (int)d1, (int)d2, (int)d3};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mb], bf, acc[mb][nb], 0, 0, 0);
      }
    }
    if (more) {
#pragma unroll
      for (int c = 0; c < A_CHUNKS; ++c) {
        const int ch = t + 256 * c;
        *reinterpret_cast<u32x4_t*>(&lds[buf ^ 1][(ch >> 2) * LDS_ROW + (ch & 3) * 16]) = areg[c];
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wcur[nb] = wnxt[nb];
    }
    __syncthreads();
  }

  // epilogue; 32x32 accumulator layout: lane -> column l32, register r -> row 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n0 + wave * NB * 32 + nb * 32 + l32;
    if (n >= p.N) continue;
    const float swn = f16_bits_to_f32(p.sw[n]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (m < p.M) {
          const int a = acc[mb][nb][r] >> 4;
          if (p.acc_out) p.acc_out[(long)m * p.N + n] = a;
          p.y[(long)m * p.N + n] = f32_to_f16_bits(((float)a * p.sx[m]) * swn);
        }
      }
  }
}

}  // namespace

hipError_t launch_w4a8(const W4A8Args& a, hipStream_t s) {
  if (a.K % BK != 0) return hipErrorNotSupported;
  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  hipLaunchKernelGGL(w4a8_quant_kernel, dim3(M), dim3(256), 0, s, (const uint16_t*)a.x, K, a.x_q, a.s_x);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // largest tile whose grid still gives every CU at least two workgroups
  struct Tile { int mb, nb; };
  const Tile tiles[] = {{8, 2}, {4, 2}, {4, 1}, {2, 1}};
  Tile t = tiles[3];
  for (const Tile& c : tiles) {
    const long tm = (M + c.mb * 32 - 1) / (c.mb * 32), tn = (N + c.nb * 128 - 1) / (c.nb * 128);
    if (tm * tn >= 512) { t = c; break; }
  }
  if (M <= 64) t = Tile{2, 1};
  Params p;
  p.xq = a.x_q;
  p.sx = a.s_x;
  p.w = a.w;
  p.sw = (const uint16_t*)a.s_w;
  p.y = (uint16_t*)a.y;
  p.acc_out = a.acc;
  p.M = M;
  p.N = N;
  p.K = K;
  p.Tm = (M + t.mb * 32 - 1) / (t.mb * 32);
  p.Tn = (N + t.nb * 128 - 1) / (t.nb * 128);
  p.per_xcd = (p.Tm * p.Tn + 7) / 8;
  const dim3 grid(8 * p.per_xcd);
  if (t.mb == 8)
    hipLaunchKernelGGL((w4a8_gemm_kernel<8, 2>), grid, dim3(256), 0, s, p);
  else if (t.mb == 4 && t.nb == 2)
    hipLaunchKernelGGL((w4a8_gemm_kernel<4, 2>), grid, dim3(256), 0, s, p);
  else if (t.mb == 4)
    hipLaunchKernelGGL((w4a8_gemm_kernel<4, 1>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((w4a8_gemm_kernel<2, 1>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace qaff
