// Decode GEMV for group-wise affine weights, M <= 16 (memory-bound path).
//
//   y[m, n] = sum_k x[m, k] * (q(n,k) * scale[n, k/G] + bias[n, k/G])
//
// The weight layout (uint32 words, lowest column in the low bits, per-group
// scale and bias) is the one of the mlx_int8.rs API page ("Layout") and of
// the Transformers "Metal" quantization page (bits 2/4/8).
//
// Design for CDNA4:
//  * work unit: one wave owns R = 4 rows and one K part; a 256-thread
//    workgroup holds 4/KS row groups x KS K parts (KS = 1, 2, 4 by row length);
//  * every global read is a buffer load: one 16-byte (dwordx4) load per lane
//    per row and 1 KiB chunk of K, fully coalesced; a lane past the end of
//    the row, or a row past N, reads through an offset outside the buffer's
//    range and gets zeros, so no load sits behind a branch;
//  * the lane's slice of x is rearranged once per chunk into the pair order
//    of the decode and reused for the R rows; codes become exact half values
//    with the exponent-bias trick (code | 0x4300 is 128+code in bf16,
//    code | 0x6400 is 1024+code in f16) and feed v_dot2_f32_{bf16,f16};
//  * per group segment a lane folds its scale and bias into its partial sum,
//    s*sum(c*x) + (b - off*s)*sum(x), so every weight stays exact;
//  * row offsets go in the uniform soffset field, clamped to a row that
//    exists, so per-row address arithmetic is scalar;
//  * the four row sums of a wave are reduced together: two permlane32 swaps,
//    one permlane16 swap, four DPP row rotations (10 VALU ops for 4 rows);
//    with KS > 1 the K parts meet in LDS;
//  * one launch serves up to MAXP independent problems that share M, G,
//    bits and dtypes (grouped launch): workgroups are numbered across the
//    problems and each finds its own by a binary search over the descriptor
//    table, which travels in the kernel arguments.  Linears that share an
//    input (q/k/v, gate/up), or a whole set of them, then cost one launch.
#include <algorithm>
#include <new>
#include <type_traits>

#include <vector>

#include "common.h"

namespace qaff {
namespace {

constexpr uint32_t OOB = 0x80000000u;  // buffer offset past every range: the load returns zeros
constexpr int MAXP = 56;               // problems per launch (a 3.6 KB descriptor table in the kernel arguments)

template <typename T>
__device__ __forceinline__ T bc(uint32_t v) { return __builtin_bit_cast(T, v); }

template <bool F16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (F16)
    return __builtin_amdgcn_fdot2(bc<f16x2_t>(a), bc<f16x2_t>(b), c, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(bc<bf16x2_t>(a), bc<bf16x2_t>(b), c, false);
}

// (low half of a, low half of b) or (high half of a, high half of b)
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Buffer loads.  voff carries everything the range check must see (the lane's
// position, or OOB); soff is a uniform byte offset of a row that is known to
// exist, so the access stays inside the buffer whether or not the hardware
// adds soff into its range check.
// AUX is the cache-policy field; 2 sets `nt` (streaming), used for the
// weight words, which are read exactly once.
template <int AUX = 0>
__device__ __forceinline__ u32x4_t ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}
constexpr int NT = 2;
__device__ __forceinline__ uint32_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// One codec per (bits, activation dtype).  A lane's chunk is 16 bytes of
// codes (CPL codes); its x arrives as XR 16-byte raw loads and is held as XP
// words; PPS decoded pairs per group segment meet those words in order.
template <int BITS, bool F16>
struct Codec;

// 4-bit: a word holds codes 8w..8w+7; ((w >> 4i) & 0x000F000F) is the pair
// (code i, code i+4).  x is held as the matching pairs (x[i], x[i+4]).
template <bool F16>
struct Codec<4, F16> {
  static constexpr int CPL = 32, NSEG = 1, SEGK = 32, XR = 4, XP = 16, PPS = 16;
  static constexpr float OFF = F16 ? 1024.f : 128.f;
  static constexpr uint32_t MAGIC = F16 ? 0x64006400u : 0x43004300u;
  static constexpr uint32_t ONES = F16 ? 0x3C003C00u : 0x3F803F80u;
  static __device__ __forceinline__ void build(const u32x4_t (&raw)[XR], uint32_t (&xp)[XP], float (&sum)[NSEG]) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      xp[4 * w + 0] = pair_lo(raw[w][0], raw[w][2]);
      xp[4 * w + 1] = pair_hi(raw[w][0], raw[w][2]);
      xp[4 * w + 2] = pair_lo(raw[w][1], raw[w][3]);
      xp[4 * w + 3] = pair_hi(raw[w][1], raw[w][3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) t = dot2<F16>(xp[4 * w + i], ONES, t);
    }
    sum[0] = t;
  }
  static __device__ __forceinline__ uint32_t pair(const u32x4_t& c, int p, uint32_t magic) {
    const int w = p >> 2, i = p & 3;
    return ((c[w] >> (4 * i)) & 0x000F000Fu) | magic;  // v_and_or_b32
  }
  static __device__ __forceinline__ float xdot(uint32_t pr, const uint32_t (&xp)[XP], int p, float acc) {
    return dot2<F16>(pr, xp[p], acc);
  }
};

// 2-bit: a word holds codes 16w..16w+15; ((w >> 2i) & 0x00030003) is the pair
// (code i, code i+8).  A chunk is 64 codes = two 32-code segments, each
// inside one group (G >= 32).
template <bool F16>
struct Codec<2, F16> {
  static constexpr int CPL = 64, NSEG = 2, SEGK = 32, XR = 8, XP = 32, PPS = 16;
  static constexpr float OFF = F16 ? 1024.f : 128.f;
  static constexpr uint32_t MAGIC = F16 ? 0x64006400u : 0x43004300u;
  static constexpr uint32_t ONES = F16 ? 0x3C003C00u : 0x3F803F80u;
  static __device__ __forceinline__ void build(const u32x4_t (&raw)[XR], uint32_t (&xp)[XP], float (&sum)[NSEG]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float t = 0.f;
#pragma unroll
      for (int w = 2 * h; w < 2 * h + 2; ++w)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t a = raw[2 * w][i >> 1], b = raw[2 * w + 1][i >> 1];
          xp[8 * w + i] = (i & 1) ? pair_hi(a, b) : pair_lo(a, b);
          t = dot2<F16>(xp[8 * w + i], ONES, t);
        }
      sum[h] = t;
    }
  }
  static __device__ __forceinline__ uint32_t pair(const u32x4_t& c, int p, uint32_t magic) {
    const int w = p >> 3, i = p & 7;
    return ((c[w] >> (2 * i)) & 0x00030003u) | magic;
  }
  static __device__ __forceinline__ float xdot(uint32_t pr, const uint32_t (&xp)[XP], int p, float acc) {
    return dot2<F16>(pr, xp[p], acc);
  }
};

// 8-bit codes, bf16 activations: 128+code does not fit a bf16 significand,
// so bytes go to fp32 (v_cvt_f32_ubyte*) and meet fp32 x in an FMA.  A
// "pair" here is a single code; xp holds x as fp32 bits.
template <>
struct Codec<8, false> {
  static constexpr int CPL = 16, NSEG = 1, SEGK = 16, XR = 2, XP = 16, PPS = 16;
  static constexpr float OFF = 0.f;
  static __device__ __forceinline__ void build(const u32x4_t (&raw)[XR], uint32_t (&xp)[XP], float (&sum)[NSEG]) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t d = raw[i >> 2][i & 3];
      xp[2 * i] = d << 16;
      xp[2 * i + 1] = d & 0xffff0000u;
      t += bc<float>(xp[2 * i]) + bc<float>(xp[2 * i + 1]);
    }
    sum[0] = t;
  }
  static constexpr uint32_t MAGIC = 0;
  static __device__ __forceinline__ uint32_t pair(const u32x4_t& c, int p, uint32_t) {
    return (c[p >> 2] >> (8 * (p & 3))) & 0xffu;
  }
  static __device__ __forceinline__ float xdot(uint32_t code, const uint32_t (&xp)[XP], int p, float acc) {
    return fmaf((float)code, bc<float>(xp[p]), acc);
  }
};

// 8-bit codes, f16 activations: v_perm_b32 builds (0x6400|b0, 0x6400|b2)
// and (0x6400|b1, 0x6400|b3) = 1024+code, exact in f16.
template <>
struct Codec<8, true> {
  static constexpr int CPL = 16, NSEG = 1, SEGK = 16, XR = 2, XP = 8, PPS = 8;
  static constexpr float OFF = 1024.f;
  static constexpr uint32_t ONES = 0x3C003C00u;
  static __device__ __forceinline__ void build(const u32x4_t (&raw)[XR], uint32_t (&xp)[XP], float (&sum)[NSEG]) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = raw[w >> 1][2 * (w & 1)], b = raw[w >> 1][2 * (w & 1) + 1];
      xp[2 * w] = pair_lo(a, b);      // (x[4w], x[4w+2])
      xp[2 * w + 1] = pair_hi(a, b);  // (x[4w+1], x[4w+3])
      t = dot2<true>(xp[2 * w], ONES, t);
      t = dot2<true>(xp[2 * w + 1], ONES, t);
    }
    sum[0] = t;
  }
  static constexpr uint32_t MAGIC = 0x64646464u;
  static __device__ __forceinline__ uint32_t pair(const u32x4_t& c, int p, uint32_t magic) {
    return __builtin_amdgcn_perm(magic, c[p >> 1], (p & 1) ? 0x04030401u : 0x04020400u);
  }
  static __device__ __forceinline__ float xdot(uint32_t pr, const uint32_t (&xp)[XP], int p, float acc) {
    return dot2<true>(pr, xp[p], acc);
  }
};

struct GemvDesc {
  const void* x;      // [M, K] activations
  const void* w;      // [N, K*BITS/32] uint32
  const void* s;      // [N, K/G]
  const void* b;      // [N, K/G]
  void* y;            // [M, N]
  int N, K, blk0, ks;  // ks: log2 of the waves that split a row's K
};

struct GemvBatch {
  GemvDesc d[MAXP];
  int count, M, gsh, sdt, bdt;
  // SiLU-gated input (one problem): x of the descriptor is the gate, `up`
  // the up projection, both [M, K]; `resid` [M, N] or NULL is added to y;
  // act_f16 is the dtype of gate, up, resid and y (the codes always take
  // the f16 path there)
  const void* up;
  const void* resid;
  int act_f16;
};
static_assert(sizeof(GemvBatch) <= 4096, "kernel arguments are limited to 4 KiB");

// A scale or bias element: byte offset voff (lane part) + soff (row part).
// SBM 0: bf16, 1: f16, 2: any of bf16 / f16 / f32, picked at run time with
// selects rather than branches (both widths are loaded; one is used).
template <int SBM>
__device__ __forceinline__ float load_param(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, int dt) {
  if constexpr (SBM == 0) {
    return bf16_bits_to_f32(ld16(r, voff, soff));
  } else if constexpr (SBM == 1) {
    return f16_bits_to_f32(ld16(r, voff, soff));
  } else {
    const uint32_t h = ld16(r, voff, soff);
    const uint32_t f = ld32(r, voff, soff);
    const float hv = dt == F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
    return dt == F32 ? __uint_as_float(f) : hv;
  }
}

// Sum over the 64 lanes of each of four values at once: two permlane32 swaps,
// one permlane16 swap and four DPP row rotations.  Row q (lanes 16q..16q+15)
// of the result holds the total of v[q].
__device__ __forceinline__ float wave_sum4(const float (&v)[4]) {
  auto sw32 = [](float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };
  const float s02 = sw32(v[0], v[2]);  // lanes 0-31: halves of v0, lanes 32-63: halves of v2
  const float s13 = sw32(v[1], v[3]);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  float t = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // row q: quarters of v[q]
  t += dpp_mov<0x128>(t);  // row_ror:8
  t += dpp_mov<0x124>(t);  // row_ror:4
  t += dpp_mov<0x122>(t);  // row_ror:2
  t += dpp_mov<0x121>(t);  // row_ror:1
  return t;
}

// silu(t) = t / (1 + e^-t) in fp32, the quotient as t times the hardware
// reciprocal (about 1 ulp; e^-t overflows to inf for t below about -88,
// and t * rcp(inf) = t * 0 is the correct limit -0)
__device__ __forceinline__ float silu_f32(float t) { return t * __builtin_amdgcn_rcpf(1.f + __expf(-t)); }

// Eight 16-bit gate and up values -> eight f16 values of silu(gate) * up
__device__ __forceinline__ u32x4_t silu_gate_f16(const u32x4_t& g, const u32x4_t& u, bool act_f16) {
  u32x4_t h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float r[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t gb = (g[i] >> (16 * j)) & 0xFFFFu, ub = (u[i] >> (16 * j)) & 0xFFFFu;
      const float gv = act_f16 ? f16_bits_to_f32(gb) : bf16_bits_to_f32(gb);
      const float uv = act_f16 ? f16_bits_to_f32(ub) : bf16_bits_to_f32(ub);
      r[j] = silu_f32(gv) * uv;
    }
    h[i] = (uint32_t)f32_to_f16_bits(r[0]) | ((uint32_t)f32_to_f16_bits(r[1]) << 16);
  }
  return h;
}

// R rows per wave (a multiple of 4), MT x rows per pass (1, 2 or 4).
// XM = 0: x as given.  XM = 1: x = silu(gate) * up formed in registers from
// the gate (the descriptor's x) and B.up, rounded to f16 (F16 is then true),
// with B.resid added to each output before its one rounding.
template <int BITS, bool F16, int MT, int SBM, int R, int XM = 0>
__global__ __launch_bounds__(256) void gemv_affine_kernel(GemvBatch B) {
  static_assert(R % 4 == 0, "rows are reduced in fours");
  static_assert(XM == 0 || F16, "the gated input takes the f16 code path");
  using C = Codec<BITS, F16>;

  // problem of this workgroup (uniform)
  const int bid = blockIdx.x;
  int lo = 0, hi = B.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (B.d[mid].blk0 <= bid) lo = mid; else hi = mid - 1;
  }
  const GemvDesc& D = B.d[lo];
  const int ksh = D.ks, KS = 1 << ksh, N = D.N, K = D.K, M = B.M;
  // the wave index is uniform: keep it (and every buffer range) in SGPRs
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave >> ksh, kpart = wave & (KS - 1);
  const int row0 = (bid - D.blk0) * ((4 >> ksh) * R) + rg * R;
  const int L = K * BITS / 128;  // 16-byte chunks per row
  const int nch = (L + 63) >> 6;
  const int ng = K >> B.gsh;
  const int nrows = __builtin_amdgcn_readfirstlane(min(max(N - row0, 0), R));
  const int ssh = (SBM == 2 && B.sdt == F32) ? 2 : 1, bsh = (SBM == 2 && B.bdt == F32) ? 2 : 1;
  const int ssz = 1 << ssh, bsz = 1 << bsh;
  const int rlast = max(nrows - 1, 0);  // loads of rows past N read this row; their sums are dropped

  // each range covers exactly this wave's rows
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(static_cast<const uint32_t*>(D.w) + (long)row0 * L * 4, (uint32_t)(nrows * L * 16));
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(static_cast<const char*>(D.s) + (long)row0 * ng * ssz, (uint32_t)(nrows * ng * ssz));
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(static_cast<const char*>(D.b) + (long)row0 * ng * bsz, (uint32_t)(nrows * ng * bsz));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(D.x, (uint32_t)(M * K * 2));
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(XM ? B.up : D.x, (uint32_t)(M * K * 2));
  // output dtype, and the residual added to each output
  const bool out_f16 = XM ? B.act_f16 != 0 : F16;
  const uint16_t* resid = XM ? static_cast<const uint16_t*>(B.resid) : nullptr;
  auto finish = [&](float v, int m, int n) -> uint16_t {
    if (XM && resid) {
      const uint32_t rb = resid[(long)m * N + n];
      v += out_f16 ? f16_bits_to_f32(rb) : bf16_bits_to_f32(rb);
    }
    return f32_to_act_bits(v, out_f16);
  };

  uint16_t* y = static_cast<uint16_t*>(D.y);
  __shared__ float red[4][R * MT];

  // x rows in passes of MT; W of the wave's rows is re-read from L2 per pass
  for (int m0 = 0; m0 < M; m0 += MT) {
  // The exponent-bias constant lives in a VGPR, so that mask-and-insert is
  // one v_and_or_b32 (a VOP3 op reads at most one SGPR or literal here).
  uint32_t magic = C::MAGIC;
  asm volatile("" : "+v"(magic));

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

  for (int c = kpart; c < nch; c += KS) {
    const int j = c * 64 + lane;
    const bool jok = j < L;
    const uint32_t k0 = (uint32_t)j * C::CPL;

    // weights, scales and biases of the R rows: all issued before any use.
    // A lane past the row end starts from OOB; adding a row offset (< 2^31)
    // keeps it out of range.
    const uint32_t wo = jok ? (uint32_t)j * 16u : OOB;
    u32x4_t wv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wv[r] = ld128<NT>(rw, wo, (uint32_t)(min(r, rlast) * L) * 16u);
    float sv[R][C::NSEG], bv[R][C::NSEG];
#pragma unroll
    for (int seg = 0; seg < C::NSEG; ++seg) {
      const uint32_t g = (k0 + seg * C::SEGK) >> B.gsh;
      const uint32_t so = jok ? g << ssh : OOB, bo = jok ? g << bsh : OOB;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t rr = (uint32_t)(min(r, rlast) * ng);
        sv[r][seg] = load_param<SBM>(rs, so, rr << ssh, B.sdt);
        bv[r][seg] = load_param<SBM>(rb, bo, rr << bsh, B.bdt);
      }
    }

    {
      u32x4_t raw[MT][C::XR];
      {
        const uint32_t xo = jok ? k0 * 2u : OOB;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int q = 0; q < C::XR; ++q) raw[m][q] = ld128(rx, xo + 16u * q, (uint32_t)min(m0 + m, M - 1) * K * 2u);
        if constexpr (XM == 1) {
          u32x4_t rup[MT][C::XR];
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int q = 0; q < C::XR; ++q) rup[m][q] = ld128(ru, xo + 16u * q, (uint32_t)min(m0 + m, M - 1) * K * 2u);
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int q = 0; q < C::XR; ++q) raw[m][q] = silu_gate_f16(raw[m][q], rup[m][q], B.act_f16 != 0);
        }
      }
      // every load of the chunk issued before any result is used: otherwise
      // the scheduler may put each parameter's use right after its load,
      // and each then waits for that load alone
      __builtin_amdgcn_sched_barrier(0);
      uint32_t xp[MT][C::XP];
      float xs[MT][C::NSEG];
#pragma unroll
      for (int m = 0; m < MT; ++m) C::build(raw[m], xp[m], xs[m]);

#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int seg = 0; seg < C::NSEG; ++seg) {
          float d[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m) d[m] = 0.f;
#pragma unroll
          for (int p = seg * C::PPS; p < (seg + 1) * C::PPS; ++p) {
            const uint32_t pr = C::pair(wv[r], p, magic);
#pragma unroll
            for (int m = 0; m < MT; ++m) d[m] = C::xdot(pr, xp[m], p, d[m]);
          }
          const float s = sv[r][seg], b = fmaf(-C::OFF, s, bv[r][seg]);
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[r][m] = fmaf(s, d[m], fmaf(b, xs[m][seg], acc[r][m]));
        }
    }
  }

  // row q of tot[g][m] holds the sum of acc[4g+q][m]
  float tot[R / 4][MT];
#pragma unroll
  for (int g = 0; g < R / 4; ++g)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v[4] = {acc[4 * g][m], acc[4 * g + 1][m], acc[4 * g + 2][m], acc[4 * g + 3][m]};
      tot[g][m] = wave_sum4(v);
    }
  const int q = lane >> 4;
  if (KS == 1) {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int g = 0; g < R / 4; ++g)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (4 * g + q < nrows && m0 + m < M)
            y[(long)(m0 + m) * N + row0 + 4 * g + q] = finish(tot[g][m], m0 + m, row0 + 4 * g + q);
    }
  } else {
    if ((lane & 15) == 0) {
#pragma unroll
      for (int g = 0; g < R / 4; ++g)
#pragma unroll
        for (int m = 0; m < MT; ++m) red[wave][(4 * g + q) * MT + m] = tot[g][m];
    }
    __syncthreads();
    if (kpart == 0 && lane < R * MT) {
      const int r = lane / MT, m = lane % MT;
      float v = 0.f;
      for (int p = 0; p < KS; ++p) v += red[rg * KS + p][lane];
      if (r < nrows && m0 + m < M) y[(long)(m0 + m) * N + row0 + r] = finish(v, m0 + m, row0 + r);
    }
    __syncthreads();  // red is written again by the next pass
  }
  }  // passes over x rows
}

// ---------------------------------------------------------------------------
// Skinny MFMA path: 4-bit codes, 2 <= M <= 16, 16-bit scales and biases.
// A dot2 GEMV spends one VALU op per code and per x row, so with several x
// rows it is bound by VALU, not by HBM.  Here the x rows (padded to 16) are
// the A operand of v_mfma_f32_16x16x32_{bf16,f16} and the codes, as
// exponent-bias values (code | 0x4300 = 128 + code in bf16, code | 0x6400 =
// 1024 + code in f16), the B operand, so a code costs well under one VALU op
// whatever M is.
//   * Every MFMA covers 32 codes of one group, so its result is scaled once:
//     y += s * sum(x * (off + q)) + (b - off * s) * X_g, with X_g the group
//     sums of x from one more MFMA against an all-ones B.
//   * A workgroup owns 64 columns and walks K in stages of 512 codes.  The
//     packed words of a stage (64 rows x 256 bytes) are loaded with every
//     wave-level load covering whole 128-byte lines (4 rows x 256 bytes)
//     into registers, three stages ahead, and written to LDS the stage
//     before their use; the fragments are read back from LDS.  A load
//     shaped like the MFMA operand (16 rows x 16-64 bytes per instruction)
//     reaches well under half the bandwidth.  Scales and biases take the
//     same route, two lanes per row.
//   * Wave w takes span w (codes 128w .. 128w+127) of every stage for all 64
//     columns (four 16-column blocks, one shared x fragment), and the four
//     partial sums are added through LDS at the end.
//   * In a span, lane (c, h) = (lane % 16, lane / 16) of block nb holds
//     column nb*16 + c and words h*wpg .. h*wpg + wpg - 1 of every group
//     (wpg = G / 32): MFMA j of a group takes word h*wpg + j, the x fragment
//     of row c comes from the same 8 columns, in the decode's pair order.
//   * LDS holds four stages in a ring; rows are 256 bytes with the 16-byte
//     pieces XOR-swizzled by row, so the 16 columns of a fragment read hit
//     16 different bank groups.
//   * Accumulator layout of the 16x16 MFMA: lane (c, h) holds column c and
//     rows 4h .. 4h+3.
struct MfmaDesc {
  const void* x;  // [M, K] activations (row stride kfull)
  const void* w;  // [N, K/8] uint32 (row stride kfull/8)
  const void* s;  // [N, K/G] 16-bit (row stride kfull/G)
  const void* b;  // [N, K/G] 16-bit
  void* y;        // [M, N]: activation dtype, or fp32 partial sums when part != 0
  int N, K, blk0;
  int kfull;      // K of the whole problem: a K slice has K < kfull
  int part;
  int pad;
};
struct MfmaBatch {
  MfmaDesc d[MAXP];
  int count, M;
};
static_assert(sizeof(MfmaBatch) <= 4096, "kernel arguments are limited to 4 KiB");

template <int G>
struct MfmaGeo {
  static constexpr int GPS = 128 / G, WPG = G / 32;
  static constexpr int STAGE = 64 * 256;  // packed words of a stage
  // Scales and biases arrive in chunks of 128 bytes (64 groups) per row,
  // CS stages, into one LDS region [parameter][row][128 bytes] whose 16-byte
  // pieces are XOR-swizzled by row.
  static constexpr int CS = 64 * G / 512;
  static constexpr int PREG = 2 * 64 * 128;
  // word of the span used by lane quarter h in MFMA j
  __device__ static constexpr int word(int h, int j) {
    return G == 128 ? 4 * h + j : (G == 64 ? (j >> 1) * 8 + 2 * h + (j & 1) : 4 * j + h);
  }
};
__device__ __forceinline__ int par_swz(int r, int piece) { return r * 128 + ((piece ^ ((r >> 1) & 7)) << 4); }

// Stage t of the MFMA GEMV: wait for this wave's copies of stage t's packed
// words (issued three stages ago; the 16 vector-memory operations issued
// since, two stages of copies and x loads, may still be in flight, and a
// parameter chunk's loads in between only make the wait stricter), barrier
// (stage t is in LDS for every wave, and every wave is done with stage t-1,
// whose buffer the copies of stage t+3 reuse), copy stage t+3 into LDS,
// load the x fragments of stage t+2, compute stage t.
template <class IssueW, class IssueX, class Compute, class X>
__device__ __forceinline__ void mfma_stage(IssueW& issue_w, IssueX& issue_x, Compute& compute, int t, bool active,
                                           const unsigned char* cur, const X& xc, unsigned char* nxt3, X& xf) {
  __builtin_amdgcn_s_waitcnt((16 & 15) | (7 << 4) | (0 << 8) | ((16 >> 4) << 14));  // vmcnt(16) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  issue_w(t + 3, nxt3);
  issue_x(t + 2, xf);
  __builtin_amdgcn_sched_barrier(0);
  if (active) compute(cur, xc, t);
}

template <bool F16, int G>
__global__ __launch_bounds__(256, 2) void gemv_mfma4_kernel(MfmaBatch B) {
  using Geo = MfmaGeo<G>;
  constexpr int NB = 4, GPS = Geo::GPS, WPG = Geo::WPG;
  using frag_t = typename std::conditional<F16, f16x8_t, bf16x8_t>::type;
  using X = u32x4_t[4];
  constexpr int CS = Geo::CS;
  constexpr float OFF = F16 ? 1024.f : 128.f;
  __shared__ __attribute__((aligned(1024))) unsigned char st0[Geo::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[Geo::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[Geo::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[Geo::STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char prm[Geo::PREG];

  const int bid = blockIdx.x;
  int lo = 0, hi = B.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (B.d[mid].blk0 <= bid) lo = mid; else hi = mid - 1;
  }
  const MfmaDesc& D = B.d[lo];
  const int N = D.N, K = D.K, M = B.M;
  const int KF = D.kfull, LF = KF >> 3, ngf = KF / G;  // row strides of x (values), W (words), params
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col0 = (bid - D.blk0) * 64;
  const int c = lane & 15, h = lane >> 4;
  const int L = K >> 3, ng = K / G, nsp = K >> 7, nst = (K + 511) >> 9;
  const int ncols = min(N - col0, 64);

  // Packed words go global -> LDS directly (a copy of 16 bytes per lane,
  // lane l of a wave's copy i landing at row 16i + 4*wave + l/16, slot
  // l % 16).  Slot s of row r holds the stage's 16-byte piece s ^ (r % 16),
  // so lane l reads that piece.  Rows past N are out of range (zeros); a
  // piece past the row end reads the next row.
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(static_cast<const uint32_t*>(D.w) + (long)col0 * LF,
                                                (uint32_t)(((ncols - 1) * LF + L) * 4));
  const int wrow = 4 * wave + (lane >> 4);
  const uint32_t wv = (uint32_t)(wrow * LF * 4 + (((lane & 15) ^ (wrow & 15)) * 16));
  // Scale (waves 0, 1) or bias (waves 2, 3) chunks: rows 32*(wave&1) + 8i +
  // lane/8 (i < 4), piece lane % 8 of the row's 128 bytes; every wave-level
  // load covers 8 whole rows' chunks.
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(static_cast<const uint16_t*>((wave >> 1) ? D.b : D.s) + (long)col0 * ngf,
                                                (uint32_t)(((ncols - 1) * ngf + ng) * 2));
  const int prow = 32 * (wave & 1) + (lane >> 3);
  const uint32_t pv = (uint32_t)(prow * ngf * 2 + (lane & 7) * 16);
  int pdst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pdst[i] = (wave >> 1) * 64 * 128 + par_swz(prow + 8 * i, lane & 7);
  const int nchunk = (nst + CS - 1) / CS;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(D.x, (uint32_t)(((M - 1) * KF + K) * 2));
  const uint32_t xv = c < M ? (uint32_t)(c * KF * 2) : OOB;

  // copies of stage tw's packed words into LDS stage st; a stage past the
  // end copies zeros (offsets out of range) into a buffer no one reads
  auto issue_w = [&](int tw, unsigned char* __restrict__ st) __attribute__((always_inline)) {
    const uint32_t wo = (tw < nst ? wv : OOB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int so = __builtin_amdgcn_readfirstlane(tw * 256 + 16 * i * LF * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(st + (16 * i + 4 * wave) * 256),
                                               16, wo, so, 0, 2);  // streamed once: non-temporal
    }
  };
  // loads of parameter chunk ch
  auto issue_p = [&](int ch, u32x4_t (&pr)[4]) __attribute__((always_inline)) {
    const uint32_t po = (ch < nchunk ? pv : OOB) + (uint32_t)ch * 128u;
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = ld128(rp, po + (uint32_t)(8 * i * ngf * 2));
  };
  auto put_p = [&](const u32x4_t (&pr)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(prm + pdst[i]) = pr[i];
  };
  // x fragments of span 4*tx + wave
  auto issue_x = [&](int tx, X& xr) __attribute__((always_inline)) {
    const int sp = 4 * tx + wave;
    const uint32_t xo = (sp < nsp ? xv : OOB) + (uint32_t)sp * 256u;
#pragma unroll
    for (int j = 0; j < 4; ++j) xr[j] = ld128(rx, xo + Geo::word(h, j) * 16);
  };

  uint32_t magic = F16 ? 0x64006400u : 0x43004300u;
  asm volatile("" : "+v"(magic));
  const uint32_t ones = F16 ? 0x3C003C00u : 0x3F803F80u;
  const frag_t onesf = __builtin_bit_cast(frag_t, u32x4_t{ones, ones, ones, ones});
  f32x4_t y[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) y[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const unsigned char* __restrict__ st, const X& xr, int t) __attribute__((always_inline)) {
    // packed words of the span for the four blocks
    u32x4_t wq[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const unsigned char* row = st + (nb * 16 + c) * 256;
      if constexpr (G == 128) {
        wq[nb] = *reinterpret_cast<const u32x4_t*>(row + (((4 * wave + h) ^ c) << 4));
      } else if constexpr (G == 64) {
        // whole 16-byte pieces, the lane's half selected after: two 8-byte
        // reads would be merged into one instruction that the compiler can
        // no longer tell apart from the LDS copies in flight (and would wait
        // for all of them)
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(row + (((4 * wave + (h >> 1)) ^ c) << 4));
        const u32x4_t b = *reinterpret_cast<const u32x4_t*>(row + (((4 * wave + 2 + (h >> 1)) ^ c) << 4));
        wq[nb] = (h & 1) ? u32x4_t{a.z, a.w, b.z, b.w} : u32x4_t{a.x, a.y, b.x, b.y};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wq[nb][j] = *reinterpret_cast<const uint32_t*>(row + (((4 * wave + j) ^ c) << 4) + h * 4);
      }
    }
    // the span's GPS scales and biases of column nb*16 + c: bytes
    // 2 * GPS * (4u + wave) .. + 2 * GPS of the row's chunk, u = t % CS
    uint32_t sp_[NB][2], bp_[NB][2];
    const int byte = 2 * GPS * (4 * (t % CS) + wave);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const unsigned char* ps = prm + par_swz(nb * 16 + c, byte >> 4) + (byte & 15);
      const unsigned char* pb = ps + 64 * 128;
      if constexpr (GPS == 4) {
        const uint2 a = *reinterpret_cast<const uint2*>(ps), b = *reinterpret_cast<const uint2*>(pb);
        sp_[nb][0] = a.x; sp_[nb][1] = a.y; bp_[nb][0] = b.x; bp_[nb][1] = b.y;
      } else if constexpr (GPS == 2) {
        sp_[nb][0] = *reinterpret_cast<const uint32_t*>(ps); bp_[nb][0] = *reinterpret_cast<const uint32_t*>(pb);
        sp_[nb][1] = 0; bp_[nb][1] = 0;
      } else {
        sp_[nb][0] = *reinterpret_cast<const uint16_t*>(ps); bp_[nb][0] = *reinterpret_cast<const uint16_t*>(pb);
        sp_[nb][1] = 0; bp_[nb][1] = 0;
      }
    }
#pragma unroll
    for (int gi = 0; gi < GPS; ++gi) {
      f32x4_t xs = {0.f, 0.f, 0.f, 0.f};
      f32x4_t a[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) a[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < WPG; ++jj) {
        const int j = gi * WPG + jj;
        const u32x4_t rr = xr[j];
        const frag_t af = __builtin_bit_cast(
            frag_t, u32x4_t{pair_lo(rr[0], rr[2]), pair_hi(rr[0], rr[2]), pair_lo(rr[1], rr[3]), pair_hi(rr[1], rr[3])});
        if constexpr (F16)
          xs = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, onesf, xs, 0, 0, 0);
        else
          xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, onesf, xs, 0, 0, 0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t wd = wq[nb][j];
          const frag_t bf = __builtin_bit_cast(
              frag_t, u32x4_t{(wd & 0x000F000Fu) | magic, ((wd >> 4) & 0x000F000Fu) | magic,
                              ((wd >> 8) & 0x000F000Fu) | magic, ((wd >> 12) & 0x000F000Fu) | magic});
          if constexpr (F16)
            a[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, a[nb], 0, 0, 0);
          else
            a[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, a[nb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t sh = (sp_[nb][gi >> 1] >> (16 * (gi & 1))) & 0xFFFFu;
        const uint32_t bh = (bp_[nb][gi >> 1] >> (16 * (gi & 1))) & 0xFFFFu;
        const float sv = F16 ? f16_bits_to_f32(sh) : bf16_bits_to_f32(sh);
        const float bv = fmaf(-OFF, sv, F16 ? f16_bits_to_f32(bh) : bf16_bits_to_f32(bh));
#pragma unroll
        for (int i = 0; i < 4; ++i) y[nb][i] = fmaf(sv, a[nb][i], fmaf(bv, xs[i], y[nb][i]));
      }
    }
  };

  // four stages in a ring, unrolled so that every buffer is static
  X x0, x1, x2, x3;
  u32x4_t pc[4];
  // parameter chunk 0 to LDS, chunk 1 in flight
  issue_p(0, pc);
  put_p(pc);
  __builtin_amdgcn_sched_barrier(0);
  issue_p(1, pc);
  // the prologue keeps the loop's load order (copies of stage t, then x of
  // stage t), so that 16 operations follow stage t's copies when stage t
  // waits for them
  issue_w(0, st0);
  issue_x(0, x0);
  __builtin_amdgcn_sched_barrier(0);
  issue_w(1, st1);
  issue_x(1, x1);
  __builtin_amdgcn_sched_barrier(0);
  issue_w(2, st2);
  __builtin_amdgcn_sched_barrier(0);
  // Whole rounds of four stages (K = 2048 n needs no other): a stage past
  // the end loads nothing and computes nothing, and the loop body has no
  // branch around a stage.  A chunk of CS (a multiple of 4) stages ends with
  // a round; then, once every wave is done with it, the next chunk's scales
  // and biases replace it in LDS (visible after the next barrier) and the
  // one after that is loaded.
  for (int t = 0; t < nst; t += 4) {
    mfma_stage(issue_w, issue_x, compute, t, 4 * t + wave < nsp, st0, x0, st3, x2);
    mfma_stage(issue_w, issue_x, compute, t + 1, 4 * t + 4 + wave < nsp, st1, x1, st0, x3);
    mfma_stage(issue_w, issue_x, compute, t + 2, 4 * t + 8 + wave < nsp, st2, x2, st1, x0);
    mfma_stage(issue_w, issue_x, compute, t + 3, 4 * t + 12 + wave < nsp, st3, x3, st2, x1);
    if ((t + 4) % CS == 0 && t + 4 < nst) {
      __builtin_amdgcn_s_barrier();
      put_p(pc);
      issue_p((t + 4) / CS + 1, pc);
    }
  }

  // the four waves' partial sums: block nb is finished by wave nb
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* red = reinterpret_cast<float*>(st0);  // [wave][nb][i][lane]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * NB + nb) * 4 + i) * 64 + lane] = y[nb][i];
  __syncthreads();
  const int col = wave * 16 + c;
  if (col >= ncols) return;
  uint16_t* yo = static_cast<uint16_t*>(D.y);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * h + i;
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) v += red[((q * NB + wave) * 4 + i) * 64 + lane];
    if (row < M) {
      if (D.part)
        static_cast<float*>(D.y)[(long)row * N + col0 + col] = v;
      else
        yo[(long)row * N + col0 + col] = f32_to_act_bits(v, F16);
    }
  }
}

// y = the sum of S fp32 partial planes [S][M*N] in slice order, rounded to
// the activation dtype
__global__ __launch_bounds__(256) void mfma_split_sum_kernel(const float* __restrict__ part, uint16_t* __restrict__ y,
                                                             long MN, int S, bool f16) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[(long)s * MN + i];
  y[i] = f32_to_act_bits(v, f16);
}

template <bool F16>
void launch_mfma4(int G, dim3 grid, hipStream_t s, const MfmaBatch& b) {
  if (G == 32) gemv_mfma4_kernel<F16, 32><<<grid, dim3(256), 0, s>>>(b);
  else if (G == 64) gemv_mfma4_kernel<F16, 64><<<grid, dim3(256), 0, s>>>(b);
  else gemv_mfma4_kernel<F16, 128><<<grid, dim3(256), 0, s>>>(b);
}

// x rows from which the MFMA kernel beats the dot2 one
constexpr int MFMA_MIN_M = 2;

template <int BITS, bool F16, int MT, int R, int XM = 0>
void launch_r(const GemvBatch& b, int blocks, int sbm, hipStream_t s) {
  if (sbm == 0)
    hipLaunchKernelGGL((gemv_affine_kernel<BITS, F16, MT, 0, R, XM>), dim3(blocks), dim3(256), 0, s, b);
  else if (sbm == 1)
    hipLaunchKernelGGL((gemv_affine_kernel<BITS, F16, MT, 1, R, XM>), dim3(blocks), dim3(256), 0, s, b);
  else
    hipLaunchKernelGGL((gemv_affine_kernel<BITS, F16, MT, 2, R, XM>), dim3(blocks), dim3(256), 0, s, b);
}

template <int BITS, bool F16, int XM = 0>
void launch_bits(const GemvBatch& b, int blocks, int sbm, int, hipStream_t s) {
  // x rows per pass: 1, 2, or 4 (passes of 4 rows from M = 3 on)
  if (b.M == 1)
    launch_r<BITS, F16, 1, 4, XM>(b, blocks, sbm, s);
  else if (b.M == 2)
    launch_r<BITS, F16, 2, 4, XM>(b, blocks, sbm, s);
  else
    launch_r<BITS, F16, 4, 4, XM>(b, blocks, sbm, s);
}

// x_p[m, j] = x[m, k_perm[j]] (16-bit values): one thread per 8 outputs of
// a row.  An index outside [0, K) reads 0.
__global__ __launch_bounds__(256) void permute_x_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ kp,
                                                        uint16_t* __restrict__ xp, int M, int K) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const int cpr = K / 8;
  if (i >= (long)M * cpr) return;
  const int m = (int)(i / cpr), j0 = (int)(i % cpr) * 8;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp, (uint32_t)K * 4u);
  uint32_t e[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t k = ld32(rk, (uint32_t)(j0 + t) * 4u);
    e[t] = ld16(rx, k < (uint32_t)K ? ((uint32_t)m * K + k) * 2u : OOB);
  }
  *reinterpret_cast<u32x4_t*>(xp + (long)m * K + j0) =
      u32x4_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
}

// ws_used: bytes at the start of the stream's workspace that the caller
// still needs (permuted copies of x)
hipError_t launch_gemv_core(const AffineArgs* probs, int count, hipStream_t s, size_t ws_used);

// Rows that are not whole 16-byte chunks (K*BITS % 128 != 0; with G >= 32
// only 2-bit codes with K an odd multiple of 32): one wave per row of W,
// lanes over the row's words, 4-byte loads, k_perm read per code.  A plain
// path for a rare shape, exact in the same way as the main kernel: per word
// (never across a group, since P <= 16 <= G) s * sum(q*x) + b * sum(x).
template <int BITS>
__global__ __launch_bounds__(256) void gemv_tail_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ w,
                                                        const void* __restrict__ sc, const void* __restrict__ bi,
                                                        const int32_t* __restrict__ kp, uint16_t* __restrict__ y,
                                                        int M, int N, int K, int G, int sdt, int bdt, bool f16) {
  constexpr int P = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (n >= N) return;  // a whole wave leaves together
  const int nw = K / P, ng = K / G;
  const uint32_t* wr = w + (long)n * nw;
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.f;
  for (int j = lane; j < nw; j += 64) {
    const uint32_t word = wr[j];
    const int g = j * P / G;
    const float s = load_as_f32(sc, (long)n * ng + g, sdt);
    const float b = load_as_f32(bi, (long)n * ng + g, bdt);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m >= M) continue;  // (uniform)
      float dq = 0.f, sx = 0.f;
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int k = j * P + i;
        const uint32_t h = x[(long)m * K + (kp ? kp[k] : k)];
        const float xv = f16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
        dq = fmaf((float)((word >> (BITS * i)) & MASK), xv, dq);
        sx += xv;
      }
      acc[m] = fmaf(s, dq, fmaf(b, sx, acc[m]));
    }
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m >= M) continue;  // (uniform)
    const float v = wave_sum(acc[m]);
    if (lane == 0) y[(long)m * N + n] = f32_to_act_bits(v, f16);
  }
}

hipError_t launch_gemv_tail(const AffineArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + 3) / 4));
  const bool f16 = a.act_dt == F16;
  auto* x = static_cast<const uint16_t*>(a.x);
  auto* y = static_cast<uint16_t*>(a.y);
  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  if (a.bits == 2)
    hipLaunchKernelGGL(gemv_tail_kernel<2>, grid, dim3(256), 0, s, x, a.w, a.scales, a.biases, a.k_perm, y, M, N, K,
                       a.G, a.s_dt, a.b_dt, f16);
  else if (a.bits == 4)
    hipLaunchKernelGGL(gemv_tail_kernel<4>, grid, dim3(256), 0, s, x, a.w, a.scales, a.biases, a.k_perm, y, M, N, K,
                       a.G, a.s_dt, a.b_dt, f16);
  else
    hipLaunchKernelGGL(gemv_tail_kernel<8>, grid, dim3(256), 0, s, x, a.w, a.scales, a.biases, a.k_perm, y, M, N, K,
                       a.G, a.s_dt, a.b_dt, f16);
  return hipGetLastError();
}

}  // namespace

// Problems with a column permutation run on a permuted copy of x, written
// by one small kernel per distinct (x, k_perm) pair into the stream's
// workspace; then every problem takes the unpermuted kernels.
hipError_t launch_gemv_grouped(const AffineArgs* probs, int count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  // rows that are not whole 16-byte chunks take the plain tail kernel, one
  // launch per problem; the rest go on together
  bool ragged = false;
  for (int i = 0; i < count; ++i) ragged |= (probs[i].K * probs[i].bits) % 128 != 0;
  if (ragged) {
    std::vector<AffineArgs> rest;
    for (int i = 0; i < count; ++i) {
      if ((probs[i].K * probs[i].bits) % 128 != 0) {
        const hipError_t e = launch_gemv_tail(probs[i], s);
        if (e != hipSuccess) return e;
      } else {
        rest.push_back(probs[i]);
      }
    }
    return rest.empty() ? hipSuccess : launch_gemv_grouped(rest.data(), (int)rest.size(), s);
  }
  bool any = false;
  for (int i = 0; i < count; ++i) any |= probs[i].k_perm != nullptr;
  if (!any) return launch_gemv_core(probs, count, s, 0);
  std::vector<AffineArgs> q(probs, probs + count);
  std::vector<int> src(count, -1);  // problem whose permuted x this one shares
  size_t total = 0;
  std::vector<size_t> off(count, 0);
  for (int i = 0; i < count; ++i) {
    if (!q[i].k_perm) continue;
    for (int j = 0; j < i && src[i] < 0; ++j)
      if (q[j].k_perm == q[i].k_perm && probs[j].x == q[i].x && q[j].K == q[i].K) src[i] = j;
    if (src[i] >= 0) continue;
    if (q[i].M * q[i].K * 2 >= (int64_t(1) << 31)) return hipErrorNotSupported;
    off[i] = total;
    total += ((size_t)q[i].M * q[i].K * 2 + 255) & ~size_t(255);
  }
  char* scratch = nullptr;
  hipError_t e = stream_workspace(s, total, (void**)&scratch);
  if (e != hipSuccess) return e;
  for (int i = 0; i < count && e == hipSuccess; ++i) {
    if (!q[i].k_perm) continue;
    if (src[i] < 0) {
      const long chunks = q[i].M * q[i].K / 8;
      hipLaunchKernelGGL(permute_x_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s,
                         static_cast<const uint16_t*>(q[i].x), q[i].k_perm, (uint16_t*)(scratch + off[i]), (int)q[i].M,
                         (int)q[i].K);
      e = hipGetLastError();
      q[i].x = scratch + off[i];
    } else {
      q[i].x = q[src[i]].x;
    }
    q[i].k_perm = nullptr;
  }
  if (e == hipSuccess) e = launch_gemv_core(q.data(), count, s, total);
  return e;
}

namespace {

hipError_t launch_gemv_core(const AffineArgs* probs, int count, hipStream_t s, size_t ws_used) {
  if (count <= 0) return hipSuccess;
  const AffineArgs& a0 = probs[0];
  const int M = (int)a0.M, bits = a0.bits;
  if (M < 1 || M > 16) return hipErrorInvalidValue;
  const bool f16 = a0.act_dt == F16;
  int sbm = 2;
  if (a0.s_dt == a0.act_dt && a0.b_dt == a0.act_dt) sbm = f16 ? 1 : 0;
  int gsh = 0;
  while ((1 << gsh) < a0.G) ++gsh;
  for (int p0 = 0; p0 < count; p0 += MAXP) {
    GemvBatch b{};
    b.M = M;
    b.gsh = gsh;
    b.sdt = a0.s_dt;
    b.bdt = a0.b_dt;
    // 4 rows per wave: 8 rows (half the x preparation per row) measured
    // slower on every shape, from lower occupancy (109 vs 68 VGPRs).
    const int R = 4;
    int64_t blocks = 0;
    for (int i = 0; i < MAXP && p0 + i < count; ++i) {
      const AffineArgs& a = probs[p0 + i];
      if (a.N == 0) continue;
      // buffer offsets are 32-bit: R rows of W, their parameters and all of x must fit
      if (a.K * a.bits / 8 * R >= (int64_t(1) << 31) || a.M * a.K * 2 >= (int64_t(1) << 31)) return hipErrorNotSupported;
      const int64_t L = a.K * a.bits / 128;
      const int64_t nch = (L + 63) / 64;
      const int ksh = nch >= 4 ? 2 : (nch >= 2 ? 1 : 0);  // K split over 1, 2 or 4 waves
      const int64_t rows_per_wg = (4 >> ksh) * R;
      const int64_t nblk = (a.N + rows_per_wg - 1) / rows_per_wg;
      if (blocks + nblk >= (int64_t(1) << 31)) return hipErrorNotSupported;
      GemvDesc& d = b.d[b.count++];
      d.x = a.x;
      d.w = a.w;
      d.s = a.scales;
      d.b = a.biases;
      d.y = a.y;
      d.N = (int)a.N;
      d.K = (int)a.K;
      d.blk0 = (int)blocks;
      d.ks = ksh;
      blocks += nblk;
    }
    if (blocks == 0) continue;
    // 4-bit codes with several x rows, K a multiple of 512, 16-bit scales
    // and biases of the activation type: the skinny MFMA kernel
    bool mfma = bits == 4 && M >= MFMA_MIN_M && sbm != 2 && (a0.G == 32 || a0.G == 64 || a0.G == 128);
    for (int i = 0; mfma && i < b.count; ++i) {
      const GemvDesc& d = b.d[i];
      // whole 512-code stages, and rows of scales and biases a multiple of
      // 16 bytes, so that every chunk load is aligned
      mfma = d.K % 512 == 0 && (d.K / a0.G) % 8 == 0 && (int64_t)d.K * 32 < (int64_t(1) << 31) &&
             (((uintptr_t)d.w | (uintptr_t)d.s | (uintptr_t)d.b) & 15) == 0;
    }
    // up to 4 x rows, a grid of fewer than 128 64-column workgroups is
    // latency-bound, and the dot2 kernel, with a workgroup per 16 rows or
    // fewer, is faster (M = 4, N = K = 4096: 5.7 against 9.5 us)
    if (mfma && M <= 4) {
      int64_t mb = 0;
      for (int i = 0; i < b.count; ++i) mb += (b.d[i].N + 63) / 64;
      if (mb < 128) mfma = false;
    }
    if (mfma) {
      int64_t mblocks = 0;
      for (int i = 0; i < b.count; ++i) mblocks += (b.d[i].N + 63) / 64;
      // K split when the grid is narrow (64 workgroups or fewer: a single
      // call with N <= 4096): slices of whole 1024-code pieces that keep the
      // scale rows 16-byte aligned (8 groups), as many as keep the grid
      // within one round of 512 workgroups (two per CU) and the descriptors
      // within one launch; each slice writes fp32 partials, and a second
      // kernel adds them.  From 128 workgroups on, the partials and the
      // second kernel cost more than they save (M = 4, N = 11008, K = 4096:
      // 12.6 against 10.2 us); at 32, M = 16, N = 2048, K = 8192 goes from
      // 16.3 to 10.4 us.
      int S = 1;
      const int q = std::max(1024, 8 * (int)a0.G);
      if (mblocks <= 64) {
        int kmin = 1 << 30;
        for (int i = 0; i < b.count; ++i) kmin = std::min(kmin, b.d[i].K / q);
        S = (int)std::max<int64_t>(1, std::min<int64_t>({512 / mblocks, (int64_t)kmin, (int64_t)(MAXP / b.count)}));
      }
      MfmaBatch bm{};
      bm.M = M;
      int nd = 0;
      mblocks = 0;
      float* part = nullptr;
      std::vector<int> slices(b.count, 1);
      if (S > 1) {
        size_t bytes = 0;
        for (int i = 0; i < b.count; ++i) {
          const int per = (b.d[i].K / S + q - 1) / q * q;
          slices[i] = (b.d[i].K + per - 1) / per;  // no empty slice
          bytes += (size_t)slices[i] * M * b.d[i].N * 4;
        }
        const size_t base = (ws_used + 255) & ~size_t(255);
        char* ws = nullptr;
        hipError_t e = stream_workspace(s, base + bytes, (void**)&ws);
        if (e != hipSuccess) return e;
        part = reinterpret_cast<float*>(ws + base);
      }
      std::vector<float*> plane(b.count, nullptr);
      float* next = part;
      for (int i = 0; i < b.count; ++i) {
        const GemvDesc& d = b.d[i];
        const int per = slices[i] > 1 ? (d.K / S + q - 1) / q * q : d.K;
        plane[i] = next;
        for (int j = 0; j < slices[i]; ++j) {
          MfmaDesc& e = bm.d[nd++];
          const int k0 = j * per;
          e.x = static_cast<const uint16_t*>(d.x) + k0;
          e.w = static_cast<const uint32_t*>(d.w) + k0 / 8;
          e.s = static_cast<const uint16_t*>(d.s) + k0 / a0.G;
          e.b = static_cast<const uint16_t*>(d.b) + k0 / a0.G;
          e.N = d.N;
          e.K = std::min(per, d.K - k0);
          e.kfull = d.K;
          e.blk0 = (int)mblocks;
          if (slices[i] > 1) {
            e.y = next + (size_t)j * M * d.N;
            e.part = 1;
          } else {
            e.y = d.y;
            e.part = 0;
          }
          mblocks += (d.N + 63) / 64;
        }
        if (slices[i] > 1) next += (size_t)slices[i] * M * d.N;
      }
      bm.count = nd;
      if (f16) launch_mfma4<true>((int)a0.G, dim3((unsigned)mblocks), s, bm);
      else launch_mfma4<false>((int)a0.G, dim3((unsigned)mblocks), s, bm);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      for (int i = 0; i < b.count; ++i) {
        if (slices[i] == 1) continue;
        const long MN = (long)M * b.d[i].N;
        hipLaunchKernelGGL(mfma_split_sum_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, plane[i],
                           static_cast<uint16_t*>(b.d[i].y), MN, slices[i], f16);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      continue;
    }
    switch (bits) {
      case 2: f16 ? launch_bits<2, true>(b, (int)blocks, sbm, R, s) : launch_bits<2, false>(b, (int)blocks, sbm, R, s); break;
      case 4: f16 ? launch_bits<4, true>(b, (int)blocks, sbm, R, s) : launch_bits<4, false>(b, (int)blocks, sbm, R, s); break;
      default: f16 ? launch_bits<8, true>(b, (int)blocks, sbm, R, s) : launch_bits<8, false>(b, (int)blocks, sbm, R, s); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemv_affine(const AffineArgs& a, hipStream_t s) { return launch_gemv_grouped(&a, 1, s); }

// y = W (silu(gate) * up) [+ resid]: the dot2 kernel with the gated input
// formed in registers (XM = 1).  a.x is the gate; rows must be whole
// 16-byte chunks (K*bits % 128 == 0) and there is no k_perm.
hipError_t launch_gemv_silu(const AffineArgs& a, const void* up, const void* resid, hipStream_t s) {
  const int M = (int)a.M;
  if (M < 1 || M > 16 || (a.K * a.bits) % 128 != 0 || a.k_perm) return hipErrorInvalidValue;
  if (a.K * a.bits / 8 * 4 >= (int64_t(1) << 31) || a.M * a.K * 2 >= (int64_t(1) << 31)) return hipErrorNotSupported;
  GemvBatch b{};
  b.M = M;
  int gsh = 0;
  while ((1 << gsh) < a.G) ++gsh;
  b.gsh = gsh;
  b.sdt = a.s_dt;
  b.bdt = a.b_dt;
  b.up = up;
  b.resid = resid;
  b.act_f16 = a.act_dt == F16;
  // the f16 code path: scales and biases take the any-dtype loader unless
  // they are both f16
  const int sbm = (a.s_dt == F16 && a.b_dt == F16) ? 1 : 2;
  const int64_t L = a.K * a.bits / 128, nch = (L + 63) / 64;
  const int ksh = nch >= 4 ? 2 : (nch >= 2 ? 1 : 0);
  const int64_t rows_per_wg = (4 >> ksh) * 4;
  const int64_t blocks = (a.N + rows_per_wg - 1) / rows_per_wg;
  if (blocks >= (int64_t(1) << 31)) return hipErrorNotSupported;
  GemvDesc& d = b.d[b.count++];
  d.x = a.x;
  d.w = a.w;
  d.s = a.scales;
  d.b = a.biases;
  d.y = a.y;
  d.N = (int)a.N;
  d.K = (int)a.K;
  d.blk0 = 0;
  d.ks = ksh;
  switch (a.bits) {
    case 2: launch_bits<2, true, 1>(b, (int)blocks, sbm, 4, s); break;
    case 4: launch_bits<4, true, 1>(b, (int)blocks, sbm, 4, s); break;
    default: launch_bits<8, true, 1>(b, (int)blocks, sbm, 4, s); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode chain: the linears of a decode step in dependency order, one launch.
//
// A decode step runs its linears in stages: q/k/v read the hidden state, o
// reads their result, gate/up read o's, down reads silu(gate) * up (the
// fused inputs of the mlx_int8.rs API page: `gemv_gate_up`,
// `gemv_silu_gate`, `gemv_silu_gate_resid`).  Here one cooperative launch
// of two workgroups per CU runs every stage:
//   * a stage's linears are cut into items of about 16 KiB of codes (16 rows
//     at K <= 2048, 8 at K <= 4096, 4 beyond, the waves then splitting K),
//     dealt to the workgroups in turn;
//   * a workgroup loads the weights, scales and biases of its next item
//     before it computes the current one, and the first item of a stage
//     before it waits for the stage before: weights do not depend on the
//     chain, so their latency overlaps the previous stage and the wait;
//   * a workgroup reads an item's input once per stage into LDS (x, or
//     silu(gate) * x rounded to f16, as in qgemv_affine_silu_gate), and its
//     waves read it from there;
//   * stages meet at arrival counts: a workgroup waits for its stores, then
//     adds 1 to one of CHAIN_SUB sub counts of the stage, and the last
//     arrival of a sub count raises the stage's top count; a workgroup with
//     an item in the next stage polls the top count.  Outputs are written
//     through to memory and inputs read from it at device scope (sc1), and
//     the counts are device-scope atomics, so no cache is written back or
//     invalidated and the XCDs' L2s keep their lines.  The wait is bounded:
//     past CHAIN_POLLS polls it sets an error word and goes on, so no launch
//     can hang (with a cooperative launch every workgroup is resident and
//     the bound is never reached);
//   * the last workgroup to finish sets the counts back to zero.
// The arithmetic of an item is the dot2 GEMV's (4-bit codes, exact weights,
// fp32 sums).
namespace {

constexpr int CP_DEV = 16;                   // cache policy sc1: device scope
constexpr uint32_t CHAIN_POLLS = 1u << 20;   // polls of one count before giving up
// Arrival counts: per stage CHAIN_SUB counts (workgroup bid counts in
// bid % CHAIN_SUB) and a top count that the last arrival of each sub count
// raises; every count on a cache line of its own.
constexpr int CHAIN_SUB = 16;
constexpr int CHAIN_LINE = 32;                       // uint32 per 128-byte line
constexpr int CHAIN_STAGE = (CHAIN_SUB + 1) * CHAIN_LINE;  // uint32 per stage

struct ChainLin {
  const uint16_t* x;      // [K]; with a gate: the up projection
  const uint16_t* gate;   // [K] or null: the input is silu(gate) * x
  const uint16_t* resid;  // [N] or null: added to y before its rounding
  const void* w;          // [N, K/8]
  const void* s;          // [N, K/G]
  const void* b;          // [N, K/G]
  uint16_t* y;            // [N]
  int N, K, ks;           // ks: log2 of the waves that split a row's K
};

// The weights, scales and biases of one item's first K chunk, per wave
struct ChainRegs {
  u32x4_t wv[4];
  float sv[4], bv[4];
};

template <int SBM>
__device__ __forceinline__ void chain_load(const ChainLin& D, int row0base, int gsh, ChainRegs& g) {
  constexpr int R = 4;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ksh = D.ks, N = D.N, K = D.K;
  const int row0 = row0base + (wave >> ksh) * R, kpart = wave & ((1 << ksh) - 1);
  const int L = K / 32, ng = K >> gsh;  // 16-byte chunks per row (4-bit)
  const int nrows = __builtin_amdgcn_readfirstlane(min(max(N - row0, 0), R));
  const int rlast = max(nrows - 1, 0);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(static_cast<const uint32_t*>(D.w) + (long)row0 * L * 4, (uint32_t)(nrows * L * 16));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<const char*>(D.s) + (long)row0 * ng * 2, (uint32_t)(nrows * ng * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(static_cast<const char*>(D.b) + (long)row0 * ng * 2, (uint32_t)(nrows * ng * 2));
  const int j = kpart * 64 + lane;
  const bool jok = j < L;
  const uint32_t wo = jok ? (uint32_t)j * 16u : OOB;
  const uint32_t gr = ((uint32_t)j * 32u) >> gsh;
  const uint32_t po = jok ? gr * 2u : OOB;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t rr = (uint32_t)min(r, rlast);
    g.wv[r] = ld128<NT>(rw, wo, rr * (uint32_t)L * 16u);
    g.sv[r] = load_param<SBM>(rs, po, rr * (uint32_t)ng * 2u, 0);
    g.bv[r] = load_param<SBM>(rb, po, rr * (uint32_t)ng * 2u, 0);
  }
}

// The stage's top count polled by thread 0 until every sub count has
// closed (min(P, CHAIN_SUB) of them), then a barrier.
__device__ __forceinline__ void chain_wait(uint32_t* stage, int P, uint32_t* err) {
  if (threadIdx.x == 0) {
    uint32_t n = 0;
    const uint32_t want = (uint32_t)min(P, CHAIN_SUB);
    while (__hip_atomic_load(stage + CHAIN_SUB * CHAIN_LINE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
      __builtin_amdgcn_s_sleep(1);
      if (++n == CHAIN_POLLS) {
        __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// Every wave's stores done (written through), then one arrival in the sub
// count of bid; the sub count's last arrival raises the top count.
__device__ __forceinline__ void chain_arrive(uint32_t* stage, int P, int bid) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int g = bid % CHAIN_SUB;
    const uint32_t size = (uint32_t)(P / CHAIN_SUB + (g < P % CHAIN_SUB ? 1 : 0));
    if (__hip_atomic_fetch_add(stage + g * CHAIN_LINE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == size - 1)
      __hip_atomic_fetch_add(stage + CHAIN_SUB * CHAIN_LINE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The item's input into LDS (xl, K values): x, or silu(gate) * x rounded to
// f16 (as qgemv_affine_silu_gate), read from memory at device scope; every
// load of a thread issued before any is used.
template <bool ACT_F16>
__device__ __forceinline__ void chain_stage_x(const ChainLin& D, uint16_t* xl) {
  constexpr int U = 4;  // 16-byte loads per thread per pass: 256 * 8 * U values
  const int K = D.K;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(D.x, (uint32_t)(K * 2));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(D.gate, D.gate ? (uint32_t)(K * 2) : 0u);
  __syncthreads();  // every wave done with the previous input
  for (int i0 = 0; i0 < K; i0 += 256 * 8 * U) {
    u32x4_t v[U], g[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t o = (uint32_t)(i0 + (u * 256 + (int)threadIdx.x) * 8) * 2u;  // past K: zeros
      v[u] = ld128<CP_DEV>(rx, o);
      if (D.gate) g[u] = ld128<CP_DEV>(rg, o);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + (u * 256 + (int)threadIdx.x) * 8;
      if (i < K)
        *reinterpret_cast<u32x4_t*>(xl + i) = D.gate ? silu_gate_f16(g[u], v[u], ACT_F16) : v[u];
    }
  }
  __syncthreads();
}

// One item: rows row0base.. of D (4 per row group of waves), the first K
// chunk's operands in g, the input in LDS (xl).  F16C: the f16 code path
// (f16 activations, or a gated input).
template <bool F16C, int SBM>
__device__ __forceinline__ void chain_compute(const ChainLin& D, int row0base, int gsh, bool out_f16, const ChainRegs& g,
                                              const uint16_t* xl, float (&red)[4][4]) {
  using C = Codec<4, F16C>;
  constexpr int R = 4;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ksh = D.ks, KS = 1 << ksh, N = D.N, K = D.K;
  const int rg = wave >> ksh, kpart = wave & (KS - 1);
  const int row0 = row0base + rg * R;
  const int L = K / 32, nch = (L + 63) >> 6, ng = K >> gsh;
  const int nrows = __builtin_amdgcn_readfirstlane(min(max(N - row0, 0), R));
  const int rlast = max(nrows - 1, 0);
  uint32_t magic = C::MAGIC;
  asm volatile("" : "+v"(magic));
  float acc[R] = {0.f, 0.f, 0.f, 0.f};
  auto chunk = [&](int c, const u32x4_t (&wv)[R], const float (&sv)[R], const float (&bv)[R]) {
    const int j = c * 64 + lane;
    const bool jok = j < L;  // (lanes past the row read x as 0: their codes decode to the offset, not 0)
    const u32x4_t* xq = reinterpret_cast<const u32x4_t*>(xl + (jok ? j : 0) * 32);  // 32 codes = 64 bytes of x
    u32x4_t raw[C::XR];
#pragma unroll
    for (int q = 0; q < C::XR; ++q) {
      const u32x4_t v = xq[q];
      raw[q] = jok ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
    uint32_t xp[C::XP];
    float xs[C::NSEG];
    C::build(raw, xp, xs);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float d = 0.f;
#pragma unroll
      for (int p = 0; p < C::PPS; ++p) d = C::xdot(C::pair(wv[r], p, magic), xp, p, d);
      const float s = sv[r], b = fmaf(-C::OFF, s, bv[r]);
      acc[r] = fmaf(s, d, fmaf(b, xs[0], acc[r]));
    }
  };
  if (kpart < nch) chunk(kpart, g.wv, g.sv, g.bv);
  for (int c = kpart + KS; c < nch; c += KS) {  // rows longer than KS chunks
    ChainRegs h;
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(static_cast<const uint32_t*>(D.w) + (long)row0 * L * 4, (uint32_t)(nrows * L * 16));
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(static_cast<const char*>(D.s) + (long)row0 * ng * 2, (uint32_t)(nrows * ng * 2));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(static_cast<const char*>(D.b) + (long)row0 * ng * 2, (uint32_t)(nrows * ng * 2));
    const int j = c * 64 + lane;
    const bool jok = j < L;
    const uint32_t wo = jok ? (uint32_t)j * 16u : OOB, po = jok ? (((uint32_t)j * 32u) >> gsh) * 2u : OOB;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t rr = (uint32_t)min(r, rlast);
      h.wv[r] = ld128<NT>(rw, wo, rr * (uint32_t)L * 16u);
      h.sv[r] = load_param<SBM>(rs, po, rr * (uint32_t)ng * 2u, 0);
      h.bv[r] = load_param<SBM>(rb, po, rr * (uint32_t)ng * 2u, 0);
    }
    chunk(c, h.wv, h.sv, h.bv);
  }
  // row q of tot holds the sum of acc[q]
  const float tot = wave_sum4(acc);
  const int q = lane >> 4;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(D.y, (uint32_t)(N * 2));
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(D.resid, D.resid ? (uint32_t)(N * 2) : 0u);
  auto store = [&](int row, float v) {
    if (D.resid) {
      const uint32_t rb = __builtin_amdgcn_raw_buffer_load_b16(rr, (uint32_t)row * 2u, 0, CP_DEV);
      v += out_f16 ? f16_bits_to_f32(rb) : bf16_bits_to_f32(rb);
    }
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_act_bits(v, out_f16), ry, (uint32_t)row * 2u, 0, CP_DEV);
  };
  if (KS == 1) {
    if ((lane & 15) == 0 && q < nrows) store(row0 + q, tot);
  } else {
    if ((lane & 15) == 0) red[wave][q] = tot;
    __syncthreads();
    if (kpart == 0 && lane < nrows) {
      float v = 0.f;
      for (int p = 0; p < KS; ++p) v += red[rg * KS + p][lane];
      store(row0 + lane, v);
    }
    __syncthreads();  // red is written again by the next item
  }
}

// The item after `it` of stage st for workgroup bid, in this stage or the
// first later stage that has one: (stage, item), or (nst, -1).
__device__ __forceinline__ int2 chain_next(const int* __restrict__ sb, int nst, int st, int it, int P, int bid) {
  if (it + P < sb[st + 1]) return make_int2(st, it + P);
  for (int s = st + 1; s < nst; ++s)
    if (sb[s] + bid < sb[s + 1]) return make_int2(s, sb[s] + bid);
  return make_int2(nst, -1);
}

// bar: the stages' counts (CHAIN_STAGE uint32 each, stages 0 .. nst-2),
// then the finished count and the error word (set by a wait that gave up)
template <bool ACT_F16>
__global__ __launch_bounds__(256) void gemv_chain_kernel(const ChainLin* __restrict__ lins, const int2* __restrict__ items,
                                                          const int* __restrict__ sb, int nst, int gsh,
                                                          uint32_t* __restrict__ bar) {
  constexpr int SBM = ACT_F16 ? 1 : 0;
  __shared__ float red[4][4];
  extern __shared__ __attribute__((aligned(16))) uint16_t xl[];  // the current input: K values
  const int P = gridDim.x, bid = blockIdx.x;
  uint32_t* done = bar + (long)nst * CHAIN_STAGE;
  uint32_t* err = done + CHAIN_LINE;
  auto load = [&](int it, ChainRegs& g) {
    const int2 w = items[it];
    chain_load<SBM>(lins[w.x], w.y, gsh, g);
  };
  ChainRegs cur, nxt;
  // first item of the workgroup: the first stage that has one
  int2 at = make_int2(nst, -1);
  for (int s = 0; s < nst; ++s)
    if (sb[s] + bid < sb[s + 1]) {
      at = make_int2(s, sb[s] + bid);
      break;
    }
  if (at.y >= 0) load(at.y, cur);
  int arrived = 0;  // stages 0 .. arrived-1 counted
  int staged_st = -1;  // the stage and input whose values xl holds
  const uint16_t* staged_x = nullptr;
  const uint16_t* staged_g = nullptr;
  while (at.y >= 0) {
    const int st = at.x;
    // stages done before this one: count them, then wait for the last
    for (; arrived < st; ++arrived) chain_arrive(bar + (long)arrived * CHAIN_STAGE, P, bid);
    const int2 nx = chain_next(sb, nst, st, at.y, P, bid);
    if (nx.y >= 0) load(nx.y, nxt);  // the next item's operands, before the wait and the work
    if (st > 0 && at.y == sb[st] + bid) chain_wait(bar + (long)(st - 1) * CHAIN_STAGE, P, err);
    const int2 w = items[at.y];
    const ChainLin& D = lins[w.x];
    // the input into LDS once per stage and (x, gate) pair: a later stage may
    // have rewritten a buffer of the same address, so a stage starts afresh
    if (st != staged_st || D.x != staged_x || D.gate != staged_g) {
      chain_stage_x<ACT_F16>(D, xl);
      staged_st = st;
      staged_x = D.x;
      staged_g = D.gate;
    }
    if (D.gate)
      chain_compute<true, SBM>(D, w.y, gsh, ACT_F16, cur, xl, red);
    else
      chain_compute<ACT_F16, SBM>(D, w.y, gsh, ACT_F16, cur, xl, red);
    cur = nxt;
    at = nx;
  }
  for (; arrived < nst - 1; ++arrived) chain_arrive(bar + (long)arrived * CHAIN_STAGE, P, bid);
  // the last workgroup to finish sets the counts back to zero
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(P - 1)) {
    for (int st = 0; st + 1 < nst; ++st)
      for (int g = 0; g <= CHAIN_SUB; ++g)
        __hip_atomic_store(bar + (long)st * CHAIN_STAGE + g * CHAIN_LINE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

// Host side of a chain: the descriptors and the stage items in one device
// allocation, built once; each run is one cooperative launch.
struct ChainPlan {
  int dev, act_f16, gsh, nst, P, lds;
  void* mem;
  ChainLin* lins;
  int2* items;
  int* sb;
  uint32_t* bar;
};

hipError_t chain_plan_create(const ChainSpec* spec, int count, int G, int act_f16, void** out) {
  *out = nullptr;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int gsh = 0;
  while ((1 << gsh) < G) ++gsh;
  const int nst = spec[count - 1].stage + 1;
  std::vector<ChainLin> lins(count);
  std::vector<int2> items;
  std::vector<int> sb(nst + 1, 0);
  int next = 0;
  for (int st = 0; st < nst; ++st) {
    sb[st] = (int)items.size();
    for (; next < count && spec[next].stage == st; ++next) {
      const ChainSpec& c = spec[next];
      const int64_t L = c.K / 32, nch = (L + 63) / 64;
      const int ksh = nch >= 4 ? 2 : (nch >= 2 ? 1 : 0);
      ChainLin& d = lins[next];
      d.x = static_cast<const uint16_t*>(c.x);
      d.gate = static_cast<const uint16_t*>(c.gate);
      d.resid = static_cast<const uint16_t*>(c.resid);
      d.w = c.w;
      d.s = c.scales;
      d.b = c.biases;
      d.y = static_cast<uint16_t*>(c.y);
      d.N = (int)c.N;
      d.K = (int)c.K;
      d.ks = ksh;
      const int rows = (4 >> ksh) * 4;
      for (int64_t r = 0; r < c.N; r += rows) items.push_back(make_int2(next, (int)r));
    }
  }
  sb[nst] = (int)items.size();
  int64_t kmax = 0;
  for (int i = 0; i < count; ++i) kmax = std::max<int64_t>(kmax, spec[i].K);
  const int lds = (int)(kmax * 2);  // the input of the longest row
  if (items.size() >= (size_t(1) << 30)) return hipErrorNotSupported;
  // workgroups all resident at once (cooperative launch)
  const void* k = act_f16 ? reinterpret_cast<const void*>(gemv_chain_kernel<true>)
                          : reinterpret_cast<const void*>(gemv_chain_kernel<false>);
  e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 256, (size_t)lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorNotSupported;
  const size_t lb = ((size_t)count * sizeof(ChainLin) + 255) & ~size_t(255);
  const size_t ib = (items.size() * sizeof(int2) + 255) & ~size_t(255);
  const size_t sbb = ((size_t)(nst + 1) * sizeof(int) + 255) & ~size_t(255);
  const size_t bb = ((size_t)nst * CHAIN_STAGE + 2 * CHAIN_LINE) * sizeof(uint32_t);
  ChainPlan* p = new (std::nothrow) ChainPlan{};
  if (!p) return hipErrorOutOfMemory;
  p->dev = dev;
  p->act_f16 = act_f16;
  p->gsh = gsh;
  p->nst = nst;
  p->P = cus * std::min(per_cu, 2);  // two per CU: more loads in flight (one measured 5% slower)
  p->lds = lds;
  e = hipMalloc(&p->mem, lb + ib + sbb + bb);
  if (e != hipSuccess) {
    delete p;
    return e;
  }
  char* m = static_cast<char*>(p->mem);
  p->lins = reinterpret_cast<ChainLin*>(m);
  p->items = reinterpret_cast<int2*>(m + lb);
  p->sb = reinterpret_cast<int*>(m + lb + ib);
  p->bar = reinterpret_cast<uint32_t*>(m + lb + ib + sbb);
  e = hipMemcpy(p->lins, lins.data(), (size_t)count * sizeof(ChainLin), hipMemcpyHostToDevice);
  if (e == hipSuccess && !items.empty())
    e = hipMemcpy(p->items, items.data(), items.size() * sizeof(int2), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(p->sb, sb.data(), (size_t)(nst + 1) * sizeof(int), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemset(p->bar, 0, bb);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(p->mem);
    delete p;
    return e;
  }
  *out = p;
  return hipSuccess;
}

hipError_t chain_plan_run(void* plan, hipStream_t s) {
  ChainPlan* p = static_cast<ChainPlan*>(plan);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev != p->dev) return hipErrorInvalidDevice;
  const ChainLin* lins = p->lins;
  const int2* items = p->items;
  const int* sb = p->sb;
  int nst = p->nst, gsh = p->gsh;
  uint32_t* bar = p->bar;
  void* args[] = {&lins, &items, &sb, &nst, &gsh, &bar};
  const void* k = p->act_f16 ? reinterpret_cast<const void*>(gemv_chain_kernel<true>)
                             : reinterpret_cast<const void*>(gemv_chain_kernel<false>);
  return hipLaunchCooperativeKernel(k, dim3((unsigned)p->P), dim3(256), args, (unsigned)p->lds, s);
}

hipError_t chain_plan_status(void* plan, int* timed_out) {
  ChainPlan* p = static_cast<ChainPlan*>(plan);
  uint32_t v = 0;
  const hipError_t e = hipMemcpy(&v, p->bar + (long)p->nst * CHAIN_STAGE + CHAIN_LINE, sizeof(v), hipMemcpyDeviceToHost);
  *timed_out = v != 0;
  return e;
}

hipError_t chain_plan_free(void* plan) {
  ChainPlan* p = static_cast<ChainPlan*>(plan);
  if (!p) return hipSuccess;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess) e = hipSetDevice(p->dev);
  if (e == hipSuccess) e = hipFree(p->mem);
  (void)hipSetDevice(cur);
  delete p;
  return e;
}

}  // namespace qaff
