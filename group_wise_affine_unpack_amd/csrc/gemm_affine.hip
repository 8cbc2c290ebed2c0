// Prefill GEMM for group-wise affine weights (M > 16): y = x . W^T with
// W[n,k] = q(n,k) * scale[n, k/G] + bias[n, k/G] (mlx_int8.rs "Layout";
// Transformers "Metal" page: 2/4/8-bit codes, per-group scale and bias).
//
// Exactness.  Rounding the dequantized weight to bf16 or fp16 is not accurate
// enough for the elementwise bound (8-bit codes especially), so the kernel
// never rounds a weight.  It writes
//     q = sum_a c_a * p_a + OFF            (code pieces p_a in [-8, 7], c_a a power of 2)
//     scale * 2^-e_n = sum_j s_j            (pieces s_j with <= 8 significant bits)
//     W = 2^e_n * sum_{a,j} c_a p_a s_j + (OFF*scale + bias)
// Every c_a p_a s_j has at most 3 + 8 = 11 significant bits, so it is EXACT in
// fp16.  x is scaled per row by a power of two (2^-e_m) into fp16, exact in
// fp16's normal range.  Then
//     y[m,n] = 2^(e_m+e_n) * ( sum_k xh[m,k] * sum_{a,j} c_a p_a s_j
//                            + sum_g xs[m,g] * cb[n,g] )
// with xs the group sums of xh and cb = (OFF*scale + bias) * 2^-e_n.  The
// first sum runs on v_mfma_f32_32x32x16_f16 (one pass per (a, j) pair: 1 for
// 4-bit codes with bf16 scales, 2 for 8-bit codes or f16 scales); the second
// is a short tail of v_mfma_f32_32x32x16_bf16 over 3*K/G columns carrying
// hi/lo bf16 splits of xs and cb.  Everything accumulates in one fp32 tile.
//
// Kernels:
//   prep    : one launch, two halves.  Per row of x: e_m, xh (fp16, permuted
//             to the code decode order, read through k_perm when given), tail
//             A = [xs_hi, xs_hi, xs_lo].  Per row of W: e_n, scale pieces s_j
//             (fp16 pairs), tail B = [cb_hi, cb_lo, cb_hi]
//   gemm    : 256 threads, tile BM x 256 (4 waves along N, each BM x 64);
//             x tiles in a 4-stage LDS ring, stored two steps ahead; packed codes go from
//             global memory straight to registers, are decoded with the
//             exponent-bias trick (code | 0x6400 = 1024 + code in fp16) and
//             scaled with packed fp16 math; XCD-aware tile order.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace qaff {

hipError_t launch_gemv_affine(const AffineArgs& a, hipStream_t s);

namespace {

constexpr int BN = 256;       // tile width along N (4 waves x 64)
constexpr int BK = 64;        // codes per K tile

__device__ __forceinline__ uint32_t f32_bits(float v) { return __float_as_uint(v); }
__device__ __forceinline__ float trunc_bf16(float v) { return __uint_as_float(f32_bits(v) & 0xffff0000u); }

// Position, within its block, of the source column of permuted column j.
// It matches the order in which the kernel decodes codes from a word:
//   4-bit: (c0,c4),(c1,c5),(c2,c6),(c3,c7)            block of 8
//   8-bit: (c0,c2),(c1,c3) per word, two words          block of 8
//   2-bit: (c0,c8),(c1,c9),...,(c7,c15)                 block of 16
template <int BITS>
struct Perm {
  static constexpr int BLK = BITS == 2 ? 16 : 8;
  static __device__ __forceinline__ int src(int j) {
    if (BITS == 4) return (j >> 1) + ((j & 1) << 2);
    if (BITS == 8) return (j & 4) + (j >> 1 & 1) + ((j & 1) << 1);
    return (j >> 1) + ((j & 1) << 3);
  }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// exponent e with |v| * 2^-e in [1, 2) (0 for v == 0)
__device__ __forceinline__ int exp_of(float v) {
  if (!(v > 0.f)) return 0;
  int e;
  (void)frexpf(v, &e);
  return e - 1;
}

// ---------------------------------------------------------------------------
// prep_x: one block (256 threads) per padded row m.  Pass 1 reads the row
// with 16-byte loads for its max |x| (a permutation does not change it);
// pass 2 (an L2 hit) writes blocks of BLK permuted, scaled fp16 values.
// xh is tile-blocked: the BM x 64 block of K tile kt of row tile mt is one
// contiguous 16 KiB..32 KiB piece, row r of it at r*64 elements, so a GEMM
// step reads a single contiguous block.
template <int BITS>
__device__ __forceinline__ void prep_x_row(int m, const void* __restrict__ x, int act_dt,
                                           const int32_t* __restrict__ k_perm, int M, int K, int G, int Kt, int BM,
                                           _Float16* __restrict__ xh, uint16_t* __restrict__ tA,
                                           int* __restrict__ em) {
  constexpr int BLK = Perm<BITS>::BLK;
  const int t = threadIdx.x;
  const int ng = K / G;
  const int nkt = K / 64;
  // element (m, k) of xh sits at xrow[(k/64)*BM*64 + k%64]
  _Float16* xrow = xh + ((long)(m / BM) * nkt * BM + (m % BM)) * 64;
  const long kt_stride = (long)BM * 64;
  uint16_t* trow = tA + (long)m * Kt;
  if (m >= M) {  // padding rows of the tile grid are zero
    for (int c = t; c < K / 8; c += 256)
      reinterpret_cast<u32x4_t*>(xrow + (c >> 3) * kt_stride)[c & 7] = u32x4_t{0, 0, 0, 0};
    for (int k = t; k < Kt; k += 256) trow[k] = 0;
    if (t == 0) em[m] = 0;
    return;
  }
  const bool f16 = act_dt == F16;
  const uint16_t* xr = static_cast<const uint16_t*>(x) + (long)m * K;
  __shared__ float red[4];
  float amax = 0.f;
  for (int c = t; c < K / 8; c += 256) {
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(xr)[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = f16 ? f16_bits_to_f32(v[i] & 0xffffu) : bf16_bits_to_f32(v[i] & 0xffffu);
      const float hi = f16 ? f16_bits_to_f32(v[i] >> 16) : bf16_bits_to_f32(v[i] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
    }
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = exp_of(amax);
  if (t == 0) em[m] = e;
  const float sc = ldexpf(1.f, -e);

  // blocks of BLK permuted columns; the lanes that share a group are
  // consecutive and aligned, so the group sum is a butterfly over them
  const int nblk = K / BLK;
  const int bpg = G / BLK;  // blocks per group: 2..16, a power of two
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int bi = b0 + t;
    float part = 0.f;
    if (bi < nblk) {
      float src[BLK];
      if (k_perm == nullptr) {
#pragma unroll
        for (int q = 0; q < BLK / 8; ++q) {
          const u32x4_t v = reinterpret_cast<const u32x4_t*>(xr + bi * BLK)[q];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            src[8 * q + 2 * i] = f16 ? f16_bits_to_f32(v[i] & 0xffffu) : bf16_bits_to_f32(v[i] & 0xffffu);
            src[8 * q + 2 * i + 1] = f16 ? f16_bits_to_f32(v[i] >> 16) : bf16_bits_to_f32(v[i] >> 16);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < BLK; ++j) {
          const uint32_t h = xr[k_perm[bi * BLK + j]];
          src[j] = f16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
        }
      }
      _Float16 out[BLK];
#pragma unroll
      for (int j = 0; j < BLK; ++j) {
        const float v = src[Perm<BITS>::src(j)] * sc;
        out[j] = (_Float16)v;
        part += v;
      }
#pragma unroll
      for (int j = 0; j < BLK; j += 8) {
        const int k = bi * BLK + j;
        *reinterpret_cast<f16x8_t*>(xrow + (k >> 6) * kt_stride + (k & 63)) =
            f16x8_t{out[j], out[j + 1], out[j + 2], out[j + 3], out[j + 4], out[j + 5], out[j + 6], out[j + 7]};
      }
    }
    for (int o = 1; o < bpg; o <<= 1) part += __shfl_xor(part, o);
    if (bi < nblk && (bi % bpg) == 0) {
      const int g = bi / bpg;
      const uint16_t hi = f32_to_bf16_bits(part);
      const uint16_t lo = f32_to_bf16_bits(part - bf16_bits_to_f32(hi));
      trow[3 * g] = hi;
      trow[3 * g + 1] = hi;
      trow[3 * g + 2] = lo;
    }
  }
  for (int k = 3 * ng + t; k < Kt; k += 256) trow[k] = 0;
}

// ---------------------------------------------------------------------------
// prep_w: one wave per padded row n.  PS = number of scale pieces; each is
// stored twice, as an fp16 pair (s, s), ready to multiply packed code pairs.
template <int PS>
__device__ __forceinline__ void prep_w_rows(int blk, const void* __restrict__ scales, int s_dt,
                                            const void* __restrict__ biases, int b_dt, float off, int N, int ng,
                                            int Kt, f16x2_t* __restrict__ sh, uint16_t* __restrict__ tB,
                                            int* __restrict__ en) {
  const int n = blk * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  f16x2_t* srow = sh + (long)n * ng * PS;
  uint16_t* trow = tB + (long)n * Kt;
  if (n >= N) {
    for (int i = lane; i < ng * PS; i += 64) srow[i] = f16x2_t{(_Float16)0.f, (_Float16)0.f};
    for (int k = lane; k < Kt; k += 64) trow[k] = 0;
    if (lane == 0) en[n] = 0;
    return;
  }
  const long base = (long)n * ng;
  float smax = 0.f;
  for (int g = lane; g < ng; g += 64) smax = fmaxf(smax, fabsf(load_as_f32(scales, base + g, s_dt)));
  smax = wave_max(smax);
  const int e = exp_of(smax);
  if (lane == 0) en[n] = e;
  const float sc = ldexpf(1.f, -e);
  for (int g = lane; g < ng; g += 64) {
    const float s = load_as_f32(scales, base + g, s_dt);
    const float b = load_as_f32(biases, base + g, b_dt);
    float r = s * sc;  // exact: a power-of-two scaling
#pragma unroll
    for (int j = 0; j < PS; ++j) {
      const float p = (j == PS - 1) ? r : trunc_bf16(r);
      srow[g * PS + j] = f16x2_t{(_Float16)p, (_Float16)p};
      r -= p;
    }
    const float cb = fmaf(off, s, b) * sc;
    const uint16_t hi = f32_to_bf16_bits(cb);
    const uint16_t lo = f32_to_bf16_bits(cb - bf16_bits_to_f32(hi));
    trow[3 * g] = hi;
    trow[3 * g + 1] = lo;
    trow[3 * g + 2] = hi;
  }
  for (int k = 3 * ng + lane; k < Kt; k += 64) trow[k] = 0;
}

// prep_x and prep_w in one launch: blocks [0, Mp) take the rows of x, the
// rest take four rows of W each; the two halves run side by side.
struct PrepArgs {
  const void* x;
  const int32_t* k_perm;
  const void* scales;
  const void* biases;
  _Float16* xh;
  uint16_t* tA;
  int* em;
  f16x2_t* sh;
  uint16_t* tB;
  int* en;
  float off;
  int act_dt, s_dt, b_dt;
  int M, N, K, G, Kt, BM, Mp, ng;
};

template <int BITS, int PS>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  const int b = blockIdx.x;
  if (b < a.Mp)
    prep_x_row<BITS>(b, a.x, a.act_dt, a.k_perm, a.M, a.K, a.G, a.Kt, a.BM, a.xh, a.tA, a.em);
  else
    prep_w_rows<PS>(b - a.Mp, a.scales, a.s_dt, a.biases, a.b_dt, a.off, a.N, a.ng, a.Kt, a.sh, a.tB, a.en);
}

// ---------------------------------------------------------------------------
// main GEMM

struct GemmParams {
  const _Float16* xh;
  const uint16_t* tA;
  const int* em;
  const uint32_t* w;
  const f16x2_t* sh;
  const uint16_t* tB;
  const int* en;
  uint16_t* y;
  int M, N, K, ng, Kt, G;
  int Np, gsh;  // padded row count of the W-side scratch; log2(G) - 5
  int Tm, Tn, per_xcd;
  int out_f16;
  int S;        // K splits; S > 1 writes fp32 partials [S][M][N] to `part`
  float* part;
};

__device__ __forceinline__ f16x2_t h2(uint32_t v) { return __builtin_bit_cast(f16x2_t, v); }

// B fragment (8 fp16 = 4 dwords) for one 32x32x16 step, one code piece, one
// scale piece.  `wd` holds the lane's words for this step (1 for 4-bit, 2 for
// 8-bit, 1 (half used) for 2-bit).
template <int BITS>
struct Decode {
  // integer pieces as exact fp16 pairs, in the kernel's decode order
  static constexpr int NPIECE = BITS == 8 ? 2 : 1;
  static constexpr float OFFQ = BITS == 4 ? 8.f : (BITS == 8 ? 136.f : 0.f);
  // `magic` holds 0x64006400 in a VGPR, so mask-and-insert is one
  // v_and_or_b32 (a VOP3 op reads at most one literal or SGPR on gfx950)
  static __device__ __forceinline__ void pieces(const uint32_t* wd, int half, uint32_t magic,
                                                f16x2_t (&v)[NPIECE][4]) {
    const f16x2_t k1032 = {(_Float16)-1032.f, (_Float16)-1032.f};
    const f16x2_t k1024 = {(_Float16)-1024.f, (_Float16)-1024.f};
    if constexpr (BITS == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[0][i] = h2(((wd[0] >> (4 * i)) & 0x000F000Fu) | magic) + k1032;
    } else if constexpr (BITS == 8) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        v[0][2 * w] = h2(((wd[w] >> 4) & 0x000F000Fu) | magic) + k1032;       // hi nibbles (c0,c2)
        v[0][2 * w + 1] = h2(((wd[w] >> 12) & 0x000F000Fu) | magic) + k1032;  // (c1,c3)
        v[1][2 * w] = h2((wd[w] & 0x000F000Fu) | magic) + k1032;              // lo nibbles
        v[1][2 * w + 1] = h2(((wd[w] >> 8) & 0x000F000Fu) | magic) + k1032;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[0][i] = h2(((wd[0] >> (2 * (i + 4 * half))) & 0x00030003u) | magic) + k1024;
    }
  }
  // multiplier of piece a
  static constexpr float piece_mult(int a) { return (BITS == 8 && a == 0) ? 16.f : 1.f; }
};

// Main GEMM.  256 threads = 4 waves, one per SIMD, side by side along N:
// wave w computes rows [0, BM) x columns [64w, 64w+64) of the BM x 256 tile,
// so every weight word is decoded once per BM rows.
//
// Pipeline:
//   * x tiles go global -> registers (one step before the store) -> LDS,
//     stored two steps before use into a 4-stage ring; 16-byte chunks are
//     XOR-swizzled by row ((r ^ r>>1) & 7) so the MFMA operand reads are
//     bank-conflict free;
//   * weight words and scale pieces go through buffer loads with the K
//     offset in an SGPR, into a 4-deep register ring (three steps ahead);
//   * the A reads and the B decode of a tile's first 16-column step run
//     during the previous tile's last step, so a tile starts with MFMAs
//     (the tile's x is in LDS for every wave one barrier earlier);
//   * the loop is unrolled by 4 so every ring index and LDS stage is a
//     constant.
// Rows of W past N are read through per-lane offsets past the buffer's range
// and come back as zeros, so the last row tile needs no clamping.

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 1)) & 7; }

template <int BITS, int PS, int MB>
struct Stage {
  static constexpr int WPL = BITS;  // words per lane per K tile
  uint32_t w[2][WPL];
  uint32_t s[2][PS];  // scale pieces as fp16 pairs (s, s)
};

template <int BITS, int PS, int MB>
struct Pipe {
  using D = Decode<BITS>;
  using St = Stage<BITS, PS, MB>;
  static constexpr int WPL = BITS;
  static constexpr int WPR = 2 * BITS;
  static constexpr int A_DMA = MB;

  __amdgpu_buffer_rsrc_t rw, rs, rx;
  uint32_t w_off[2], s_off[2], x_off;
  int half, l32, gsh;
  int kbase;       // first K tile of this workgroup's split
  int last_kt;     // index of the last K tile, relative to kbase
  int a_dst;       // this thread's first LDS chunk in a stage

  // Loads for K tile kt: the x chunks (into registers; written to LDS one
  // step later), then the weight words and scale pieces (into a ring entry
  // used two steps later).
  // A prefetch past the last tile re-reads the last tile: every address stays
  // inside its buffer, whatever the hardware does with soffset in its range
  // check; the data is never used.
  __device__ __forceinline__ void issue_x(int kt, u32x4_t (&xr)[A_DMA]) const {
    kt = kbase + min(kt, last_kt);
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
      xr[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, x_off, kt * (MB * 32 * 128) + i * 4096, 0));
  }
  __device__ __forceinline__ void issue_w(int kt, St& st) const {
    kt = kbase + min(kt, last_kt);
    // group of this tile: (2*kt + half) >> gsh, whose lane part (half, for
    // G = 32 only) is folded into s_off; the rest is uniform
    const int sg = ((2 * kt) >> gsh) * PS * 4;
    const int so = kt * WPR * 4;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if constexpr (WPL == 2) {
        const u32x2_t u = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, w_off[nb], so, 0));
        st.w[nb][0] = u.x;
        st.w[nb][1] = u.y;
      } else {
#pragma unroll
        for (int q = 0; q < WPL / 4; ++q) {
          const u32x4_t u = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, w_off[nb] + q * 16, so, 0));
          st.w[nb][4 * q] = u.x;
          st.w[nb][4 * q + 1] = u.y;
          st.w[nb][4 * q + 2] = u.z;
          st.w[nb][4 * q + 3] = u.w;
        }
      }
#pragma unroll
      for (int j = 0; j < PS; ++j) st.s[nb][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, s_off[nb] + j * 4, sg, 0);
    }
  }

  // x chunk i of this thread lands at LDS byte a_dst + i*4096 of a stage:
  // row 32i + t/8, position t%8 (already swizzled on the global side)
  __device__ __forceinline__ void store_x(unsigned char* sA, const u32x4_t (&xr)[A_DMA]) const {
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) *reinterpret_cast<u32x4_t*>(sA + a_dst + i * 4096) = xr[i];
  }

  __device__ __forceinline__ void read_a(const unsigned char* __restrict__ sA, int s, f16x8_t (&af)[MB]) const {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = mb * 32 + l32;
      af[mb] = *reinterpret_cast<const f16x8_t*>(sA + r * 128 + (((4 * half + s) ^ swz(r)) << 4));
    }
  }

  // B fragments of the 16-column step s for both n blocks: one per (code
  // piece, scale piece)
  static constexpr int NF = D::NPIECE * PS;
  __device__ __forceinline__ void decode_b(const St& st, int s, uint32_t magic, f16x8_t (&bf)[2][NF]) const {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      uint32_t wd[2];
      if constexpr (BITS == 4) {
        wd[0] = st.w[nb][s];
      } else if constexpr (BITS == 8) {
        wd[0] = st.w[nb][2 * s];
        wd[1] = st.w[nb][2 * s + 1];
      } else {
        wd[0] = st.w[nb][s >> 1];
      }
      f16x2_t vv[D::NPIECE][4];
      D::pieces(wd, s & 1, magic, vv);
#pragma unroll
      for (int a = 0; a < D::NPIECE; ++a)
#pragma unroll
        for (int j = 0; j < PS; ++j) {
          f16x2_t sj = h2(st.s[nb][j]);  // (s, s)
          if (D::piece_mult(a) != 1.f) sj = sj * f16x2_t{(_Float16)16.f, (_Float16)16.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f16x2_t q = vv[a][i] * sj;
            bf[nb][a * PS + j][2 * i] = q[0];
            bf[nb][a * PS + j][2 * i + 1] = q[1];
          }
        }
    }
  }

  __device__ __forceinline__ void mfma_b(const f16x8_t (&af)[MB], const f16x8_t (&bf)[2][NF],
                                         f32x16_t (&acc)[MB][2]) const {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mb], bf[nb][f], acc[mb][nb], 0, 0, 0);
  }

  // Scheduling of one step: its MFMAs with the next step's decode (VALU)
  // and the A reads two steps ahead (DS) spread between them, so VALU and
  // LDS work co-issue with the matrix pipe instead of following it.
  static constexpr int N_MFMA = 2 * NF * MB;
  template <int NVALU, int NDS>
  static __device__ __forceinline__ void interleave() {
    constexpr int per = (NVALU + N_MFMA - 1) / N_MFMA;
#pragma unroll
    for (int i = 0; i < N_MFMA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (per > 0) __builtin_amdgcn_sched_group_barrier(0x002, per, 0);  // VALU
      if (i < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
    }
  }

  // The four 16-column steps of a tile, software-pipelined: step s runs its
  // MFMAs while step s+1's B fragments are decoded and its A fragments are
  // read from LDS.  a0/b0 hold step 0 of this tile on entry, and step 0 of
  // the next tile (stage sAn, ring entry stn) on exit.
  __device__ __forceinline__ void compute(const St& st, const unsigned char* __restrict__ sA, const St& stn,
                                          const unsigned char* __restrict__ sAn, uint32_t magic,
                                          f16x8_t (&a0)[MB], f16x8_t (&b0)[2][NF], f32x16_t (&acc)[MB][2]) const {
    constexpr int DEC = 2 * NF * 16;  // VALU ops of one step's decode, roughly
    f16x8_t a1[MB];
    f16x8_t b1[2][NF];
    read_a(sA, 1, a1);
    decode_b(st, 1, magic, b1);
    mfma_b(a0, b0, acc);
    interleave<DEC, MB>();
    __builtin_amdgcn_sched_barrier(0);
    read_a(sA, 2, a0);
    decode_b(st, 2, magic, b0);
    mfma_b(a1, b1, acc);
    interleave<DEC, MB>();
    __builtin_amdgcn_sched_barrier(0);
    read_a(sA, 3, a1);
    decode_b(st, 3, magic, b1);
    mfma_b(a0, b0, acc);
    interleave<DEC, MB>();
    __builtin_amdgcn_sched_barrier(0);
    read_a(sAn, 0, a0);
    decode_b(stn, 0, magic, b0);
    mfma_b(a1, b1, acc);
    interleave<DEC, MB>();
    __builtin_amdgcn_sched_barrier(0);
  }

  // One K tile kt (stage kt%4, ring entry kt%4):
  //   barrier                 tile kt+1's x (stored last step) visible to all
  //                           waves; everyone done with tile kt-1
  //   store x of tile kt+2    registers loaded last step -> stage (kt+2)%4
  //   issue tile kt+3         x into registers, weights/scales into the ring
  //   compute tile kt         ending with step 0 of tile kt+1 prepared
  // Loads past the last tile re-read the last tile and land nowhere that is
  // read, so the step has no branch.  S = kt % 4, a compile-time constant,
  // so the LDS stage offsets are immediates.
  template <int S>
  __device__ __forceinline__ void step(int kt, const St& cur, const St& nxt, St& fut, unsigned char* lds,
                                       u32x4_t (&xr)[A_DMA], uint32_t magic, f16x8_t (&a0)[MB], f16x8_t (&b0)[2][NF],
                                       f32x16_t (&acc)[MB][2]) const {
    constexpr int SB = MB * 32 * 128;  // bytes of one stage
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0): own LDS writes done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    store_x(lds + ((S + 2) & 3) * SB, xr);
    issue_x(kt + 3, xr);   // x three tiles ahead (L2), stored next step
    issue_w(kt + 3, fut);  // weights three tiles ahead (HBM)
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
    compute(cur, lds + S * SB, nxt, lds + ((S + 1) & 3) * SB, magic, a0, b0, acc);
  }
};

template <int BITS, int PS, int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_affine_kernel(GemmParams p) {
  using St = Stage<BITS, PS, MB>;
  constexpr int BM = MB * 32;
  constexpr int WPL = BITS;
  constexpr int STAGE_BYTES = BM * 128; // one x tile, 64 fp16 per row, no padding

  const int b = blockIdx.x;
  const int vs = (b & 7) * p.per_xcd + (b >> 3);
  if (vs >= p.Tm * p.Tn * p.S) return;
  const int v = vs / p.S, sp = vs % p.S;
  const int tm = v / p.Tn, tn = v % p.Tn;
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l32 = lane & 31, half = lane >> 5;
  // K tiles [kt0, kt1) of split sp
  const int nkt_all = p.K / BK, per_split = (nkt_all + p.S - 1) / p.S;
  const int kt0 = sp * per_split, kt1 = min(nkt_all, kt0 + per_split);

  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) int em_s[BM];
  for (int i = t; i < BM; i += 256) em_s[i] = p.em[m0 + i];

  f32x16_t acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // ---- buffer resources and per-lane offsets
  Pipe<BITS, PS, MB> P;
  const uint32_t row_bytes = (uint32_t)p.K * BITS / 8;
  P.rw = make_rsrc(p.w, (uint32_t)p.N * row_bytes);
  P.rs = make_rsrc(p.sh, (uint32_t)p.Np * p.ng * PS * 4);
  P.rx = make_rsrc(p.xh + (long)m0 * p.K, (uint32_t)BM * p.K * 2);  // this row tile's blocks
  P.half = half;
  P.l32 = l32;
  P.gsh = p.gsh;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const uint32_t n = n0 + wave * 64 + nb * 32 + l32;
    P.w_off[nb] = n * row_bytes + half * WPL * 4;
    P.s_off[nb] = (n * (uint32_t)p.ng + (p.gsh == 0 ? half : 0)) * PS * 4;
  }
  // x tile chunks: thread t moves chunks q = i*256 + t, i.e. row 32i + t/8,
  // LDS position t%8, which holds source chunk (t%8)^swz(row); swz(32i + t/8)
  // does not depend on i.
  {
    const int r = t >> 3, pos = t & 7;
    P.x_off = (uint32_t)r * 128 + ((pos ^ swz(r)) << 4);  // inside the contiguous BM x 64 block
    P.a_dst = t * 16;
  }

  const int nkt = kt1 - kt0;
  P.kbase = kt0;
  P.last_kt = nkt - 1;
  St st0, st1, st2, st3;
  u32x4_t xr[MB];
  // prologue: x of tiles 0 and 1 in LDS, tile 2 in registers, weights of
  // tiles 0..2 in the ring, step 0 of tile 0 prepared
  P.issue_x(0, xr);
  P.issue_w(0, st0);
  P.issue_w(1, st1);
  P.issue_w(2, st2);
  P.store_x(lds, xr);
  P.issue_x(1, xr);
  P.store_x(lds + STAGE_BYTES, xr);
  P.issue_x(2, xr);
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();

  // ---- main loop
  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));
  f16x8_t a0[MB];
  f16x8_t b0[2][Pipe<BITS, PS, MB>::NF];
  P.read_a(lds, 0, a0);
  P.decode_b(st0, 0, magic, b0);
  // unrolled by 4 = the ring size and the stage count: every index is static
  for (int kt = 0; kt < nkt; kt += 4) {
    P.template step<0>(kt, st0, st1, st3, lds, xr, magic, a0, b0, acc);
    if (kt + 1 < nkt) P.template step<1>(kt + 1, st1, st2, st0, lds, xr, magic, a0, b0, acc);
    if (kt + 2 < nkt) P.template step<2>(kt + 2, st2, st3, st1, lds, xr, magic, a0, b0, acc);
    if (kt + 3 < nkt) P.template step<3>(kt + 3, st3, st0, st2, lds, xr, magic, a0, b0, acc);
  }

  // ---- tail: sum_g xs * cb on bf16 MFMA, operands straight from global
  // (L2-resident), in the first split only.  It runs after the main loop so
  // that its loads do not blur the compiler's count of outstanding loads at
  // the loop header.
  if (sp == 0) {
    const uint16_t* tb_row[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) tb_row[nb] = p.tB + (long)(n0 + wave * 64 + nb * 32 + l32) * p.Kt + 8 * half;
    const uint16_t* ta_row = p.tA + (long)(m0 + l32) * p.Kt + 8 * half;
    const long ta_mb = (long)32 * p.Kt;
    for (int kt = 0; kt < p.Kt; kt += 16) {
      bf16x8_t bt[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bt[nb] = *reinterpret_cast<const bf16x8_t*>(tb_row[nb] + kt);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8_t at = *reinterpret_cast<const bf16x8_t*>(ta_row + mb * ta_mb + kt);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at, bt[nb], acc[mb][nb], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: y = 2^(e_m + e_n) * acc, rounded to the activation dtype.
  // 32x32 accumulator layout: lane -> column l32; register r -> row
  // 8*(r/4) + 4*half + r%4.  Stores go through a buffer resource over y: a
  // column past N starts from an out-of-range offset and a row past M lands
  // past the range, so neither is written.
  if (p.S > 1) {
    // fp32 partial of split sp, scaled (exact: a power of two); rows past M
    // land past the range, columns past N start from an out-of-range offset
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(p.part + (long)sp * p.M * p.N, (uint32_t)p.M * p.N * 4);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = n0 + wave * 64 + nb * 32 + l32;
      const bool nok = n < p.N;
      const int e_n = nok ? p.en[n] : 0;
      const uint32_t vb = nok ? ((uint32_t)(m0 + 4 * half) * p.N + n) * 4u : 0x80000000u;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const i32x4_t e4 = *reinterpret_cast<const i32x4_t*>(&em_s[mb * 32 + 8 * rq + 4 * half]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ldexpf(acc[mb][nb][4 * rq + j], e4[j] + e_n)), rp,
                                                  vb + (uint32_t)((mb * 32 + 8 * rq + j) * p.N) * 4u, 0, 0);
        }
    }
    return;
  }
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y, (uint32_t)p.M * p.N * 2);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = n0 + wave * 64 + nb * 32 + l32;
    const bool nok = n < p.N;
    const int e_n = nok ? p.en[n] : 0;
    const uint32_t vb = nok ? ((uint32_t)(m0 + 4 * half) * p.N + n) * 2u : 0x80000000u;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const i32x4_t e4 = *reinterpret_cast<const i32x4_t*>(&em_s[mb * 32 + 8 * rq + 4 * half]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float val = ldexpf(acc[mb][nb][4 * rq + j], e4[j] + e_n);
          const uint16_t h = p.out_f16 ? f32_to_f16_bits(val) : f32_to_bf16_bits(val);
          __builtin_amdgcn_raw_buffer_store_b16(h, ry, vb + (uint32_t)((mb * 32 + 8 * rq + j) * p.N) * 2u, 0, 0);
        }
      }
  }
}

// ---------------------------------------------------------------------------

// y = the sum of the S fp32 partials, rounded to the activation type
__global__ __launch_bounds__(256) void gemm_split_sum_kernel(const float* __restrict__ part, uint16_t* __restrict__ y,
                                                             long MN, int S, int out_f16) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[(long)s * MN + i];
  y[i] = out_f16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

template <int BITS, int PS>
hipError_t run(const AffineArgs& a, hipStream_t s) {
  // buffer resources address W, the scale pieces and one x tile with 32-bit offsets
  if (a.N * a.K * BITS / 8 >= (int64_t(1) << 31) || a.K * 2 * 256 >= (int64_t(1) << 31))
    return hipErrorNotSupported;
  const int M = (int)a.M, N = (int)a.N, K = (int)a.K, G = a.G;
  const int ng = K / G;
  const int Kt = (3 * ng + 15) / 16 * 16;
  // the largest row tile whose grid still fills three quarters of the CUs
  // in one round: a bigger tile's efficiency is worth a few idle CUs, and a
  // grid just past one round runs its last tiles as a second round alone
  int MB = 2;
  if (M > 64) {
    const int64_t tn = (N + BN - 1) / BN;
    if ((int64_t)((M + 255) / 256) * tn >= 192) MB = 8;
    else if ((int64_t)((M + 127) / 128) * tn >= 192) MB = 4;
  }
  const int BM = MB * 32;
  const int Mp = (M + BM - 1) / BM * BM, Np = (N + BN - 1) / BN * BN;
  // The epilogue stores padded rows m in [M, Mp) too, relying on their
  // offsets (m*N + n)*2 (y) or *4 (fp32 partials) landing past the buffer's
  // range; they must not wrap around 2^32, so every padded offset stays
  // below 2^31.
  if ((int64_t)Mp * N * 2 >= (int64_t(1) << 31)) return hipErrorNotSupported;
  // K splits when the tiles leave CUs idle: as many as keep the grid in one
  // round of workgroups, each split at least 4 K tiles, partials within
  // 32-bit buffer offsets
  const int64_t tiles = (int64_t)(Mp / BM) * (Np / BN);
  int S = 1;
  if (tiles < 256) {
    S = (int)std::min<int64_t>(std::max<int64_t>(1, 256 / tiles), std::max(1, K / BK / 4));
    if ((int64_t)Mp * N * 4 >= (int64_t(1) << 31)) S = 1;  // partial offsets as above
    const int per = (K / BK + S - 1) / S;
    S = (K / BK + per - 1) / per;  // no empty split
  }

  const size_t o_xh = 0, s_xh = align256((size_t)Mp * K * 2);
  const size_t o_ta = o_xh + s_xh, s_ta = align256((size_t)Mp * Kt * 2);
  const size_t o_em = o_ta + s_ta, s_em = align256((size_t)Mp * 4);
  const size_t o_sh = o_em + s_em, s_sh = align256((size_t)Np * ng * PS * 4);
  const size_t o_tb = o_sh + s_sh, s_tb = align256((size_t)Np * Kt * 2);
  const size_t o_en = o_tb + s_tb, s_en = align256((size_t)Np * 4);
  const size_t o_pt = o_en + s_en, s_pt = S > 1 ? align256((size_t)S * M * N * 4) : 0;
  const size_t total = o_pt + s_pt;

  char* scratch = nullptr;
  hipError_t e = stream_workspace(s, total, (void**)&scratch);
  if (e != hipSuccess) return e;

  _Float16* xh = (_Float16*)(scratch + o_xh);
  uint16_t* tA = (uint16_t*)(scratch + o_ta);
  int* em = (int*)(scratch + o_em);
  f16x2_t* sh = (f16x2_t*)(scratch + o_sh);
  uint16_t* tB = (uint16_t*)(scratch + o_tb);
  int* en = (int*)(scratch + o_en);

  PrepArgs pa;
  pa.x = a.x;
  pa.k_perm = a.k_perm;
  pa.scales = a.scales;
  pa.biases = a.biases;
  pa.xh = xh;
  pa.tA = tA;
  pa.em = em;
  pa.sh = sh;
  pa.tB = tB;
  pa.en = en;
  pa.off = Decode<BITS>::OFFQ;
  pa.act_dt = a.act_dt;
  pa.s_dt = a.s_dt;
  pa.b_dt = a.b_dt;
  pa.M = M;
  pa.N = N;
  pa.K = K;
  pa.G = G;
  pa.Kt = Kt;
  pa.BM = BM;
  pa.Mp = Mp;
  pa.ng = ng;
  hipLaunchKernelGGL((prep_kernel<BITS, PS>), dim3(Mp + Np / 4), dim3(256), 0, s, pa);

  GemmParams p;
  p.xh = xh;
  p.tA = tA;
  p.em = em;
  p.w = a.w;
  p.sh = sh;
  p.tB = tB;
  p.en = en;
  p.y = (uint16_t*)a.y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.ng = ng;
  p.Kt = Kt;
  p.G = G;
  p.Np = Np;
  p.gsh = G == 32 ? 0 : (G == 64 ? 1 : 2);
  p.Tm = Mp / BM;
  p.Tn = Np / BN;
  p.per_xcd = (p.Tm * p.Tn + 7) / 8;
  p.out_f16 = a.act_dt == F16;
  p.S = S;
  p.part = S > 1 ? (float*)(scratch + o_pt) : nullptr;
  p.per_xcd = (p.Tm * p.Tn * S + 7) / 8;
  const dim3 grid(8 * p.per_xcd);
  if (MB == 2)
    hipLaunchKernelGGL((gemm_affine_kernel<BITS, PS, 2>), grid, dim3(256), 0, s, p);
  else if (MB == 4)
    hipLaunchKernelGGL((gemm_affine_kernel<BITS, PS, 4>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_affine_kernel<BITS, PS, 8>), grid, dim3(256), 0, s, p);
  e = hipGetLastError();
  if (e == hipSuccess && S > 1) {
    const long MN = (long)M * N;
    hipLaunchKernelGGL(gemm_split_sum_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, p.part,
                       (uint16_t*)a.y, MN, S, p.out_f16);
    e = hipGetLastError();
  }
  return e;
}

template <int BITS>
hipError_t run_bits(const AffineArgs& a, hipStream_t s) {
  switch (a.s_dt) {
    case BF16: return run<BITS, 1>(a, s);
    case F16: return run<BITS, 2>(a, s);
    default: return run<BITS, 3>(a, s);
  }
}

}  // namespace

namespace {

// The GEMV on slices of 16 x rows, each slice reading W once more.
hipError_t rows_via_gemv(const AffineArgs& a, hipStream_t s) {
  const size_t esz = 2;  // bf16 / f16 activations and outputs
  for (int64_t m0 = 0; m0 < a.M; m0 += 16) {
    AffineArgs b = a;
    b.M = a.M - m0 < 16 ? a.M - m0 : 16;
    b.x = static_cast<const char*>(a.x) + m0 * a.K * esz;
    b.y = static_cast<char*>(a.y) + m0 * a.N * esz;
    const hipError_t e = launch_gemv_affine(b, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Whether a 16-row slice takes the MFMA GEMV (the conditions it checks:
// 4-bit codes, scales and biases in the activation dtype, whole 512-code
// stages, scale rows a multiple of 16 bytes, 16-byte aligned tensors).
bool gemv_mfma_eligible(const AffineArgs& a) {
  return a.bits == 4 && a.s_dt == a.act_dt && a.b_dt == a.act_dt && (a.G == 32 || a.G == 64 || a.G == 128) &&
         a.K % 512 == 0 && (a.K / a.G) % 8 == 0 && a.K * 32 < (int64_t(1) << 31) &&
         (((uintptr_t)a.w | (uintptr_t)a.scales | (uintptr_t)a.biases) & 15) == 0;
}

}  // namespace

hipError_t launch_gemm_affine(const AffineArgs& a, hipStream_t s) {
  // whole 64-code K tiles only; otherwise the GEMV kernel runs on slices of
  // 16 x rows (a rare shape, not a fast path)
  if (a.K % BK != 0) return rows_via_gemv(a, s);
  // Up to 48 x rows, 16-row slices on the 4-bit MFMA GEMV (W read once per
  // slice, the later times mostly from the last-level cache) beat this
  // kernel, whose 64-row tiles are a quarter or more padding there: M = 32,
  // N = 11008, K = 4096 takes 21 us instead of 33, M = 17 17 instead of 32,
  // M = 48 31 instead of 34; at M = 64 the GEMM is ahead (35 against 42).
  if (a.M <= 48 && gemv_mfma_eligible(a)) return rows_via_gemv(a, s);
  switch (a.bits) {
    case 2: return run_bits<2>(a, s);
    case 4: return run_bits<4>(a, s);
    default: return run_bits<8>(a, s);
  }
}

}  // namespace qaff
