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
// with xs the group sums of xh and cb = (OFF*scale + bias) * 2^-e_n.  (At
// 4-bit every B value carries an extra factor 16, a free by-product of the
// decode; the tail entries carry it too and e_n is 4 lower.)  The
// first sum runs on v_mfma_f32_32x32x16_f16 (one pass per (a, j) pair: 1 for
// 4-bit codes with bf16 scales, 2 for 8-bit codes or f16 scales); the second
// is a short tail of v_mfma_f32_32x32x16_bf16 over 3*K/G columns carrying
// hi/lo bf16 splits of xs and cb.  Everything accumulates in one fp32 tile.
//
// Kernels:
//   prep    : one launch, two halves.  Per row of x: e_m, xh (fp16, permuted
//             to the code decode order, read through k_perm when given), tail
//             A = [xs_hi, xs_hi, xs_lo].  Per row of W: e_n, scale pieces s_j
//             (fp16 pairs), tail B = [cb_hi, cb_lo, cb_hi].  Tail operands
//             are stored in MFMA fragment order.
//   gemm    : 512 threads (8 waves, 2 along M x 4 along N), tile BM x 256.
//             The bias tail runs first.  Then per 64-code K tile: x, code
//             and scale-piece copies go global -> LDS directly into a 3-stage
//             ring two tiles ahead; the codes are decoded with the
//             exponent-bias trick (code | 0x6400 = 1024 + code in fp16) and
//             scaled with packed fp16 math between the MFMAs; the barrier
//             for the next tile sits before the last 16-code step, whose
//             MFMAs cover the next tile's first reads.  XCD-aware tile order.
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
// Tail operands (rows x Kt bf16) are stored in the order the GEMM's MFMA
// fragments read them: 32-row x 16-column blocks, row block major, 512
// elements each, element (r, k) of a block at ((k/8)%2)*256 + (r%32)*8 + k%8.
// One 16-byte load per lane (lane = r%32 + 32*((k/8)%2)) then reads a whole
// block as 1 KiB of consecutive bytes.
__device__ __forceinline__ long tail_idx(int r, int k, int Kt) {
  return ((long)(r >> 5) * (Kt >> 4) + (k >> 4)) * 512 + ((k >> 3) & 1) * 256 + (r & 31) * 8 + (k & 7);
}

// RC > 0: the row is read once, into registers (RC 16-byte chunks a
// thread: blocks t + 256 i of BLK columns, i < RC / CPB, all loads in flight
// at once), and both passes work from there.  The host takes it when the row
// fits and no k_perm is given; RC = 0 reads the row twice, one loop trip at
// a time.
template <int BITS, int RC>
__device__ __forceinline__ void prep_x_row(int m, const void* __restrict__ x, int act_dt,
                                           const int32_t* __restrict__ k_perm, int M, int K, int G, int Kt, int BM,
                                           _Float16* __restrict__ xh, uint16_t* __restrict__ tA,
                                           int* __restrict__ em) {
  constexpr int BLK = Perm<BITS>::BLK;
  constexpr int CPB = BLK / 8;                              // 16-byte chunks per block
  constexpr int RB = RC > 0 ? (RC + CPB - 1) / CPB : 1;    // blocks a thread holds
  const int t = threadIdx.x;
  const int ng = K / G;
  const int nkt = K / 64;
  // element (m, k) of xh sits at xrow[(k/64)*BM*64 + k%64]
  _Float16* xrow = xh + ((long)(m / BM) * nkt * BM + (m % BM)) * 64;
  const long kt_stride = (long)BM * 64;
  if (m >= M) {  // padding rows of the tile grid are zero
    for (int c = t; c < K / 8; c += 256)
      reinterpret_cast<u32x4_t*>(xrow + (c >> 3) * kt_stride)[c & 7] = u32x4_t{0, 0, 0, 0};
    for (int k = t; k < Kt; k += 256) tA[tail_idx(m, k, Kt)] = 0;
    if (t == 0) em[m] = 0;
    return;
  }
  const bool f16 = act_dt == F16;
  const uint16_t* xr = static_cast<const uint16_t*>(x) + (long)m * K;
  const int nblk = K / BLK;
  auto to_f32 = [&](uint32_t h) { return f16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h); };
  auto chunk_max = [&](const u32x4_t& v, float a) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a = fmaxf(a, fmaxf(fabsf(to_f32(v[i] & 0xffffu)), fabsf(to_f32(v[i] >> 16))));
    return a;
  };
  __shared__ float red[4];
  float amax = 0.f;
  u32x4_t xc[RB][CPB];
  if constexpr (RC > 0) {
    // a block past the row reads zeros (offset past the buffer's range)
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(xr, (uint32_t)K * 2);
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int q = 0; q < CPB; ++q) {
        const int bi = t + 256 * i;
        const uint32_t off = bi < nblk ? (uint32_t)(bi * BLK + 8 * q) * 2u : 0x80000000u;
        xc[i][q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, 0));
      }
    // max |x| on the raw bits: for bf16 and f16 alike, |x| orders as
    // (bits & 0x7fff); NaN patterns (above infinity's) are taken as zero,
    // as the float maximum above ignores a NaN
    const uint32_t inf = f16 ? 0x7c00u : 0x7f80u;
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int q = 0; q < CPB; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t lo = xc[i][q][u] & 0x7fffu, hi = (xc[i][q][u] >> 16) & 0x7fffu;
          mb = max(mb, max(lo > inf ? 0u : lo, hi > inf ? 0u : hi));
        }
    amax = to_f32(mb);
  } else {
    for (int c = t; c < K / 8; c += 256) amax = chunk_max(reinterpret_cast<const u32x4_t*>(xr)[c], amax);
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = exp_of(amax);
  if (t == 0) em[m] = e;
  // (the exponent applied with ldexp: 2^-e itself overflows fp32 for rows
  // whose largest |x| is below 2^-127, bf16 subnormals)

  // blocks of BLK permuted columns; the lanes that share a group are
  // consecutive and aligned, so the group sum is a butterfly over them
  const int bpg = G / BLK;  // blocks per group: 2..16, a power of two
  auto emit = [&](int bi, const float (&src)[BLK]) {
    float part = 0.f;
    if (bi < nblk) {
      _Float16 out[BLK];
#pragma unroll
      for (int j = 0; j < BLK; ++j) {
        const float v = ldexpf(src[Perm<BITS>::src(j)], -e);
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
      tA[tail_idx(m, 3 * g, Kt)] = hi;
      tA[tail_idx(m, 3 * g + 1, Kt)] = hi;
      tA[tail_idx(m, 3 * g + 2, Kt)] = lo;
    }
  };
  if constexpr (RC > 0) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float src[BLK];
#pragma unroll
      for (int q = 0; q < CPB; ++q)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          src[8 * q + 2 * u] = to_f32(xc[i][q][u] & 0xffffu);
          src[8 * q + 2 * u + 1] = to_f32(xc[i][q][u] >> 16);
        }
      emit(t + 256 * i, src);
      // one block at a time: its values die before the next one's are made
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    for (int b0 = 0; b0 < nblk; b0 += 256) {
      const int bi = b0 + t;
      float src[BLK];
      if (bi < nblk) {
        if (k_perm == nullptr) {
#pragma unroll
          for (int q = 0; q < CPB; ++q) {
            const u32x4_t v = reinterpret_cast<const u32x4_t*>(xr + bi * BLK)[q];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              src[8 * q + 2 * u] = to_f32(v[u] & 0xffffu);
              src[8 * q + 2 * u + 1] = to_f32(v[u] >> 16);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < BLK; ++j) src[j] = to_f32(xr[k_perm[bi * BLK + j]]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < BLK; ++j) src[j] = 0.f;
      }
      emit(bi, src);
    }
  }
  for (int k = 3 * ng + t; k < Kt; k += 256) tA[tail_idx(m, k, Kt)] = 0;
}

// ---------------------------------------------------------------------------
// prep_w: one block per PW = 8 padded rows n0 .. n0+7.  PS = number of scale
// pieces; each is stored twice, as an fp16 pair (s, s), ready to multiply
// packed code pairs.  Layout K-tile-major, sh[kt][Np][SPT][PS] (one u32
// each, SPT = 2 groups per 64-code K tile for G = 32, else 1; a G = 128
// group serves two K tiles and is written for both), so the 32 rows a wave
// of the GEMM needs for one K tile are one coalesced load.
//   1. e_n: the exponent of the row's largest |scale|, less ESHIFT (a wave
//      per two rows); the tail entries and the output use e_n - MSHIFT
//   2. per (row, group), n fastest across the threads: the bias tail
//      entries cb = (off*s + b) * 2^-e_n as bf16 (hi, lo, hi) and the scale
//      pieces, from one load of the scale and the bias
// Small blocks keep every loop short: a loop of dependent loads per thread
// would wait out one memory latency per iteration.
constexpr int PW = 8;
template <int PS>
__device__ __forceinline__ void prep_w_rows(int blk, const void* __restrict__ scales, int s_dt,
                                            const void* __restrict__ biases, int b_dt, float off, int eshift, int mshift,
                                            int N,
                                            int Np,
                                            int ng, int G, int Kt, uint32_t* __restrict__ sh, uint16_t* __restrict__ tB,
                                            int* __restrict__ en) {
  __shared__ int e_s[PW];
  const int n0 = blk * PW, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  {
    float smax[PW / 4];
#pragma unroll
    for (int u = 0; u < PW / 4; ++u) {
      const int n = n0 + wave + 4 * u;
      smax[u] = 0.f;
      if (n < N)
        for (int g = lane; g < ng; g += 64) smax[u] = fmaxf(smax[u], fabsf(load_as_f32(scales, (long)n * ng + g, s_dt)));
    }
#pragma unroll
    for (int u = 0; u < PW / 4; ++u) {
      const int r = wave + 4 * u;
      const int e = exp_of(wave_max(smax[u])) - eshift;  // of the scale pieces
      if (lane == 0) {
        e_s[r] = e;
        en[n0 + r] = e - mshift;  // the output's: B values carry 2^mshift
      }
    }
  }
  __syncthreads();
  // per (row, group), n fastest: one load of the scale and the bias for the
  // tail entries cb = (off*s + b) * 2^-e_n as bf16 (hi, lo, hi) and the
  // scale pieces (whose stores, n fastest, are contiguous per K tile)
  const int tpg = G == 128 ? 2 : 1;  // K tiles per group
  for (int i = t; i < PW * ng; i += 256) {
    const int r = i % PW, g = i / PW, n = n0 + r;
    uint32_t pc[PS];
    uint16_t th = 0, tl = 0;
    if (n < N) {
      const float sv = load_as_f32(scales, (long)n * ng + g, s_dt);
      const float bv = load_as_f32(biases, (long)n * ng + g, b_dt);
      // with the B values' factor 2^mshift; ldexp, as 2^-e overflows fp32 for
      // scales below about 2^-121
      const float cb = ldexpf(fmaf(off, sv, bv), mshift - e_s[r]);
      th = f32_to_bf16_bits(cb);
      tl = f32_to_bf16_bits(cb - bf16_bits_to_f32(th));
      float rr = ldexpf(sv, -e_s[r]);  // exact
#pragma unroll
      for (int j = 0; j < PS; ++j) {
        const float q = (j == PS - 1) ? rr : trunc_bf16(rr);
        const uint32_t h = f32_to_f16_bits(q);
        pc[j] = h | (h << 16);
        rr -= q;
      }
    } else {
#pragma unroll
      for (int j = 0; j < PS; ++j) pc[j] = 0u;
    }
    tB[tail_idx(n, 3 * g, Kt)] = th;
    tB[tail_idx(n, 3 * g + 1, Kt)] = tl;
    tB[tail_idx(n, 3 * g + 2, Kt)] = th;
#pragma unroll
    for (int j = 0; j < PS; ++j) {
      if (G == 32) {
        sh[(((long)(g >> 1) * Np + n) * 2 + (g & 1)) * PS + j] = pc[j];
      } else {
        for (int u = 0; u < tpg; ++u) sh[((long)(g * tpg + u) * Np + n) * PS + j] = pc[j];
      }
    }
  }
  // the tail's zero padding columns
  const int pad = Kt - 3 * ng;
  for (int i = t; i < PW * pad; i += 256) tB[tail_idx(n0 + i / pad, 3 * ng + i % pad, Kt)] = 0;
}

// The same W-side pass with every load issued at once: thread t takes row
// t % PW and groups t / PW + 32 i (i < WI), so PW * ng <= 256 * WI.  The
// loop above waits out one memory latency per trip (ng/64 + ng/32 trips: 11
// at K = 14336, G = 64), and its blocks start after the rows of x; here a
// block waits once.  The row maximum is reduced over the 32 threads of a
// row (three butterfly steps in a wave, then the four waves through LDS).
// Rows past N load zeros (offsets out of range) and so write zeros, as
// above.
constexpr int WI = 8;
template <int PS>
__device__ __forceinline__ void prep_w_rows_once(int blk, const void* __restrict__ scales, int s_dt,
                                                 const void* __restrict__ biases, int b_dt, float off, int eshift,
                                                 int mshift, int N, int Np, int ng, int G, int Kt,
                                                 uint32_t* __restrict__ sh, uint16_t* __restrict__ tB,
                                                 int* __restrict__ en) {
  __shared__ float wmax[4][PW];
  const int n0 = blk * PW, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = t % PW, n = n0 + r, gq = t / PW;
  const uint32_t cnt = (uint32_t)N * (uint32_t)ng;
  // Every parameter is read as the aligned 32-bit word that holds it (16-bit
  // types: the pair, its half picked by the index), so both dtypes take the
  // same load, with no branch between the loads: all 2 WI of them are in
  // flight before the first use.  (The range is rounded up to whole words;
  // the last word of a 16-bit array may hold two bytes past it, never used.)
  auto raw = [&](const void* base, int dt, uint32_t (&w)[WI]) {
    const bool wide = dt == F32;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, wide ? cnt * 4u : (cnt * 2u + 3u) & ~3u);
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const int g = gq + 32 * i;
      const uint32_t e = (uint32_t)n * ng + g;
      const uint32_t o = (n < N && g < ng) ? (wide ? e * 4u : (e * 2u) & ~3u) : 0x80000000u;
      w[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, o, 0, 0);
    }
  };
  auto val = [&](uint32_t w, int i, int dt) {
    if (dt == F32) return __uint_as_float(w);
    const uint32_t h = (((uint32_t)n * ng + gq + 32 * i) & 1u) ? (w >> 16) : (w & 0xffffu);
    return dt == F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
  };
  uint32_t rsw[WI], rbw[WI];
  raw(scales, s_dt, rsw);
  raw(biases, b_dt, rbw);
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < WI; ++i) mx = fmaxf(mx, fabsf(val(rsw[i], i, s_dt)));
  mx = fmaxf(mx, __shfl_xor(mx, 8));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (lane < PW) wmax[wave][lane] = mx;
  __syncthreads();
  const int e = exp_of(fmaxf(fmaxf(wmax[0][r], wmax[1][r]), fmaxf(wmax[2][r], wmax[3][r]))) - eshift;
  if (t < PW) en[n0 + t] = e - mshift;  // the output's: B values carry 2^mshift
  const int tpg = G == 128 ? 2 : 1;  // K tiles per group
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int g = gq + 32 * i;
    if (g < ng) {
      const float sv = val(rsw[i], i, s_dt), bv = val(rbw[i], i, b_dt);
      const float cb = ldexpf(fmaf(off, sv, bv), mshift - e);  // with the B values' factor 2^mshift
      const uint16_t th = f32_to_bf16_bits(cb);
      const uint16_t tl = f32_to_bf16_bits(cb - bf16_bits_to_f32(th));
      float rr = ldexpf(sv, -e);  // exact
      uint32_t pc[PS];
#pragma unroll
      for (int j = 0; j < PS; ++j) {
        const float q = (j == PS - 1) ? rr : trunc_bf16(rr);
        const uint32_t h = f32_to_f16_bits(q);
        pc[j] = h | (h << 16);
        rr -= q;
      }
      tB[tail_idx(n, 3 * g, Kt)] = th;
      tB[tail_idx(n, 3 * g + 1, Kt)] = tl;
      tB[tail_idx(n, 3 * g + 2, Kt)] = th;
#pragma unroll
      for (int j = 0; j < PS; ++j) {
        if (G == 32) {
          sh[(((long)(g >> 1) * Np + n) * 2 + (g & 1)) * PS + j] = pc[j];
        } else {
          for (int u = 0; u < tpg; ++u) sh[((long)(g * tpg + u) * Np + n) * PS + j] = pc[j];
        }
      }
    }
  }
  // the tail's zero padding columns
  const int pad = Kt - 3 * ng;
  for (int i = t; i < PW * pad; i += 256) tB[tail_idx(n0 + i / pad, 3 * ng + i % pad, Kt)] = 0;
}

// prep_x and prep_w in one launch: blocks [0, Mp) take the rows of x, the
// rest take PW rows of W each; the two halves run side by side.
struct PrepArgs {
  const void* x;
  const int32_t* k_perm;
  const void* scales;
  const void* biases;
  _Float16* xh;
  uint16_t* tA;
  int* em;
  uint32_t* sh;
  uint16_t* tB;
  int* en;
  float off;
  int eshift, mshift;
  int act_dt, s_dt, b_dt;
  int M, N, K, G, Kt, BM, Mp, Np, ng;
};

template <int BITS, int PS, int RC>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  // the W rows first: their blocks are short and latency-bound, and run
  // beside the rows of x instead of after them
  const int nw = a.Np / PW;
  const int b = blockIdx.x;
  if (b >= nw)
    prep_x_row<BITS, RC>(b - nw, a.x, a.act_dt, a.k_perm, a.M, a.K, a.G, a.Kt, a.BM, a.xh, a.tA, a.em);
  else if (PW * a.ng <= 256 * WI)
    prep_w_rows_once<PS>(b, a.scales, a.s_dt, a.biases, a.b_dt, a.off, a.eshift, a.mshift, a.N, a.Np, a.ng, a.G, a.Kt,
                         a.sh, a.tB, a.en);
  else
    prep_w_rows<PS>(b, a.scales, a.s_dt, a.biases, a.b_dt, a.off, a.eshift, a.mshift, a.N, a.Np, a.ng, a.G, a.Kt, a.sh,
                    a.tB, a.en);
}

// ---------------------------------------------------------------------------
// main GEMM

struct GemmParams {
  const _Float16* xh;
  const uint16_t* tA;
  const int* em;
  const uint32_t* w;
  const uint32_t* sh;  // scale pieces, sh[kt][Np][SPT][PS]
  const uint16_t* tB;
  const int* en;
  uint16_t* y;
  int M, N, K, ng, Kt, G;
  int Np, gsh;  // padded row count of the W-side scratch; log2(G) - 5
  int Tm, Tn, per_xcd;
  int rect;     // XCD tile rectangles: 0, or the row-block split a (4 or 2; see the kernel)
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
  // The row's largest |scale| is brought to [2^ESHIFT, 2^(ESHIFT+1)): as
  // high as the largest code piece times scale piece still fits fp16 (4-bit:
  // 128 * 2^8, with the factor 16 below; 8-bit: 128 * 2^9; 2-bit:
  // 3 * 2^13), so that scales down to 2^-(14+ESHIFT) of the row's largest
  // stay normal fp16 numbers, exact.
  static constexpr int ESHIFT = BITS == 4 ? 7 : (BITS == 8 ? 8 : 12);
  // 4-bit B values carry a factor 16 (below); the pre-pass takes it out of
  // the row exponent e_n that scales the tail operand and the output
  static constexpr int MSHIFT = BITS == 4 ? 4 : 0;
  // `magic` holds 0x64006400 in a VGPR, so mask-and-insert is one
  // v_and_or_b32 (a VOP3 op reads at most one literal or SGPR on gfx950).
  // A nibble masked in place at bits 0-3 of a half gives 1024 + q; one at
  // bits 4-7 gives 1024 + 16 q with no shift (the fp16 ulp at 1024 is 1), so
  // a 32-bit word needs one shift (by 8) for its four nibble positions.
  // 4-bit: v[0][i] = (q - 8) for i even, 16 (q - 8) for i odd; decode_b
  // multiplies the even ones by 16 s, the odd ones by s: every B value is
  // 16 (q - 8) s, exact (at most 128 * 2^8 < 2^15 in magnitude).
  // 8-bit: the high nibble (weight 16) is placed at bits 4-7, the low one at
  // bits 0-3, both multiplied by s.
  static __device__ __forceinline__ void pieces(const uint32_t* wd, int half, uint32_t magic,
                                                f16x2_t (&v)[NPIECE][4]) {
    const f16x2_t k1032 = {(_Float16)-1032.f, (_Float16)-1032.f};
    const f16x2_t k1152 = {(_Float16)-1152.f, (_Float16)-1152.f};
    const f16x2_t k1024 = {(_Float16)-1024.f, (_Float16)-1024.f};
    if constexpr (BITS == 4) {
      const uint32_t t = wd[0] >> 8;
      v[0][0] = h2((wd[0] & 0x000F000Fu) | magic) + k1032;  // codes (c0, c4)
      v[0][1] = h2((wd[0] & 0x00F000F0u) | magic) + k1152;  // (c1, c5), x16
      v[0][2] = h2((t & 0x000F000Fu) | magic) + k1032;      // (c2, c6)
      v[0][3] = h2((t & 0x00F000F0u) | magic) + k1152;      // (c3, c7), x16
    } else if constexpr (BITS == 8) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t t = wd[w] >> 8;
        v[0][2 * w] = h2((wd[w] & 0x00F000F0u) | magic) + k1152;  // hi nibbles (c0,c2), x16
        v[0][2 * w + 1] = h2((t & 0x00F000F0u) | magic) + k1152;   // (c1,c3), x16
        v[1][2 * w] = h2((wd[w] & 0x000F000Fu) | magic) + k1032;  // lo nibbles
        v[1][2 * w + 1] = h2((t & 0x000F000Fu) | magic) + k1032;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[0][i] = h2(((wd[0] >> (2 * (i + 4 * half))) & 0x00030003u) | magic) + k1024;
    }
  }
  // factor of the scale piece for entry i of piece a (4-bit even entries)
  static constexpr bool times16(int i) { return BITS == 4 && (i & 1) == 0; }
};

// Main GEMM.  512 threads = 8 waves, two per SIMD; tile BM x 256 with
// BM = 64 MB.  Wave w = 4 wm + wn computes rows [32 MB wm, +32 MB) x
// columns [64 wn, +64) of the tile (MB 32-row blocks x 2 32-column blocks).
// The two waves of a SIMD cover each other's waits, and the VALU decode of
// one co-issues with the MFMAs of the other.
//
// Everything a K tile needs arrives in a 3-stage LDS ring by direct
// global -> LDS copies (buffer_load ... lds, whole 16-byte pieces per lane),
// issued two tiles ahead:
//   x      BM rows x 64 fp16 (tile-blocked by the pre-pass: one contiguous
//          block), 16-byte pieces XOR-swizzled by row;
//   codes  the tile's 256 weight rows x 8*BITS bytes, copied ONCE per
//          workgroup (wave w copies rows 32w .. 32w+31) and read back by
//          the two waves that use them.  Loading them straight into the
//          lanes that decode them (32 rows x 32 bytes per instruction,
//          duplicated for both row halves) kept the texture units 75% busy
//          with scattered requests and bounded the whole kernel.
// Scale pieces (pre-pass layout sh[kt][Np][SPT][PS]: a tile's 256 columns
// are one contiguous run) take the same route, a third small stage.
// Stages are separate LDS arrays, so the compiler can see that a copy into
// one stage does not touch the one being read.
// Rows of W past N are read through offsets past the buffer's range and
// come back as zeros, so the last column tile needs no clamping.

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 1)) & 7; }

template <int BITS, int PS, int MB>
struct Gemm {
  using D = Decode<BITS>;
  static constexpr int BM = 64 * MB;
  static constexpr int XB = BM * 128;            // bytes of one x stage
  static constexpr int RB = 8 * BITS;            // code bytes per weight row and K tile
  static constexpr int WB = BN * RB;             // bytes of one code stage
  static constexpr int A_DMA = XB / (512 * 16);  // x copies per thread and tile
  // code copies per wave and tile: 32 rows x RB bytes, 16 (2-bit: 4) bytes a lane
  static constexpr int W_SZ = BITS == 2 ? 4 : 16;
  static constexpr int W_DMA = 32 * RB / (64 * W_SZ);
  static constexpr int NF = D::NPIECE * PS;
  // scale pieces of a tile: 256 columns x SPT x PS words (SPT <= 2), copied
  // 4 bytes a lane, 2 KiB a workgroup per copy
  static constexpr int S_DMA = PS;
  static constexpr int SB = S_DMA * 2048;           // bytes of one scale stage
  static constexpr int VM_TILE = A_DMA + W_DMA + S_DMA;
  static_assert(VM_TILE < 64, "vmcnt field");
  static constexpr int WPL = BITS;                  // words per lane and 32 columns per tile

  __amdgpu_buffer_rsrc_t rw, rs, rx;
  uint32_t x_off, w_goff[W_DMA], s_goff[S_DMA];
  int w_lds[2];                                     // this lane's code bytes in a stage, per 32-column block
  int s_lds[2];                                     // this lane's scale pieces in a stage, per 32-column block
  int half, l32, wm, wave, kbase, last_kt, Np, spt;

  // x of tile kt into stage xs: instruction i of wave w fills bytes
  // [(8i + w) KiB, +1 KiB); lane l's piece is chunk 64 (8i + w) + l
  __device__ __forceinline__ void issue(int kt, unsigned char* xs, unsigned char* ws, unsigned char* ss) const {
    kt = kbase + min(kt, last_kt);
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(xs + (i * 8 + wave) * 1024), 16, x_off, kt * XB + i * 8192, 0, 0);
#pragma unroll
    for (int i = 0; i < W_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(ws + wave * 32 * RB + i * 64 * W_SZ), W_SZ, w_goff[i],
          kt * RB, 0, 0);
    // the tile's scale pieces: row block n0 .. n0+255 of K tile kt, one
    // contiguous run of 256*SPT*PS words (lanes past the run copy zeros)
    const int so = __builtin_amdgcn_readfirstlane(kt * Np * spt * PS * 4);
#pragma unroll
    for (int i = 0; i < S_DMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(ss + i * 2048 + wave * 256),
                                               4, s_goff[i], so, 0, 0);
  }
  // this lane's scale pieces of the tile, per 32-column block
  __device__ __forceinline__ void read_s(const unsigned char* __restrict__ ss, uint32_t (&sc)[2][PS]) const {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < PS; ++j) sc[nb][j] = *reinterpret_cast<const uint32_t*>(ss + s_lds[nb] + 4 * j);
  }
  __device__ __forceinline__ void read_a(const unsigned char* __restrict__ xs, int s, f16x8_t (&af)[MB]) const {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = wm * 32 * MB + mb * 32 + l32;
      af[mb] = *reinterpret_cast<const f16x8_t*>(xs + r * 128 + (((4 * half + s) ^ swz(r)) << 4));
    }
  }
  // this lane's code words of the tile, per 32-column block
  __device__ __forceinline__ void read_w(const unsigned char* __restrict__ ws, uint32_t (&wv)[2][WPL]) const {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if constexpr (BITS == 2) {
        const u32x2_t u = *reinterpret_cast<const u32x2_t*>(ws + w_lds[nb]);
        wv[nb][0] = u.x;
        wv[nb][1] = u.y;
      } else {
#pragma unroll
        for (int q = 0; q < WPL / 4; ++q) {
          // 8-bit: the row's second 16-byte piece of this half sits one
          // swizzle step away (piece index c ^ swizzle, c = 2 half + q)
          const int o = BITS == 8 ? w_lds[nb] + (((2 * half + q) ^ ((w_lds[nb] >> 8) & 3)) << 4) : w_lds[nb];
          const u32x4_t u = *reinterpret_cast<const u32x4_t*>(ws + o);
          wv[nb][4 * q] = u.x;
          wv[nb][4 * q + 1] = u.y;
          wv[nb][4 * q + 2] = u.z;
          wv[nb][4 * q + 3] = u.w;
        }
      }
    }
  }
  __device__ __forceinline__ void decode_b(const uint32_t (&wv)[2][WPL], const uint32_t (&sc)[2][PS], int s,
                                           uint32_t magic, f16x8_t (&bf)[2][NF]) const {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      uint32_t wd[2];
      if constexpr (BITS == 4) {
        wd[0] = wv[nb][s];
      } else if constexpr (BITS == 8) {
        wd[0] = wv[nb][2 * s];
        wd[1] = wv[nb][2 * s + 1];
      } else {
        wd[0] = wv[nb][s >> 1];
      }
      f16x2_t vv[D::NPIECE][4];
      D::pieces(wd, s & 1, magic, vv);
#pragma unroll
      for (int a = 0; a < D::NPIECE; ++a)
#pragma unroll
        for (int j = 0; j < PS; ++j) {
          const f16x2_t sj = h2(sc[nb][j]);
          const f16x2_t sj16 = sj * f16x2_t{(_Float16)16.f, (_Float16)16.f};  // (unused unless 4-bit)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f16x2_t q = vv[a][i] * (D::times16(i) ? sj16 : sj);
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
  static constexpr int N_MFMA = 2 * NF * MB;
  // one MFMA at a time, with the VALU, DS reads and vector-memory loads of
  // the same region spread between them
  template <int NVALU, int NDS, int NVM = 0>
  static __device__ __forceinline__ void interleave() {
    constexpr int per = (NVALU + N_MFMA - 1) / N_MFMA;
    constexpr int vper = (NVM + N_MFMA - 1) / N_MFMA;
#pragma unroll
    for (int i = 0; i < N_MFMA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
      if (per > 0) __builtin_amdgcn_sched_group_barrier(0x002, per, 0);  // VALU
      if (i < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
      if (vper > 0 && i * vper < NVM) __builtin_amdgcn_sched_group_barrier(0x020, vper, 0);  // VMEM read
    }
  }
  // What one K tile hands to the next: the tile's code words and scale
  // pieces and its first 16-code step's A and B fragments.
  struct Carry {
    uint32_t wv[2][WPL];
    uint32_t sc[2][PS];
    f16x8_t a0[MB];
    f16x8_t b0[2][NF];
  };
  // Wait until tile kt is in LDS for every wave (this wave's copies by
  // vmcnt, with tile kt+1's still in flight; the others' by the barrier),
  // which also orders every wave's earlier LDS reads before it.
  static __device__ __forceinline__ void sync_tile() {
    __builtin_amdgcn_s_waitcnt((VM_TILE & 15) | (7 << 4) | (0 << 8) | ((VM_TILE >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  // the carry of the tile in stage S
  template <int S>
  __device__ __forceinline__ void begin(unsigned char* const (&xs)[3], unsigned char* const (&ws)[3],
                                        unsigned char* const (&ss)[3], uint32_t magic, Carry& c) const {
    read_w(ws[S], c.wv);
    read_s(ss[S], c.sc);
    read_a(xs[S], 0, c.a0);
    decode_b(c.wv, c.sc, 0, magic, c.b0);
  }
  // One K tile kt in stage / ring entry S = kt % 3, its carry ready:
  //   its four 16-code steps, each step's MFMAs with the next step's A
  //   reads and decode spread between them; the copies of tile kt+2 (into
  //   stage (kt+2)%3, free since the previous tile's barrier) go out
  //   between the first step's MFMAs, not as one burst that would stall the
  //   wave behind a full address queue;
  //   before the last step's MFMAs: sync_tile for tile kt+1, then tile
  //   kt+1's carry is read and decoded between those MFMAs, so no wave
  //   leaves the barrier with nothing for the matrix unit to do.
  // Every load of the loop is a copy into LDS (none writes a VGPR), so the
  // compiler adds no waits of its own for them: the one wait before the
  // barrier covers everything.
  template <int S>
  __device__ __forceinline__ void step(int kt, unsigned char* const (&xs)[3], unsigned char* const (&ws)[3],
                                       unsigned char* const (&ss)[3], uint32_t magic, f32x16_t (&acc)[MB][2],
                                       Carry& c) const {
    constexpr int DEC = 2 * NF * 16;
    const unsigned char* X = xs[S];
    f16x8_t a1[MB];
    f16x8_t b1[2][NF];
    read_a(X, 1, a1);
    decode_b(c.wv, c.sc, 1, magic, b1);
    issue(kt + 2, xs[(S + 2) % 3], ws[(S + 2) % 3], ss[(S + 2) % 3]);
    mfma_b(c.a0, c.b0, acc);
    interleave<DEC, MB, VM_TILE>();
    __builtin_amdgcn_sched_barrier(0);
    read_a(X, 2, c.a0);
    decode_b(c.wv, c.sc, 2, magic, c.b0);
    mfma_b(a1, b1, acc);
    interleave<DEC, MB>();
    __builtin_amdgcn_sched_barrier(0);
    read_a(X, 3, a1);
    decode_b(c.wv, c.sc, 3, magic, b1);
    mfma_b(c.a0, c.b0, acc);
    interleave<DEC, MB>();
    __builtin_amdgcn_sched_barrier(0);
    sync_tile();
    begin<(S + 1) % 3>(xs, ws, ss, magic, c);
    mfma_b(a1, b1, acc);
    interleave<DEC, MB + 2 + 2>();
    __builtin_amdgcn_sched_barrier(0);
  }
};
// ---------------------------------------------------------------------------

// Epilogue of a tile whose rows all exist: y = 2^(e_m + e_n) * acc, rounded
// to the activation dtype.  32x32 accumulator layout: lane -> column l32;
// register r -> row 8*(r/4) + 4*half + r%4, so registers 2i and 2i+1 are
// consecutive rows of one column: one packed pair (bf16: one packed
// conversion, the instruction a single value takes too; f16: two scalar
// conversions), two 2-byte stores (the second from the high half).
template <bool OUT_F16, int MB>
__device__ __forceinline__ void epilogue_full(const f32x16_t (&acc)[MB][2], const int* em_s, const GemmParams& p,
                                              int m0, int n0, int row0, int half, int l32, int wn) {
  const long N = p.N;
  // uniform part: the wave's first row and column block
  const uint64_t yw = reinterpret_cast<uint64_t>(p.y + (long)(m0 + row0) * N + n0 + wn * 64);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = n0 + wn * 64 + nb * 32 + l32;
    if (n < p.N) {
      const int e_n = p.en[n];
      const uint32_t lo = (uint32_t)(4 * half * N + nb * 32 + l32) * 2u;  // lane part, bytes
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const i32x4_t e4 = *reinterpret_cast<const i32x4_t*>(&em_s[row0 + mb * 32 + 8 * rq + 4 * half]);
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            const float v0 = ldexpf(acc[mb][nb][4 * rq + j], e4[j] + e_n);
            const float v1 = ldexpf(acc[mb][nb][4 * rq + j + 1], e4[j + 1] + e_n);
            uint32_t pk;
            if constexpr (OUT_F16)
              pk = f32x2_to_f16x2_bits(v0, v1);
            else
              pk = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){v0, v1}, bf16x2_t));
            // the rows' addresses as scalar values (kept out of the lane
            // offset, so each store is scalar base + the lane's offset)
            uint64_t r0 = yw + (uint64_t)((mb * 32 + 8 * rq + j) * N * 2);
            uint64_t r1 = r0 + (uint64_t)(N * 2);
            asm volatile("" : "+s"(r0), "+s"(r1));
            typedef __attribute__((address_space(1))) unsigned char gbyte;
            *reinterpret_cast<__attribute__((address_space(1))) uint16_t*>(reinterpret_cast<gbyte*>(r0) + lo) =
                (uint16_t)pk;
            *reinterpret_cast<__attribute__((address_space(1))) uint16_t*>(reinterpret_cast<gbyte*>(r1) + lo) =
                (uint16_t)(pk >> 16);
          }
        }
    }
  }
}

template <int BITS, int PS, int MB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_affine_kernel(GemmParams p) {
  using GK = Gemm<BITS, PS, MB>;
  constexpr int BM = GK::BM, XB = GK::XB, WB = GK::WB, RB = GK::RB;

  const int b = blockIdx.x;
  const int vs = (b & 7) * p.per_xcd + (b >> 3);
  if (vs >= p.Tm * p.Tn * p.S) return;
  const int v = vs / p.S, sp = vs % p.S;
  int tm = v / p.Tn, tn = v % p.Tn;
  if (p.rect) {
    // XCD x takes the tile rectangle (x / nb, x % nb) of an a x nb split of
    // the grid (a = p.rect, a * nb = 8), row blocks fastest (p.S == 1,
    // Tm % a == 0, Tn % nb == 0)
    const int a = p.rect, nb = 8 / a;
    const int x = b & 7, j = b >> 3, rm = p.Tm / a, rn = p.Tn / nb;
    tm = (x / nb) * rm + j % rm;
    tn = (x % nb) * rn + j / rm;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63, l32 = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int nkt_all = p.K / BK, per_split = (nkt_all + p.S - 1) / p.S;
  const int kt0 = sp * per_split, kt1 = min(nkt_all, kt0 + per_split);

  __shared__ __attribute__((aligned(1024))) unsigned char x0[XB];
  __shared__ __attribute__((aligned(1024))) unsigned char x1[XB];
  __shared__ __attribute__((aligned(1024))) unsigned char x2[XB];
  __shared__ __attribute__((aligned(1024))) unsigned char w0[WB];
  __shared__ __attribute__((aligned(1024))) unsigned char w1[WB];
  __shared__ __attribute__((aligned(1024))) unsigned char w2[WB];
  __shared__ __attribute__((aligned(1024))) unsigned char s0[GK::SB];
  __shared__ __attribute__((aligned(1024))) unsigned char s1[GK::SB];
  __shared__ __attribute__((aligned(1024))) unsigned char s2[GK::SB];
  __shared__ __attribute__((aligned(16))) int em_s[BM];
  for (int i = t; i < BM; i += 512) em_s[i] = p.em[m0 + i];
  unsigned char* const xs[3] = {x0, x1, x2};
  unsigned char* const ws[3] = {w0, w1, w2};
  unsigned char* const ss[3] = {s0, s1, s2};

  f32x16_t acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  GK P;
  const uint32_t row_bytes = (uint32_t)p.K * BITS / 8;
  P.rw = make_rsrc(p.w, (uint32_t)p.N * row_bytes);
  // (uniform values, kept in SGPRs: a buffer resource or soffset the
  // compiler takes for divergent becomes a per-lane loop around each load)
  P.Np = __builtin_amdgcn_readfirstlane(p.Np);
  P.spt = __builtin_amdgcn_readfirstlane(p.G == 32 ? 2 : 1);
  P.rs = make_rsrc(p.sh, (uint32_t)__builtin_amdgcn_readfirstlane(nkt_all * P.Np * P.spt * PS * 4));
  P.rx = make_rsrc(p.xh + (long)m0 * p.K, (uint32_t)BM * p.K * 2);
  P.half = half;
  P.l32 = l32;
  P.wm = wm;
  P.wave = wave;
  {
    // x: lane l of wave w copies chunk 64 w + l (+ 512 i): row r = 8 w + l/8
    // (+ 64 i), LDS position l % 8, which holds source chunk (l%8)^swz(r)
    const int r = wave * 8 + (lane >> 3);
    P.x_off = (uint32_t)r * 128 + (((lane & 7) ^ swz(r)) << 4);
  }
  // Code stage layout: row r (of the tile's 256) at r*RB, its 16-byte pieces
  // XOR-swizzled by row (4-bit: piece ^ (r>>3)&1; 8-bit: piece ^ (r>>2)&3),
  // so that the 16 lanes of a read phase hit 16 different bank groups.
  // Copy instruction i of wave w writes W_SZ bytes per lane from byte
  // w*32*RB + i*64*W_SZ of the stage: lane l's LDS byte is pos = that + l*W_SZ.
#pragma unroll
  for (int i = 0; i < GK::W_DMA; ++i) {
    const int pos = wave * 32 * RB + i * 64 * GK::W_SZ + lane * GK::W_SZ;
    const int r = pos / RB, in_row = pos % RB;
    int src = in_row;  // logical byte in the row's RB bytes of this tile
    if constexpr (BITS == 4) src = ((((in_row >> 4) ^ (r >> 3)) & 1) << 4) | (in_row & 15);
    if constexpr (BITS == 8) src = ((((in_row >> 4) ^ (r >> 2)) & 3) << 4) | (in_row & 15);
    const uint32_t n = n0 + r;
    P.w_goff[i] = n * row_bytes + (uint32_t)src;
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r = wn * 64 + nb * 32 + l32;  // row in the tile
    if constexpr (BITS == 4) P.w_lds[nb] = r * RB + (((half ^ (r >> 3)) & 1) << 4);
    else if constexpr (BITS == 8) P.w_lds[nb] = r * RB;  // pieces picked per half in read_w
    else P.w_lds[nb] = r * RB + half * 8;
    P.s_lds[nb] = (r * P.spt + (P.spt == 2 ? half : 0)) * PS * 4;
  }
  // scale copy i: lane l of wave w takes bytes 2048 i + 4 (64 w + l) of the
  // tile's run, which starts at word n0 * SPT * PS of K tile kt's block;
  // past the run it reads from an out-of-range offset (zeros)
#pragma unroll
  for (int i = 0; i < GK::S_DMA; ++i) {
    const uint32_t run = 256u * P.spt * PS * 4;
    const uint32_t b = (uint32_t)(2048 * i + 4 * (64 * wave + lane));
    P.s_goff[i] = b < run ? (uint32_t)n0 * P.spt * PS * 4 + b : 0x80000000u;
  }
  const int nkt = kt1 - kt0;
  P.kbase = kt0;
  P.last_kt = nkt - 1;

  // ---- the bias tail first: acc = sum_g xs * cb on bf16 MFMA over the Kt
  // tail columns (a multiple of 16), first split only.  Operands come
  // straight from global memory (L2-resident), TD 16-column steps in flight;
  // the first ones are issued ahead of the first two tiles' copies, so their
  // latency and the copies' overlap.  A load for a step past the end re-reads
  // the last step (in range, never used).  (Four or six steps in flight,
  // where the registers allow, measured no faster.)
  constexpr int TD = 3;
  const bool tail = sp == 0;
  const int nk = p.Kt / 16;
  // (fragment-ordered operands: a 32 x 16 block is 1 KiB, lane l's 16
  // bytes at 16 l; 32-row blocks are Kt/16 blocks apart)
  const long tblk = (long)(p.Kt >> 4) * 512;
  const uint16_t* ta_row = p.tA + ((m0 + wm * 32 * MB) >> 5) * tblk + lane * 8;
  const uint16_t* tb_row = p.tB + ((n0 + wn * 64) >> 5) * tblk + lane * 8;
  bf16x8_t ta_r[TD][MB], tb_r[TD][2];
  auto tail_load = [&](int kk, bf16x8_t (&a)[MB], bf16x8_t (&bb)[2]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) bb[nb] = *reinterpret_cast<const bf16x8_t*>(tb_row + nb * tblk + kk * 512);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a[mb] = *reinterpret_cast<const bf16x8_t*>(ta_row + mb * tblk + kk * 512);
  };
  auto tail_mfma = [&](const bf16x8_t (&a)[MB], const bf16x8_t (&bb)[2]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], bb[nb], acc[mb][nb], 0, 0, 0);
  };
  if (tail) {
#pragma unroll
    for (int i = 0; i < TD; ++i) tail_load(min(i, nk - 1), ta_r[i], tb_r[i]);
  }

  P.issue(0, xs[0], ws[0], ss[0]);
  P.issue(1, xs[1], ws[1], ss[1]);

  if (tail) {
    int k = 0;
    for (; k + TD < nk; k += TD) {
#pragma unroll
      for (int i = 0; i < TD; ++i) {
        tail_mfma(ta_r[i], tb_r[i]);
        tail_load(min(k + TD + i, nk - 1), ta_r[i], tb_r[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < TD; ++i)
      if (k + i < nk) tail_mfma(ta_r[i], tb_r[i]);
  }

  uint32_t magic = 0x64006400u;
  asm volatile("" : "+v"(magic));
  typename GK::Carry c;
  GK::sync_tile();
  P.template begin<0>(xs, ws, ss, magic, c);
  // whole rounds of three tiles with no branch inside (so the compiler's
  // count of loads in flight is the same on every path into a step), then
  // the last one or two tiles.  The last tile's step reads the carry of a
  // tile past the end (zeros or unused codes, never used).
  int kt = 0;
  for (; kt + 3 <= nkt; kt += 3) {
    P.template step<0>(kt, xs, ws, ss, magic, acc, c);
    P.template step<1>(kt + 1, xs, ws, ss, magic, acc, c);
    P.template step<2>(kt + 2, xs, ws, ss, magic, acc, c);
  }
  if (kt < nkt) P.template step<0>(kt, xs, ws, ss, magic, acc, c);
  if (kt + 1 < nkt) P.template step<1>(kt + 1, xs, ws, ss, magic, acc, c);
  // copies into LDS still in flight (the prefetches past the last tile)
  // must land before the workgroup's LDS can go to another workgroup
  __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8) | (0 << 14));

  const int row0 = wm * 32 * MB;  // this wave's first row in the tile
  // ---- epilogue: y = 2^(e_m + e_n) * acc, rounded to the activation dtype.
  // 32x32 accumulator layout: lane -> column l32; register r -> row
  // 8*(r/4) + 4*half + r%4.  Stores go through a buffer resource over y: a
  // column past N starts from an out-of-range offset and a row past M lands
  // past the range, so neither is written.
  if (p.S > 1) {
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.part + (long)sp * p.M * p.N, (uint32_t)p.M * p.N * 4);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = n0 + wn * 64 + nb * 32 + l32;
      const bool nok = n < p.N;
      const int e_n = nok ? p.en[n] : 0;
      const uint32_t vb = nok ? ((uint32_t)(m0 + row0 + 4 * half) * p.N + n) * 4u : 0x80000000u;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const i32x4_t e4 = *reinterpret_cast<const i32x4_t*>(&em_s[row0 + mb * 32 + 8 * rq + 4 * half]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ldexpf(acc[mb][nb][4 * rq + j], e4[j] + e_n)), rp,
                                                  vb + (uint32_t)((mb * 32 + 8 * rq + j) * p.N) * 4u, 0, 0);
        }
    }
    return;
  }
  if (m0 + BM <= p.M) {
    // Every row of the tile exists (all but a ragged last row tile): the
    // row offset is uniform and goes into the scalar base address, the lane
    // keeps one offset for all its stores, two rows share one packed
    // conversion, and a column past N is masked off.
    if (p.out_f16) epilogue_full<true, MB>(acc, em_s, p, m0, n0, row0, half, l32, wave & 3);
    else epilogue_full<false, MB>(acc, em_s, p, m0, n0, row0, half, l32, wave & 3);
    return;
  }
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y, (uint32_t)p.M * p.N * 2);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = n0 + wn * 64 + nb * 32 + l32;
    const bool nok = n < p.N;
    const int e_n = nok ? p.en[n] : 0;
    const uint32_t vb = nok ? ((uint32_t)(m0 + row0 + 4 * half) * p.N + n) * 2u : 0x80000000u;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const i32x4_t e4 = *reinterpret_cast<const i32x4_t*>(&em_s[row0 + mb * 32 + 8 * rq + 4 * half]);
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

// The same sum, eight outputs a thread (16-byte loads of each partial, one
// 16-byte store), for MN % 8 == 0 and y 16-byte aligned; the order of the
// additions is the same as above.
__global__ __launch_bounds__(256) void gemm_split_sum8_kernel(const float* __restrict__ part,
                                                              uint16_t* __restrict__ y, long MN, int S, int out_f16) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= MN) return;
  f32x4_t a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float* ps = part + (long)s * MN + i;
    a += *reinterpret_cast<const f32x4_t*>(ps);
    b += *reinterpret_cast<const f32x4_t*>(ps + 4);
  }
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2_t v = j < 2 ? f32x2_t{a[2 * j], a[2 * j + 1]} : f32x2_t{b[2 * j - 4], b[2 * j - 3]};
    o[j] = out_f16 ? f32x2_to_f16x2_bits(v[0], v[1]) : __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  }
  *reinterpret_cast<u32x4_t*>(y + i) = o;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

template <int BITS, int PS>
hipError_t run(const AffineArgs& a, hipStream_t s) {
  // buffer resources address W, the scale pieces and one x tile with 32-bit offsets
  if (a.N * a.K * BITS / 8 >= (int64_t(1) << 31) || a.K * 2 * 256 >= (int64_t(1) << 31))
    return hipErrorNotSupported;
  const int M = (int)a.M, N = (int)a.N, K = (int)a.K, G = a.G;
  const int ng = K / G;
  // tail columns: 3 per group, padded with zeros to whole 16-column MFMA steps
  const int Kt = (3 * ng + 15) / 16 * 16;
  // the largest row tile whose grid still fills three quarters of the CUs
  // in one round: a bigger tile's efficiency is worth a few idle CUs, and a
  // grid just past one round runs its last tiles as a second round alone.
  // With a long K, 256-row tiles that fill half the CUs take K in two
  // splits instead of 128-row tiles (the bigger tile decodes each code for
  // twice the rows; the fp32 partials cost less than that saves from K =
  // 8192 on: M = 2048, N = 4096, K = 14336: 4-bit 292-295 -> 265-268 us,
  // 8-bit 451-454 -> 430-432 us; at K = 4096 it was 4-10% slower).
  // When no tile does (few columns: K is split below), 128-row tiles from
  // M = 1024 on: each decoded code serves twice the rows of a 64-row tile,
  // against twice the splits (M = 2048, N = 1024, K = 4096: 8-bit 70-76 ->
  // 62 us, 4-bit 49-50 -> 48.5 us; 256-row tiles with 8 splits were slower)
  int MB = 2;
  if (M > 64) {
    const int64_t tn = (N + BN - 1) / BN;
    if ((int64_t)((M + 255) / 256) * tn >= 192) MB = 8;
    else if ((int64_t)((M + 255) / 256) * tn >= 96 && K >= 8192) MB = 8;
    else if ((int64_t)((M + 127) / 128) * tn >= 192) MB = 4;
    else if (M >= 1024) MB = 4;
  }
  // 8-bit codes with three scale pieces do not fit the registers of the
  // 256-row tile
  if (BITS == 8 && PS == 3 && MB == 8) MB = 4;
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
  const size_t o_sh = o_em + s_em, s_sh = align256((size_t)(K / BK) * Np * (G == 32 ? 2 : 1) * PS * 4);
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
  uint32_t* sh = (uint32_t*)(scratch + o_sh);
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
  pa.eshift = Decode<BITS>::ESHIFT;
  pa.mshift = Decode<BITS>::MSHIFT;
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
  pa.Np = Np;
  pa.ng = ng;
  // x rows held in registers between the two passes when they fit (RC
  // 16-byte chunks a thread)
  const int nch = K / 8;
  const dim3 pg(Mp + Np / PW);
  if (a.k_perm == nullptr && nch <= 256 * 2)
    hipLaunchKernelGGL((prep_kernel<BITS, PS, 2>), pg, dim3(256), 0, s, pa);
  else if (a.k_perm == nullptr && nch <= 256 * 8)
    hipLaunchKernelGGL((prep_kernel<BITS, PS, 8>), pg, dim3(256), 0, s, pa);
  else
    hipLaunchKernelGGL((prep_kernel<BITS, PS, 0>), pg, dim3(256), 0, s, pa);

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
  // Without a K split, each XCD takes a rectangle of the tile grid instead of
  // whole rows of tiles: the tiles resident on one XCD then share some of
  // x's row blocks and of W's columns through its L2 (with a 4 x 2 split,
  // M = 2048, N = 14336, 4-bit: 251-255 -> 244-246 us; 8-bit N = K = 4096:
  // 150-154 -> 145-146 us).  Of the 4 x 2 and 2 x 4 splits, the one whose
  // rectangle holds fewer bytes of x and W.
  p.rect = 0;
  if (S == 1) {
    const double xb = (double)BM * K * 2, wb = (double)BN * K * BITS / 8;
    auto bytes = [&](int a) { return (p.Tm / a) * xb + (p.Tn / (8 / a)) * wb; };
    const bool ok4 = p.Tm % 4 == 0 && p.Tn % 2 == 0, ok2 = p.Tm % 2 == 0 && p.Tn % 4 == 0;
    if (ok4 && (!ok2 || bytes(4) <= bytes(2))) p.rect = 4;
    else if (ok2) p.rect = 2;
  }
  const dim3 grid(8 * p.per_xcd);
  // row tile BM = 32 MB: each wave takes MB/2 32-row blocks
  if (MB == 2)
    hipLaunchKernelGGL((gemm_affine_kernel<BITS, PS, 1>), grid, dim3(512), 0, s, p);
  else if (MB == 4)
    hipLaunchKernelGGL((gemm_affine_kernel<BITS, PS, 2>), grid, dim3(512), 0, s, p);
  else if constexpr (!(BITS == 8 && PS == 3))
    hipLaunchKernelGGL((gemm_affine_kernel<BITS, PS, 4>), grid, dim3(512), 0, s, p);
  e = hipGetLastError();
  if (e == hipSuccess && S > 1) {
    const long MN = (long)M * N;
    if (MN % 8 == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0)
      hipLaunchKernelGGL(gemm_split_sum8_kernel, dim3((unsigned)((MN / 8 + 255) / 256)), dim3(256), 0, s, p.part,
                         (uint16_t*)a.y, MN, S, p.out_f16);
    else
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
