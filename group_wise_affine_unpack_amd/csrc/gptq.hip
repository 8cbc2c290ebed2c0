// GPTQ layout (TinyGPT "Quantization Expansion", section 1 "GPTQReader",
// "Format" and the dequant recipe):
//   qweight [K/8, N] int32: 8 codes along K per word, code i in nibble i%8
//   qzeros  [K/G, N/8] int32: 8 zero points along N per word, stored as zero-1
//   scales  [K/G, N] f16;  g_idx [K] int32 (act-order) or NULL (i/G)
//   W[n,i] = scale[g,n] * (q - (z_stored + 1)),  g = g_idx[i]
//
// qmm_gptq (direct kernel): split-K over workgroups and waves, up to four
// adjacent output columns per lane, an LDS table for the act-order group
// lookup; described at the kernel below.
//
// gptq_to_affine_repack (kernel part): gathers codes through the permutation
// (computed on the host) into the affine [N, K/8] layout and writes the
// transposed scales and the biases -scale*(z+1).
#include <algorithm>
#include <mutex>

#include "common.h"

namespace qaff {
namespace {

// Waves per workgroup of the VALU direct kernel, each on its own part of
// the K slice, and the most word rows one wave holds in registers: 16 x 8
// for one x row (latency hiding), 8 x 16 for more (the accumulators of
// 16 waves would not fit); a slice has at most WROWS word rows either way.
template <int MT> constexpr int direct_waves() { return MT == 1 ? 16 : 8; }
constexpr int WROWS = 128;
constexpr uint32_t OOB = 0x80000000u;  // a buffer offset past any range: the load reads 0
constexpr int kMaxLds = 160 * 1024;    // LDS of one CU

__device__ __forceinline__ uint32_t nib(uint32_t w, int j) { return (w >> (4 * j)) & 0xFu; }

template <int CPL> struct WordsT;
template <> struct WordsT<1> { typedef uint32_t T; };
template <> struct WordsT<2> { typedef u32x2_t T; };
template <> struct WordsT<4> { typedef u32x4_t T; };

// CPL consecutive qweight words of one row (buffer load; an offset past the
// range reads zeros)
template <int CPL>
__device__ __forceinline__ typename WordsT<CPL>::T load_words(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (CPL == 4)
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  else if constexpr (CPL == 2)
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  else
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <int CPL>
__device__ __forceinline__ uint32_t word_of(const typename WordsT<CPL>::T& v, int c) {
  if constexpr (CPL == 1) return v;
  else return v[c];
}

// (scale, bias) table of one workgroup in LDS: per group, CPL pairs for each
// of the 64 lanes.  Pairs of two adjacent columns of a lane form one 16-byte
// entry and the 64 lanes' entries are consecutive, so a lane reads its
// columns' pairs with CPL/2 conflict-free 16-byte reads (one 8-byte read
// when CPL == 1).
template <int CPL>
struct GTab {
  static constexpr int COLS = 64 * CPL;     // columns per workgroup
  static constexpr int GBYTES = COLS * 8;   // bytes per group
  static __device__ __forceinline__ int off(int c) {  // column c of the workgroup
    if constexpr (CPL == 1) return c * 8;
    const int ln = c / CPL, j = c % CPL;
    return ((j >> 1) * 64 + ln) * 16 + (j & 1) * 8;
  }
};

// LDS of one workgroup, in bytes: the (scale, bias) table, the slice's
// group offsets (one int per code), MT rows of x for the slice (fp32), and
// the waves' partial sums.
// Groups in the direct kernel's table: every group with act-order (any code
// may map to any group), else those a slice of per_sp word rows can touch.
__host__ __device__ inline int table_groups(bool act, int ng, int per_sp, int gsh) {
  return act ? ng : min(ng, ((per_sp * 8 + (1 << gsh) - 1) >> gsh) + 1);  // G = 2^gsh
}

// Where the direct kernel finds a code's (scale, bias) pair:
//   SLICE:  LDS table of the groups the workgroup's K slice touches (g_idx NULL)
//   LDS:    LDS table of every group (act-order, the table fits in LDS)
//   GLOBAL: act-order with more groups than the LDS holds: a table
//           [K/G][N] of fp32 (scale, bias) pairs, written to device memory by
//           gptq_table_kernel before the launch and read through L2
enum TabMode : int { SLICE = 0, LDS = 1, GLOBAL = 2 };
__host__ __device__ inline int direct_table_groups(int mode, int ng, int per_sp, int gsh) {
  return mode == GLOBAL ? 0 : table_groups(mode == LDS, ng, per_sp, gsh);
}

struct DirectLds {
  int tab, goff, xs, red, total;
  __host__ __device__ DirectLds(int ng, int cpl, int mt, int per_sp) {
    tab = 0;
    goff = ng * 64 * cpl * 8;
    xs = goff + per_sp * 8 * 4;
    red = xs + mt * per_sp * 8 * 4;
    total = red + (mt == 1 ? 16 : 8) * mt * 64 * cpl * 4;  // direct_waves<mt>() partial rows
  }
};

// Direct GPTQ GEMV / small GEMM.  Workgroup (cg, sp): columns
// [COLS cg, COLS cg + COLS), COLS = 64 CPL, lane l holding columns CPL l ..
// CPL l + CPL - 1, and word rows of K slice sp of S, which its GW waves split
// again.  A lane reads CPL adjacent qweight words of a row with one load,
// so a wave reads 256 CPL contiguous bytes per row: whole cache lines when
// CPL = 4.  The workgroup first builds an LDS table of (scale, -scale*(z+1))
// in fp32 for every group and column, so the act-order lookup
// g_idx[k] -> table row is one LDS read per code and two columns, and the
// weight is exact in fp32: W = scale*q + bias.  The slice's table offsets
// (from g_idx) and x values (fp32) are staged in LDS too, so the loop
// issues LDS reads only, which complete in order and pipeline.  Codes become
// floats with byte conversions (even and odd nibbles masked into bytes).
// The waves meet in LDS; each slice writes fp32 partials [S][M][N], and a
// second kernel adds the S partials into y.  Rows of x go MT at a time; the
// table serves every pass.
template <int CPL, int MT, int MODE>
__global__ __launch_bounds__(64 * direct_waves<MT>()) void gptq_direct_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint32_t* __restrict__ qz,
    const uint16_t* __restrict__ sc, const int32_t* __restrict__ g_idx, const float2* __restrict__ gtab,
    float* __restrict__ part, int M, int N, int K, int gsh, int S) {
  constexpr bool ACT = MODE != SLICE;
  constexpr int GW = direct_waves<MT>(), KB = WROWS / GW;
  using T = GTab<CPL>;
  using W = typename WordsT<CPL>::T;
  constexpr int COLS = T::COLS;
  constexpr int GB_SHIFT = CPL == 4 ? 11 : (CPL == 2 ? 10 : 9);  // log2(GBYTES)
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int ng = K >> gsh;
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int ncg = (N + COLS - 1) / COLS;
  const int cg = blockIdx.x % ncg, sp = blockIdx.x / ncg;
  const int n0 = cg * COLS;

  // this wave's word rows: slice sp of S, part `wave` of GW
  const int nw = K / 8;
  const int per_sp = (nw + S - 1) / S;
  const int sp0 = sp * per_sp, sp1 = min(nw, sp0 + per_sp);
  const int per_w = (sp1 - sp0 + GW - 1) / GW;
  const int kw0 = min(sp1, sp0 + wave * per_w), kw1 = min(sp1, kw0 + per_w);
  // the table: all ng groups with act-order, else the slice's groups from g_lo
  const int g_lo = ACT ? 0 : (sp0 * 8) >> gsh;
  const int ngt = MODE == GLOBAL ? 0 : (ACT ? ng : (sp1 > sp0 ? (((sp1 * 8 - 1) >> gsh) - g_lo + 1) : 0));
  const DirectLds L(direct_table_groups(MODE, ng, per_sp, gsh), CPL, MT, per_sp);
  // GLOBAL: the table rows of this workgroup's columns (N*8 bytes per group)
  const __amdgpu_buffer_rsrc_t rt = make_rsrc(gtab, MODE == GLOBAL ? (uint32_t)ng * (uint32_t)N * 8u : 0u);
  int* goff = reinterpret_cast<int*>(lds + L.goff);
  float* xs = reinterpret_cast<float*>(lds + L.xs);
  float* red = reinterpret_cast<float*>(lds + L.red);  // [GW][MT][COLS]

  // N % 8 == 0, so a lane's CPL columns are all inside N or all past it
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qw, (uint32_t)nw * (uint32_t)N * 4u);
  const uint32_t loff = n0 + lane * CPL < N ? (uint32_t)(n0 + lane * CPL) * 4u : OOB;
  const uint32_t row_bytes = (uint32_t)N * 4u;

  // Set-up: every global load is issued before any is used, so the weight
  // rows (all of this wave's: at most KB), the table sources, the codes'
  // groups and the first rows of x share one memory latency.
  W wv[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) wv[j] = load_words<CPL>(rq, kw0 + j < kw1 ? loff + (uint32_t)(kw0 + j) * row_bytes : OOB);
  // table sources: chunk i = (group, 8 columns), a qzeros word and 8 scales
  constexpr int TC = 3;  // chunks per thread: ngt * COLS / 8 <= 3 * 64 * GW
  const int nchunk = ngt * (COLS / 8);
  const bool sc16 = ((uintptr_t)sc & 15) == 0;
  u32x4_t sv[TC];
  uint32_t zv[TC];
#pragma unroll
  for (int u = 0; u < TC; ++u) {
    const int i = t + u * 64 * GW;
    const int g = g_lo + i / (COLS / 8), n = n0 + 8 * (i % (COLS / 8));
    sv[u] = u32x4_t{0, 0, 0, 0};
    zv[u] = 0;
    if (i < nchunk && n < N) {
      zv[u] = qz[(long)g * (N / 8) + n / 8];
      const uint16_t* sp8 = sc + (long)g * N + n;
      if (sc16) {
        sv[u] = *reinterpret_cast<const u32x4_t*>(sp8);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[u][j] = (uint32_t)sp8[2 * j] | (uint32_t)sp8[2 * j + 1] << 16;
      }
    }
  }
  // the slice's codes (at most 8 KB = 2 per thread): their groups
  const int nk = (sp1 - sp0) * 8;
  int gv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = t + u * 64 * GW, k = sp0 * 8 + i;
    gv[u] = i < nk ? (ACT ? g_idx[k] : (k >> gsh) - g_lo) : 0;
  }
  // x rows m0 .. m0+MT-1 over the slice, in f16 pairs (MT per thread)
  auto load_x = [&](int m0, uint32_t (&xp)[MT]) {
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const int i = t + u * 64 * GW, m = i / (nk / 2), kk = 2 * (i % (nk / 2));
      xp[u] = 0;
      if (i < MT * (nk / 2) && m0 + m < M)
        xp[u] = *reinterpret_cast<const uint32_t*>(x + (long)(m0 + m) * K + sp0 * 8 + kk);
    }
  };
  auto store_x = [&](const uint32_t (&xp)[MT]) {
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      const int i = t + u * 64 * GW, m = i / (nk / 2), kk = 2 * (i % (nk / 2));
      if (i < MT * (nk / 2))
        *reinterpret_cast<float2*>(xs + m * per_sp * 8 + kk) =
            make_float2(f16_bits_to_f32(xp[u] & 0xFFFFu), f16_bits_to_f32(xp[u] >> 16));
    }
  };
  uint32_t xp[MT];
  load_x(0, xp);

  // LDS: the table, then the offsets and x
#pragma unroll
  for (int u = 0; u < TC; ++u) {
    const int i = t + u * 64 * GW;
    if (i < nchunk) {
      const int g = i / (COLS / 8), c8 = i % (COLS / 8);
      unsigned char* row = lds + L.tab + g * T::GBYTES;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float sj = f16_bits_to_f32(j & 1 ? sv[u][j >> 1] >> 16 : sv[u][j >> 1] & 0xFFFFu);
        const float z = (float)nib(zv[u], j) + 1.f;
        // exact: an 11-bit scale times a 5-bit integer (columns past N: 0, 0)
        *reinterpret_cast<float2*>(row + T::off(8 * c8 + j)) = make_float2(sj, -sj * z);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = t + u * 64 * GW;
    // the code's group row in the table (GLOBAL: byte offset of row g)
    if (i < nk) goff[i] = MODE == GLOBAL ? gv[u] * (N * 8) : gv[u] << GB_SHIFT;
  }
  store_x(xp);

  // this lane's first entry in a group row (GLOBAL: columns n0 + CPL*lane
  // onwards, or out of range past N)
  const int lane_off = MODE == GLOBAL ? (n0 + lane * CPL < N ? (n0 + lane * CPL) * 8 : (int)OOB)
                                      : L.tab + T::off(lane * CPL);
  // the nibble mask, hidden from the optimizer: knowing that each byte holds
  // 4 bits, it would turn the byte conversions below into bit-field
  // extracts plus a conversion
  uint32_t m4 = 0x0F0F0F0Fu;
  for (int m0 = 0; m0 < M; m0 += MT) {
    // (hidden again in every pass, which also keeps the compiler from
    // hoisting the unpacked codes of all rows out of the pass loop)
    asm volatile("" : "+s"(m4));
    if (m0 != 0) {
      load_x(m0, xp);
      __syncthreads();  // every wave done with the last pass's x and sums
      store_x(xp);
    }
    __syncthreads();
    float acc[MT][CPL];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[m][c] = 0.f;
    {
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int kw = kw0 + j;
        if (kw < kw1) {  // uniform
          const int r8 = (kw - sp0) * 8;  // the row's first code in the slice
          uint32_t lo[CPL], hi[CPL];
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const uint32_t w = word_of<CPL>(wv[j], c);
            lo[c] = w & m4;          // codes 0, 2, 4, 6 in bytes 0..3
            hi[c] = (w >> 4) & m4;   // codes 1, 3, 5, 7
          }
          const i32x4_t go0 = *reinterpret_cast<const i32x4_t*>(goff + r8);
          const i32x4_t go1 = *reinterpret_cast<const i32x4_t*>(goff + r8 + 4);
          f32x4_t xv[MT][2];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            xv[m][0] = *reinterpret_cast<const f32x4_t*>(xs + m * per_sp * 8 + r8);
            xv[m][1] = *reinterpret_cast<const f32x4_t*>(xs + m * per_sp * 8 + r8 + 4);
          }
          // all 8 codes' table reads first, so they are in flight together
          float sb[8][2 * CPL];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int go = e < 4 ? go0[e] : go1[e - 4];
            if constexpr (MODE == GLOBAL) {
              // CPL consecutive (scale, bias) pairs of row g: 8*CPL bytes.
              // A lane past N keeps an offset past the range (reads 0).
              const uint32_t o = lane_off == (int)OOB ? OOB : (uint32_t)go + (uint32_t)lane_off;
              if constexpr (CPL == 1) {
                const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rt, o, 0, 0));
                sb[e][0] = __uint_as_float(v.x);
                sb[e][1] = __uint_as_float(v.y);
              } else {
#pragma unroll
                for (int h = 0; h < CPL / 2; ++h) {
                  const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rt, o + 16 * h, 0, 0));
#pragma unroll
                  for (int i = 0; i < 4; ++i) sb[e][4 * h + i] = __uint_as_float(v[i]);
                }
              }
              continue;
            }
            const unsigned char* ent = lds + go + lane_off;
            if constexpr (CPL == 1) {
              const float2 v = *reinterpret_cast<const float2*>(ent);
              sb[e][0] = v.x;
              sb[e][1] = v.y;
            } else {
#pragma unroll
              for (int h = 0; h < CPL / 2; ++h) {
                const f32x4_t v = *reinterpret_cast<const f32x4_t*>(ent + h * 1024);
#pragma unroll
                for (int i = 0; i < 4; ++i) sb[e][4 * h + i] = v[i];
              }
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              const uint32_t src = (e & 1) ? hi[c] : lo[c];
              const float q = (float)(uint8_t)(src >> (8 * (e >> 1)));  // v_cvt_f32_ubyteN
              const float w = fmaf(sb[e][2 * c], q, sb[e][2 * c + 1]);
#pragma unroll
              for (int m = 0; m < MT; ++m) acc[m][c] = fmaf(xv[m][e >> 2][e & 3], w, acc[m][c]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // one row's reads at a time: bounded registers
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < CPL; ++c) red[(wave * MT + m) * COLS + lane * CPL + c] = acc[m][c];
    __syncthreads();
    for (int i = t; i < MT * COLS; i += 64 * GW) {
      const int m = i / COLS, c = i % COLS;
      if (m0 + m < M && n0 + c < N) {
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < GW; ++q) v += red[(q * MT + m) * COLS + c];
        part[((long)sp * M + m0 + m) * N + n0 + c] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Direct GPTQ on the matrix cores (M >= 8): v_mfma_f32_32x32x16_f16 with the
// weight split into exact fp16 pieces.  Per column n, with e_n the largest
// scale exponent of the column (fp16 biased exponent E_n, e_n = E_n - 15):
//     W[n,k] = 2^e_n * (p_hi + p_lo) * d,   d = q - (z + 1) in [-16, 14]
// where p_hi + p_lo = scale * 2^-e_n, p_hi its top 6 significant bits and
// p_lo the rest (5 bits).  Each piece times d has at most 11 significant
// bits, so both B operands are exact in fp16 (for scales within 2^14 of the
// column's largest; smaller ones round below 2^-24 of it); x is fp16 as
// given, products and sums are fp32 in the MFMA, and y = 2^e_n * acc.
// The per-(group, column) entry (p_hi, p_lo, -(1024 + z + 1)) sits in an LDS
// table; d comes from the code with the exponent-bias trick:
// (code | 0x6400) is 1024 + code in fp16.
// Workgroup: 4 waves x 32 columns, one K slice; lane (l32, half) takes, in
// 16-code step j, word row 2j + half of the slice: its 8 codes are the
// lane's B fragment, ordered (c0,c4,c1,c5,c2,c6,c3,c7) by the decode, and
// its A fragment is x of the same 8 codes, permuted to match.
constexpr int MG_COLS = 128;

__device__ __forceinline__ uint32_t pair_lo16(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi16(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

struct MfmaLds {
  int tab, emax, goff, total;
  __host__ __device__ MfmaLds(int ng, int per_sp) {
    tab = 0;
    emax = ng * MG_COLS * 8;
    goff = emax + MG_COLS * 4;
    total = goff + per_sp * 8 * 4;
  }
};

template <int MB, bool ACT>
__global__ __launch_bounds__(256) void gptq_mfma_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint32_t* __restrict__ qz,
    const uint16_t* __restrict__ sc, const int32_t* __restrict__ g_idx, float* __restrict__ part,
    uint16_t* __restrict__ y, int M, int N, int K, int gsh, int S, int per_sp) {
  // per_sp: word rows per slice, even (whole 16-code steps)
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int ng = K >> gsh;
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int ncg = (N + MG_COLS - 1) / MG_COLS;
  const int cg = blockIdx.x % ncg, sp = blockIdx.x / ncg;
  const int n0 = cg * MG_COLS;
  const int nw = K / 8;
  const int sp0 = min(nw, sp * per_sp), sp1 = min(nw, sp0 + per_sp);
  const int nsteps = (sp1 - sp0) / 2;
  // the table: all ng groups with act-order, else the slice's groups from
  // g_lo (the largest exponent is then the slice's own, which the partial
  // carries: acc is scaled by it before the slices are added)
  const int g_lo = ACT ? 0 : (sp0 * 8) >> gsh;
  const int ngt = ACT ? ng : (sp1 > sp0 ? (((sp1 * 8 - 1) >> gsh) - g_lo + 1) : 0);
  const MfmaLds L(table_groups(ACT, ng, per_sp, gsh), per_sp);
  int* emax = reinterpret_cast<int*>(lds + L.emax);
  int* goff = reinterpret_cast<int*>(lds + L.goff);

  // ---- table: largest exponent per column, then the entries
  for (int i = t; i < MG_COLS; i += 256) emax[i] = 0;
  __syncthreads();
  const int nchunk = ngt * (MG_COLS / 8);
  for (int i = t; i < nchunk; i += 256) {
    const int g = g_lo + i / (MG_COLS / 8), c8 = i % (MG_COLS / 8), n = n0 + 8 * c8;
    if (n < N) {
#pragma unroll
      for (int j = 0; j < 8; ++j) atomicMax(&emax[8 * c8 + j], (int)((sc[(long)g * N + n + j] >> 10) & 31));
    }
  }
  __syncthreads();
  for (int i = t; i < nchunk; i += 256) {
    const int g = g_lo + i / (MG_COLS / 8), c8 = i % (MG_COLS / 8), n = n0 + 8 * c8;
    uint2* row = reinterpret_cast<uint2*>(lds + L.tab + (g - g_lo) * MG_COLS * 8) + 8 * c8;
    if (n < N) {
      const uint32_t zw = qz[(long)g * (N / 8) + n / 8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pv = ldexpf(f16_bits_to_f32(sc[(long)g * N + n + j]), 15 - emax[8 * c8 + j]);  // exact
        const float ph = __uint_as_float(__float_as_uint(pv) & 0xFFFC0000u);  // top 6 significant bits
        const float pl = pv - ph;                                              // exact: the other 5
        const uint32_t hl = (uint32_t)f32_to_f16_bits(ph) | (uint32_t)f32_to_f16_bits(pl) << 16;
        const uint32_t no = f32_to_f16_bits(-1024.f - ((float)nib(zw, j) + 1.f));
        row[j] = make_uint2(hl, no);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) row[j] = make_uint2(0u, 0u);
    }
  }
  const int nk = (sp1 - sp0) * 8;
  for (int i = t; i < nk; i += 256) {
    const int k = sp0 * 8 + i;
    goff[i] = (ACT ? g_idx[k] : (k >> gsh) - g_lo) * (MG_COLS * 8);
  }
  __syncthreads();

  const int cl = 32 * wave + l32;  // this lane's column in the workgroup
  const int n = n0 + cl;
  const int e_n = emax[cl] - 15;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qw, (uint32_t)nw * (uint32_t)N * 4u);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const uint32_t woff = n < N ? (uint32_t)n * 4u : OOB;
  const unsigned char* tcol = lds + L.tab + cl * 8;

  for (int m0 = 0; m0 < M; m0 += MB * 32) {
    f32x16_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
    uint32_t xoff[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + mb * 32 + l32;
      xoff[mb] = m < M ? (uint32_t)m * (uint32_t)K * 2u : OOB;
    }
    auto load = [&](int j, uint32_t& wd, u32x4_t (&a)[MB]) {
      const int kw = sp0 + 2 * min(j, nsteps - 1) + half;
      wd = __builtin_amdgcn_raw_buffer_load_b32(rq, woff + (uint32_t)kw * (uint32_t)N * 4u, 0, 0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        a[mb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[mb] + (uint32_t)kw * 16u, 0, 0));
    };
    // LDS side: a step's table offsets are read two steps ahead and its
    // entries one step ahead, so no step waits on the offset -> entry chain
    auto read_goff = [&](int j, i32x4_t (&g)[2]) {
      const int r8 = (2 * min(j, nsteps - 1) + half) * 8;
      g[0] = *reinterpret_cast<const i32x4_t*>(goff + r8);
      g[1] = *reinterpret_cast<const i32x4_t*>(goff + r8 + 4);
    };
    auto read_ent = [&](const i32x4_t (&g)[2], uint2 (&en)[8]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) en[e] = *reinterpret_cast<const uint2*>(tcol + g[e >> 2][e & 3]);
    };
    // One 16-code step: weight words and x fragments were loaded two steps
    // before (global), the table entries one step before (LDS); it loads
    // step j+2 into the buffers it frees, reads the entries of step j+1 and
    // the offsets of step j+2.  The loop is unrolled by two so the two sets
    // of buffers alternate without copies.
    uint32_t magic = 0x64006400u;
    asm volatile("" : "+v"(magic));
    i32x4_t gn[2];  // table offsets of the step after the next
    auto step = [&](int j, uint32_t& wd, u32x4_t (&a)[MB], uint2 (&ent)[8], uint2 (&en)[8]) {
      const uint32_t w = wd;
      u32x4_t ax[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) ax[mb] = a[mb];
      load(j + 2, wd, a);    // two steps ahead (clamped past the end; unused)
      read_ent(gn, en);      // step j+1
      read_goff(j + 2, gn);  // step j+2 (the read of gn above is issued first)
      u32x4_t bh, bl;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        // 1024 + (c_p, c_p+4) in fp16: one v_and_or_b32 with the constant in a VGPR
        const f16x2_t cp = __builtin_bit_cast(f16x2_t, ((w >> (4 * p)) & 0x000F000Fu) | magic);
        const f16x2_t d = cp + __builtin_bit_cast(f16x2_t, pair_lo16(ent[p].y, ent[p + 4].y));  // q - (z+1), exact
        bh[p] = __builtin_bit_cast(uint32_t, d * __builtin_bit_cast(f16x2_t, pair_lo16(ent[p].x, ent[p + 4].x)));
        bl[p] = __builtin_bit_cast(uint32_t, d * __builtin_bit_cast(f16x2_t, pair_hi16(ent[p].x, ent[p + 4].x)));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        // x of codes (0,4),(1,5),(2,6),(3,7)
        const u32x4_t ap = {pair_lo16(ax[mb][0], ax[mb][2]), pair_hi16(ax[mb][0], ax[mb][2]),
                            pair_lo16(ax[mb][1], ax[mb][3]), pair_hi16(ax[mb][1], ax[mb][3])};
        const f16x8_t af = __builtin_bit_cast(f16x8_t, ap);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, __builtin_bit_cast(f16x8_t, bh), acc[mb], 0, 0, 0);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, __builtin_bit_cast(f16x8_t, bl), acc[mb], 0, 0, 0);
      }
    };
    uint32_t wd0, wd1;
    u32x4_t a0[MB], a1[MB];
    load(0, wd0, a0);
    load(1, wd1, a1);
    uint2 e0[8], e1[8];
    {
      i32x4_t gc[2];
      read_goff(0, gc);
      read_ent(gc, e0);
    }
    read_goff(1, gn);
    int j = 0;
    for (; j + 1 < nsteps; j += 2) {
      step(j, wd0, a0, e0, e1);
      step(j + 1, wd1, a1, e1, e0);
    }
    if (j < nsteps) step(j, wd0, a0, e0, e1);
    // accumulator layout: lane -> column l32, register r -> row 8*(r/4) + 4*half + r%4
    if (n < N) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (m < M) {
            const float v = ldexpf(acc[mb][r], e_n);
            if (S > 1)
              part[((long)sp * M + m) * N + n] = v;
            else
              y[(long)m * N + n] = f32_to_f16_bits(v);
          }
        }
    }
  }
}

// y[m, n] = f16(sum over the S slices)
// The GLOBAL-mode table: tab[g][n] = (scale, -scale*(z+1)) in fp32 (exact:
// an 11-bit scale times an integer in [1, 16]).
__global__ __launch_bounds__(256) void gptq_table_kernel(const uint32_t* __restrict__ qz,
                                                         const uint16_t* __restrict__ sc, float2* __restrict__ tab,
                                                         int N, int ng) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)ng * N) return;
  const int g = (int)(i / N), n = (int)(i % N);
  const float s = f16_bits_to_f32(sc[i]);
  const float z = (float)nib(qz[(long)g * (N / 8) + n / 8], n % 8) + 1.f;
  tab[i] = make_float2(s, -s * z);
}

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

// The dynamic LDS limit of kernel k raised once per device (flags `once`),
// to the most any launch of it asks for.
inline hipError_t raise_lds_limit(const void* k, std::once_flag (&once)[64]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::call_once(once[dev], [&] { e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds); });
  return e;
}

// K slices of a split-K launch over ncg column groups: as many as the
// workgroups the device holds at once allow (`resident`), so that the grid
// runs in one round: a grid just past that leaves its last workgroups
// running alone, for as long again.  Each slice keeps at least min_rows word
// rows (the per-workgroup set-up would otherwise dominate), and there are
// never fewer than s_min slices.
inline int64_t fill_slices(int64_t resident, int64_t ncg, int64_t nw, int64_t min_rows, int64_t s_min) {
  return std::max(s_min, std::min(resident / ncg, nw / min_rows));
}

template <int CPL, int MT, int MODE>
hipError_t run_direct(const GptqArgs& a, hipStream_t s) {
  const auto k = reinterpret_cast<const void*>(gptq_direct_kernel<CPL, MT, MODE>);
  constexpr int block = 64 * direct_waves<MT>();
  static std::once_flag once[64];
  hipError_t e = raise_lds_limit(k, once);
  if (e != hipSuccess) return e;
  const int ng = (int)(a.K / a.G);
  const int64_t ncg = (a.N + 64 * CPL - 1) / (64 * CPL), nw = a.K / 8;
  // fewest slices: a wave holds all its word rows, so a slice has at most
  // WROWS; more when the slice's staged x and offsets would not fit in LDS
  auto lds_of = [&](int64_t S) {
    const int per_sp = (int)((nw + S - 1) / S);
    return DirectLds(direct_table_groups(MODE, ng, per_sp, a.G == 32 ? 5 : (a.G == 64 ? 6 : 7)), CPL, MT, per_sp).total;
  };
  int64_t s_min = std::max<int64_t>(1, (nw + WROWS - 1) / WROWS);
  while (lds_of(s_min) > kMaxLds) {
    if (s_min >= nw) return hipErrorNotSupported;
    ++s_min;
  }
  int64_t resident = 0;
  // (at most 16 waves per CU: two 8-wave workgroups or one of 16; two of
  // 16 measured slower)
  e = resident_workgroups(k, block, (size_t)lds_of(s_min), 16 / direct_waves<MT>(), &resident);
  if (e != hipSuccess) return e;
  int64_t S = fill_slices(resident, ncg, nw, 32, s_min);
  const int per_sp = (int)((nw + S - 1) / S);
  S = (nw + per_sp - 1) / per_sp;  // no empty slice
  // (the kernel derives the same per_sp from S; more slices only shrink the LDS)
  const size_t lds = (size_t)lds_of(S);
  const int64_t MN = a.M * a.N;
  // workspace: the S partial planes, then (GLOBAL) the group table
  const size_t part_bytes = ((size_t)S * MN * sizeof(float) + 255) & ~size_t(255);
  const size_t tab_bytes = MODE == GLOBAL ? (size_t)ng * a.N * 8 : 0;
  char* ws = nullptr;
  e = stream_workspace(s, part_bytes + tab_bytes, (void**)&ws);
  if (e != hipSuccess) return e;
  float* part = reinterpret_cast<float*>(ws);
  float2* gtab = MODE == GLOBAL ? reinterpret_cast<float2*>(ws + part_bytes) : nullptr;
  if (MODE == GLOBAL) {
    const long ne = (long)ng * a.N;
    hipLaunchKernelGGL(gptq_table_kernel, dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, s,
                       (const uint32_t*)a.qzeros, (const uint16_t*)a.scales, gtab, (int)a.N, ng);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gptq_direct_kernel<CPL, MT, MODE>), dim3((unsigned)(ncg * S)), dim3(block), lds, s,
                     (const uint16_t*)a.x, (const uint32_t*)a.qweight, (const uint32_t*)a.qzeros,
                     (const uint16_t*)a.scales, a.g_idx, (const float2*)gtab, part, (int)a.M, (int)a.N, (int)a.K,
                     a.G == 32 ? 5 : (a.G == 64 ? 6 : 7), (int)S);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gptq_finalize_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, part,
                     (uint16_t*)a.y, (long)MN, (int)S);
  return hipGetLastError();
}

template <int CPL, int MODE>
hipError_t run_direct_mode(const GptqArgs& a, int mt, hipStream_t s) {
  constexpr int MT8 = CPL == 4 ? 4 : 8;  // (8 rows per pass only below 4 columns per lane)
  if (mt == 1) return run_direct<CPL, 1, MODE>(a, s);
  if (mt == 2) return run_direct<CPL, 2, MODE>(a, s);
  if (mt == 4) return run_direct<CPL, 4, MODE>(a, s);
  return run_direct<CPL, MT8, MODE>(a, s);
}

template <int CPL>
hipError_t run_direct_m(const GptqArgs& a, int mt, hipStream_t s) {
  if (a.g_idx) return run_direct_mode<CPL, LDS>(a, mt, s);
  return run_direct_mode<CPL, SLICE>(a, mt, s);
}

// M >= 8 with at most 96 groups: the matrix-core kernel, K split to fill
// the CUs (two workgroups each, LDS allowing, so that one's waits overlap the
// other's work; each slice 64 to 256 word rows, an even count), partials
// summed by the finalize kernel
template <int MB, bool ACT>
hipError_t run_mfma(const GptqArgs& a, hipStream_t s) {
  const auto k = reinterpret_cast<const void*>(gptq_mfma_kernel<MB, ACT>);
  static std::once_flag once[64];
  hipError_t e = raise_lds_limit(k, once);
  if (e != hipSuccess) return e;
  const int ng = (int)(a.K / a.G);
  const int64_t nw = a.K / 8, ncg = (a.N + MG_COLS - 1) / MG_COLS;
  const int gsh = a.G == 32 ? 5 : (a.G == 64 ? 6 : 7);
  auto lds_of = [&](int per_sp) { return MfmaLds(table_groups(ACT, ng, per_sp, gsh), per_sp).total; };
  const int64_t s_min = std::max<int64_t>(1, (nw + 255) / 256);
  const int per_min = (int)(((nw + s_min - 1) / s_min + 1) & ~int64_t(1));
  if (lds_of(per_min) > kMaxLds) return hipErrorNotSupported;
  int64_t resident = 0;
  e = resident_workgroups(k, 256, (size_t)lds_of(per_min), 2, &resident);
  if (e != hipSuccess) return e;
  int64_t S = fill_slices(resident, ncg, nw, 64, s_min);
  const int per_sp = (int)(((nw + S - 1) / S + 1) & ~int64_t(1));
  S = (nw + per_sp - 1) / per_sp;  // no empty slice
  const size_t lds = (size_t)lds_of(per_sp);
  const int64_t MN = a.M * a.N;
  float* part = nullptr;
  if (S > 1) {
    e = stream_workspace(s, (size_t)S * MN * sizeof(float), (void**)&part);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gptq_mfma_kernel<MB, ACT>), dim3((unsigned)(ncg * S)), dim3(256), lds, s, (const uint16_t*)a.x,
                     (const uint32_t*)a.qweight, (const uint32_t*)a.qzeros, (const uint16_t*)a.scales, a.g_idx, part,
                     (uint16_t*)a.y, (int)a.M, (int)a.N, (int)a.K, a.G == 32 ? 5 : (a.G == 64 ? 6 : 7), (int)S,
                     per_sp);
  e = hipGetLastError();
  if (e == hipSuccess && S > 1) {
    hipLaunchKernelGGL(gptq_finalize_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, part,
                       (uint16_t*)a.y, (long)MN, (int)S);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_gptq_mfma(const GptqArgs& a, hipStream_t s) {
  const bool mb1 = a.M <= 32;
  if (a.g_idx) return mb1 ? run_mfma<1, true>(a, s) : run_mfma<2, true>(a, s);
  return mb1 ? run_mfma<1, false>(a, s) : run_mfma<2, false>(a, s);
}

hipError_t launch_gptq_direct(const GptqArgs& a, hipStream_t s) {
  const int64_t ng = a.K / a.G;
  // (without act-order a workgroup's table holds only its slice's groups)
  if (a.M >= 8 && (!a.g_idx || ng <= 96) && a.K / 8 * a.N * 4 < (int64_t(1) << 31) &&
      a.M * a.K * 2 < (int64_t(1) << 31))
    return launch_gptq_mfma(a, s);
  // columns per lane: 4 when the (scale, bias) table of 256 columns fits
  // 64 KiB of LDS, else 2, else 1 (up to 96 KiB).  Without act-order the
  // table holds only a slice's groups, so 4 always.
  const int cpl = !a.g_idx || ng <= 32 ? 4 : (ng <= 64 ? 2 : 1);
  if (a.K / 8 * a.N * 4 >= (int64_t(1) << 31)) return hipErrorNotSupported;  // 32-bit buffer offsets
  if (a.g_idx && ng * 64 * cpl * 8 > 96 * 1024) {
    // act-order with more groups than the LDS table holds (above 192): the
    // entries come from a device-memory table, 4 columns per lane
    if (ng * a.N * 8 >= (int64_t(1) << 31)) return hipErrorNotSupported;  // 32-bit table offsets
    const int mt = a.M == 1 ? 1 : (a.M == 2 ? 2 : 4);
    return run_direct_mode<4, GLOBAL>(a, mt, s);
  }
  // x rows per pass (8 would spill registers at 4 columns per lane)
  const int mt = a.M == 1 ? 1 : (a.M == 2 ? 2 : (a.M <= 4 || cpl == 4 ? 4 : 8));
  return cpl == 4 ? run_direct_m<4>(a, mt, s) : (cpl == 2 ? run_direct_m<2>(a, mt, s) : run_direct_m<1>(a, mt, s));
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
