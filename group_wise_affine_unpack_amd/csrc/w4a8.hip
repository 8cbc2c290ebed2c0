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
//   quant : each row held in the registers of one to four waves (16-byte
//           loads, 8-byte stores) for K <= 16384, else one row per block
//           in a loop; bit-exact codes and scale.
//   gemv  : M <= 16: one wave per output column, v_dot4_i32_i8 on decoded
//           codes, exact int32 wave sums.
//   gemm  : v_mfma_i32_32x32x32_i8, tile BM x BN (4 waves along N, each
//           BM x NB*32), K in stages of 128: x_q through a 4-stage LDS ring
//           stored two stages ahead; int4 words in batches of two stages
//           (8 rows x 128 bytes per load instruction, whole lines), two
//           batches in flight in registers, then through a wave-private LDS
//           region into the B fragment's shape, decoded in registers; the tile shrinks until the
//           grid gives every CU two workgroups, and when even the smallest
//           tile leaves CUs idle K is split over workgroups (int32 partials,
//           summed exactly by a second kernel).  A nibble
//           is placed in the HIGH half of its byte, which makes the byte the
//           int8 value 16*v with no sign extension step; the accumulator is
//           shifted right by 4 at the end (exact: every product is a multiple
//           of 16, and |acc| * 16 < 2^31 for K <= 2^17).
#include <algorithm>

#include "common.h"

namespace qaff {
namespace {

// One row per block, for any K.
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

// x / s rounded to nearest even, from r = 1/s refined by one Newton step:
// q0 = x r, then the residual x - s q0 (exact in an fma) corrects q0 to the
// rounded quotient (Markstein's division).  For s = a/127 over every finite
// f16 a and every f16 x with |x| <= a it equals the IEEE quotient bit for
// bit (an exhaustive test holds it to that), so rint of it gives the same
// code as rint(x / s).  s = r = 0 (an all-zero row) gives 0.  The code
// comes back as an exact float in [1, 255], biased by 128.
__device__ __forceinline__ float quant_biased(uint32_t h, float s, float r) {
  const float v = f16_bits_to_f32(h);
  const float q0 = v * r;
  const float q = __builtin_fmaf(__builtin_fmaf(-s, q0, v), r, q0);
  return __builtin_amdgcn_fmed3f(rintf(q), -127.f, 127.f) + 128.f;
}

// four f16 values (two words) -> four int8 codes in one word
__device__ __forceinline__ uint32_t quant_word(uint32_t w0, uint32_t w1, float s, float r) {
  uint32_t o = __builtin_amdgcn_cvt_pk_u8_f32(quant_biased(w0 & 0xFFFFu, s, r), 0, 0u);
  o = __builtin_amdgcn_cvt_pk_u8_f32(quant_biased(w0 >> 16, s, r), 1, o);
  o = __builtin_amdgcn_cvt_pk_u8_f32(quant_biased(w1 & 0xFFFFu, s, r), 2, o);
  o = __builtin_amdgcn_cvt_pk_u8_f32(quant_biased(w1 >> 16, s, r), 3, o);
  return o ^ 0x80808080u;  // code + 128 -> two's complement byte
}

// One row per WPR waves (a block of four waves holds 4/WPR rows), the row
// held in registers: thread i of the row takes the 8-value chunks
// i, i + 64 WPR, ... (R of them, K <= 512 WPR R), read once with 16-byte
// loads and written as 8 bytes each.  x and x_q 16-byte aligned, K % 8 == 0.
template <int WPR, int R>
__global__ __launch_bounds__(256) void w4a8_quant_rows_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                              int8_t* __restrict__ xq, float* __restrict__ sx) {
  constexpr int TPR = 64 * WPR;  // threads per row
  const int m = blockIdx.x * (4 / WPR) + (int)threadIdx.x / TPR, i = (int)threadIdx.x % TPR;
  const int C = K >> 3;
  const u32x4_t* row = reinterpret_cast<const u32x4_t*>(x + (long)min(m, M - 1) * K);
  u32x4_t v[R];
#pragma unroll
  for (int j = 0; j < R; ++j) v[j] = i + TPR * j < C ? row[i + TPR * j] : u32x4_t{0, 0, 0, 0};
  // |x| by clearing the sign bits, two values at a time; maxNum lets a NaN
  // take no part in the maximum (as in a max built from ">" compares)
  f16x2_t am2 = {0, 0};
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      am2 = __builtin_elementwise_max(am2, __builtin_bit_cast(f16x2_t, v[j][e] & 0x7FFF7FFFu));
  float am = fmaxf((float)am2[0], (float)am2[1]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
  if constexpr (WPR > 1) {
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
    __syncthreads();
    const int w0 = ((int)threadIdx.x >> 6) & ~(WPR - 1);
#pragma unroll
    for (int w = 0; w < WPR; ++w) am = fmaxf(am, red[w0 + w]);
  }
  if (m >= M) return;
  const float s = am / 127.0f;  // correctly rounded division (HIP default)
  if (i == 0) sx[m] = s;
  float r = 0.f;
  if (am != 0.f) {
    const float r0 = __builtin_amdgcn_rcpf(s);
    r = __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
  }
  u32x2_t* qrow = reinterpret_cast<u32x2_t*>(xq + (long)m * K);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (i + TPR * j >= C) break;
    qrow[i + TPR * j] = u32x2_t{quant_word(v[j][0], v[j][1], s, r), quant_word(v[j][2], v[j][3], s, r)};
  }
}

constexpr uint32_t OOB = 0x80000000u;  // a buffer offset past any range: the load reads 0

__device__ __forceinline__ u32x4_t ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

constexpr int BK = 128;  // int8 codes per K stage

struct Params {
  const int8_t* xq;
  const float* sx;
  const uint16_t* x;   // staged lowering: the f16 activations
  int8_t* xq_out;      // staged lowering: x_q and s_x, written by the
  float* sx_out;       //   workgroups of the first column tile
  const uint32_t* w;
  const uint16_t* sw;
  uint16_t* y;
  int32_t* acc_out;
  int M, N, K;
  int Tm, Tn, per_xcd;
  int S, per_split;  // K splits of per_split stages; S > 1 writes int32 partials [S][M][N]
  int32_t* part;
};

// 8 nibbles of one word -> 8 int8 (16*v) in natural k order (2 dwords)
__device__ __forceinline__ void decode_word(uint32_t w, uint32_t& d0, uint32_t& d1) {
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u;  // nibbles 0,2,4,6 in the byte high halves
  const uint32_t hi = w & 0xF0F0F0F0u;         // nibbles 1,3,5,7
  d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // (n0, n1, n2, n3)
  d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // (n4, n5, n6, n7)
}

__device__ __forceinline__ int xswz(int r) { return r & 7; }

// One wave: rows [0, MB*32) x columns [wave*NB*32, +NB*32) of the tile.
// Stage = 128 codes of K.  Lane (l32, h) takes, in 16-column sub-step s,
// codes 64h + 16s .. +15 of the stage: its B fragment is words 8h+2s, 8h+2s+1
// of its row, its A fragment the matching 16 bytes of x_q row l32.
template <int MB, int NB, bool STAGED>
struct W4Pipe {
  // 16-byte x chunks per thread and stage: x_q codes, or (staged) f16
  // values, 8 per chunk, quantized on their way into LDS
  static constexpr int A_CH = STAGED ? 2 * MB : MB;
  static constexpr int SB = MB * 32 * 128;  // bytes of one LDS stage
  __amdgpu_buffer_rsrc_t rx, rw, rq;
  uint32_t x_off[A_CH];  // this thread's chunks (OOB for rows past M)
  int x_dst;             // LDS offset of chunk 0 (chunk i at + i*4096; staged + i*2048)
  // staged: the scale and refined reciprocal of each chunk's row, and
  // whether this workgroup writes x_q (the first column tile does)
  float qs[A_CH], qr[A_CH];
  uint32_t q_off[A_CH];  // x_q byte offset of the chunk's first code, stage 0
  int q_col;             // the chunk's first code within a stage
  bool wq;
  // weight batches (two stages = 128 bytes of a row): global loads of 8
  // rows x 128 bytes per instruction, through a wave-private LDS region
  static constexpr int WB = NB * 4;  // 16-byte chunks per lane and batch
  uint32_t wb_off[WB];               // row 8i + lane/8 of the wave's rows, chunk lane%8 (OOB past N)
  int wb_dst[WB];                    // its LDS place (chunks XOR-swizzled by row)
  unsigned char* wreg;               // this wave's region: NB*32 rows x 128 bytes
  int l32, h, nst, K;
  int st0;  // first K stage of this workgroup's split

  __device__ __forceinline__ void issue_x(int t, u32x4_t (&xr)[A_CH]) const {
    const uint32_t k = (uint32_t)(st0 + min(t, nst - 1)) * BK * (STAGED ? 2 : 1);
#pragma unroll
    for (int i = 0; i < A_CH; ++i) xr[i] = ld128(rx, x_off[i] + k);
  }
  // x of stage t into an LDS stage; staged: quantized first (the same
  // arithmetic as the quantize kernel, so the same bits), and the first
  // column tile's workgroups also store the codes to x_q (a chunk past K
  // is not stored; a row past M is past the range)
  __device__ __forceinline__ void store_x(unsigned char* st, const u32x4_t (&xr)[A_CH], int t) const {
    if constexpr (STAGED) {
      const int k0 = (st0 + min(t, nst - 1)) * BK;
#pragma unroll
      for (int i = 0; i < A_CH; ++i) {
        const u32x2_t c{quant_word(xr[i][0], xr[i][1], qs[i], qr[i]), quant_word(xr[i][2], xr[i][3], qs[i], qr[i])};
        *reinterpret_cast<u32x2_t*>(st + x_dst + i * 2048) = c;
        if (wq && k0 + q_col < K)
          __builtin_amdgcn_raw_buffer_store_b64(c, rq, q_off[i] + (uint32_t)k0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_CH; ++i) *reinterpret_cast<u32x4_t*>(st + x_dst + i * 4096) = xr[i];
    }
  }
  // batch j (local stages 2j, 2j+1): a chunk whose codes start at or past K
  // reads zeros (K % 32 == 0, so a chunk is wholly inside or outside)
  __device__ __forceinline__ void issue_wb(int j, u32x4_t (&wb)[WB]) const {
    const int byte0 = (st0 + 2 * j) * (BK / 2) + (l32 & 7) * 16;  // lane%8 == l32%8
    const uint32_t o = 2 * byte0 < K ? 0u : OOB;
#pragma unroll
    for (int i = 0; i < WB; ++i) wb[i] = ld128(rw, (wb_off[i] | o) + (uint32_t)byte0);
  }
  __device__ __forceinline__ void put_wb(const u32x4_t (&wb)[WB]) const {
#pragma unroll
    for (int i = 0; i < WB; ++i) *reinterpret_cast<u32x4_t*>(wreg + wb_dst[i]) = wb[i];
  }
  static __device__ __forceinline__ int wswz(int r) { return (r >> 1) & 7; }
  // the weight words of stage u (0, 1) of the batch in LDS, in the B
  // fragment's shape: lane (l32, h), block nb takes bytes 64u + 32h .. +31
  // of row nb*32 + l32
  __device__ __forceinline__ void read_w(int u, u32x4_t (&wr)[NB][2]) const {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int r = nb * 32 + l32;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        wr[nb][j] = *reinterpret_cast<const u32x4_t*>(wreg + r * 128 + (((4 * u + 2 * h + j) ^ wswz(r)) << 4));
    }
  }
  __device__ __forceinline__ void read_a(const unsigned char* __restrict__ st, int s, i32x4_t (&af)[MB]) const {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = mb * 32 + l32;
      af[mb] = *reinterpret_cast<const i32x4_t*>(st + r * 128 + (((4 * h + s) ^ xswz(r)) << 4));
    }
  }
  __device__ __forceinline__ void decode_b(const u32x4_t (&wr)[NB][2], int s, i32x4_t (&bf)[NB]) const {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t w0 = wr[nb][s >> 1][2 * (s & 1)], w1 = wr[nb][s >> 1][2 * (s & 1) + 1];
      uint32_t d0, d1, d2, d3;
      decode_word(w0, d0, d1);
      decode_word(w1, d2, d3);
      bf[nb] = i32x4_t{(int)d0, (int)d1, (int)d2, (int)d3};
    }
  }
  __device__ __forceinline__ void mfma(const i32x4_t (&af)[MB], const i32x4_t (&bf)[NB],
                                       i32x16_t (&acc)[MB][NB]) const {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
  }
  // The four 32-code sub-steps of a stage, software-pipelined: sub-step s
  // runs its MFMAs while s+1's A fragments are read and B fragments decoded.
  // a0/b0 hold sub-step 0 of this stage on entry and of the next stage
  // (LDS stage stn, ring entry wn) on exit.
  __device__ __forceinline__ void compute(const unsigned char* __restrict__ st, const u32x4_t (&wr)[NB][2],
                                          const unsigned char* __restrict__ stn, const u32x4_t (&wn)[NB][2],
                                          i32x4_t (&a0)[MB], i32x4_t (&b0)[NB], i32x16_t (&acc)[MB][NB]) const {
    i32x4_t a1[MB], b1[NB];
    read_a(st, 1, a1);
    decode_b(wr, 1, b1);
    mfma(a0, b0, acc);
    __builtin_amdgcn_sched_barrier(0);
    read_a(st, 2, a0);
    decode_b(wr, 2, b0);
    mfma(a1, b1, acc);
    __builtin_amdgcn_sched_barrier(0);
    read_a(st, 3, a1);
    decode_b(wr, 3, b1);
    mfma(a0, b0, acc);
    __builtin_amdgcn_sched_barrier(0);
    read_a(stn, 0, a0);
    decode_b(wn, 0, b0);
    mfma(a1, b1, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Stage t (LDS stage t%4 = S):
  //   barrier              stage t+1 of x (stored last step) visible; every
  //                        wave done with stage t-1
  //   store x of t+2       registers loaded last step -> stage (t+2)%4
  //   issue x of t+3
  //   t odd: weight batch (t+1)/2 (stages t+1, t+2) from its register slot
  //          into the wave's LDS region (the wave read the previous batch's
  //          last stage one step ago), then batch (t+1)/2 + 2 into the slot
  //   read stage t+1's weight words from LDS
  //   compute t            ending with sub-step 0 of stage t+1 prepared
  //                        (skipped past the last stage)
  template <int S>
  __device__ __forceinline__ void step(int t, unsigned char* lds, u32x4_t (&xr)[A_CH], u32x4_t (&wb)[WB],
                                       const u32x4_t (&cur)[NB][2], u32x4_t (&nxt)[NB][2], i32x4_t (&a0)[MB],
                                       i32x4_t (&b0)[NB], i32x16_t (&acc)[MB][NB]) const {
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0): own LDS writes done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    store_x(lds + ((S + 2) & 3) * SB, xr, t + 2);
    issue_x(t + 3, xr);
    if constexpr (S & 1) {
      put_wb(wb);
      issue_wb((t + 1) / 2 + 2, wb);
    }
    read_w((t + 1) & 1, nxt);
    __builtin_amdgcn_sched_barrier(0);
    if (t < nst) compute(lds + S * SB, cur, lds + ((S + 1) & 3) * SB, nxt, a0, b0, acc);
  }
};

// x_q tiles go global -> registers (one stage before the store) -> a 4-stage
// LDS ring, stored two stages before use, 16-byte chunks XOR-swizzled by row;
// int4 words go in two-stage batches to registers (two batches in flight)
// and then to the wave's LDS region one step before their first stage;
// loads past the end of K or past the last row are out of range and read
// zeros.  The A reads and B decode of a stage's first sub-step run during
// the previous stage's last one.
template <int MB, int NB, bool STAGED>
__global__ __launch_bounds__(256) void w4a8_gemm_kernel(Params p) {
  constexpr int BM = MB * 32;
  constexpr int BN = NB * 128;
  const int b = blockIdx.x;
  const int vs = (b & 7) * p.per_xcd + (b >> 3);
  if (vs >= p.Tm * p.Tn * p.S) return;
  const int v = vs / p.S, sp = vs % p.S;
  const int tm = v / p.Tn, tn = v % p.Tn;
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l32 = lane & 31, h = lane >> 5;

  using PIPE = W4Pipe<MB, NB, STAGED>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * PIPE::SB + 4 * NB * 32 * 128];
  __shared__ float qsh[STAGED ? 2 * BM : 1];  // staged: per row of the tile, s then r

  i32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  PIPE P;
  P.l32 = l32;
  P.h = h;
  {
    const int nst_all = (p.K + BK - 1) / BK;
    P.st0 = sp * p.per_split;
    P.nst = min(nst_all - P.st0, p.per_split);
  }
  // the range covers the tile's rows: a row past M reads zeros.  x_q chunks
  // past K (last stage, K % 128 != 0) read the next row; the weight words
  // they meet are zeros (see issue_w), so they add nothing.
  P.rw = make_rsrc(p.w, (uint32_t)((long)p.N * p.K / 2));
  if constexpr (STAGED) {
    // f16 rows of the tile; thread t takes row t/16 (+ 16 i), 8-value chunk
    // t%16 of each 128-value stage: 8 codes, half of a 16-byte LDS chunk
    P.rx = make_rsrc(p.x + (long)m0 * p.K, (uint32_t)(min(BM, p.M - m0) * p.K * 2));
    P.rq = make_rsrc(p.xq_out + (long)m0 * p.K, (uint32_t)(min(BM, p.M - m0) * p.K));
    const int r = t >> 4, c = t & 15;
#pragma unroll
    for (int i = 0; i < PIPE::A_CH; ++i) {
      P.x_off[i] = (uint32_t)((16 * i + r) * p.K * 2 + c * 16);
      P.q_off[i] = (uint32_t)((16 * i + r) * p.K + c * 8);
    }
    P.q_col = c * 8;
    P.x_dst = r * 128 + (((c >> 1) ^ xswz(r)) << 4) + (c & 1) * 8;
    P.wq = tn == 0;
  } else {
    P.rx = make_rsrc(p.xq + (long)m0 * p.K, (uint32_t)(min(BM, p.M - m0) * p.K));
    const int r = t >> 3, c = t & 7;
#pragma unroll
    for (int i = 0; i < MB; ++i) P.x_off[i] = (uint32_t)((32 * i + r) * p.K + c * 16);
    P.x_dst = r * 128 + ((c ^ xswz(r)) << 4);
  }
  P.K = p.K;
#pragma unroll
  for (int i = 0; i < PIPE::WB; ++i) {
    const int r = 8 * i + (lane >> 3), n = n0 + wave * NB * 32 + r;
    P.wb_off[i] = n < p.N ? (uint32_t)((long)n * p.K / 2) : OOB;
    P.wb_dst[i] = r * 128 + (((lane & 7) ^ PIPE::wswz(r)) << 4);
  }
  P.wreg = lds + 4 * PIPE::SB + wave * (NB * 32 * 128);

  u32x4_t xr[PIPE::A_CH];
  u32x4_t wb0[PIPE::WB], wb1[PIPE::WB];  // weight batches, slot j % 2
  u32x4_t wA[NB][2], wB[NB][2];  // weight words of the current and the next stage
  // prologue: batch 0 in LDS, batches 1 and 2 in flight; x of stages 0 and
  // 1 in LDS, stage 2 in flight
  P.issue_wb(0, wb0);
  P.issue_wb(1, wb1);
  if constexpr (STAGED) {
    // The row maxima over all of K first (the weight batches above are in
    // flight meanwhile): TPR threads per row, eight 16-byte loads in flight
    // per thread, |x| by clearing sign bits, maxNum so that a NaN takes no
    // part (as in the quantize kernel); then s = max/127 and r = 1/s refined,
    // per row, into LDS.  The first column tile's first split writes s_x.
    constexpr int TPR = 256 / BM;
    const int row = t / TPR, part = t % TPR, C = p.K / 8;
    f16x2_t am2 = {0, 0};
    for (int j0 = part; j0 < C; j0 += 8 * TPR) {
      u32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = j0 + u * TPR < C ? ld128(P.rx, (uint32_t)(row * p.K * 2 + (j0 + u * TPR) * 16)) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          am2 = __builtin_elementwise_max(am2, __builtin_bit_cast(f16x2_t, v[u][e] & 0x7FFF7FFFu));
    }
    float am = fmaxf((float)am2[0], (float)am2[1]);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
    if (part == 0) {
      const float sv = am / 127.0f;  // correctly rounded division (HIP default)
      float rv = 0.f;
      if (am != 0.f) {
        const float r0 = __builtin_amdgcn_rcpf(sv);
        rv = __builtin_fmaf(__builtin_fmaf(-sv, r0, 1.0f), r0, r0);
      }
      qsh[row] = sv;
      qsh[BM + row] = rv;
      if (tn == 0 && sp == 0 && m0 + row < p.M) p.sx_out[m0 + row] = sv;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PIPE::A_CH; ++i) {
      P.qs[i] = qsh[(t >> 4) + 16 * i];
      P.qr[i] = qsh[BM + (t >> 4) + 16 * i];
    }
  }
  P.issue_x(0, xr);
  __builtin_amdgcn_sched_barrier(0);
  P.store_x(lds, xr, 0);
  P.issue_x(1, xr);
  __builtin_amdgcn_sched_barrier(0);
  P.store_x(lds + PIPE::SB, xr, 1);
  P.put_wb(wb0);
  P.issue_wb(2, wb0);
  P.issue_x(2, xr);
  __builtin_amdgcn_sched_barrier(0);
  // With every prologue load complete, the compiler's view of pending loads
  // at the loop head is the loop's own, so its waits there stay exact.
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  i32x4_t a0[MB], b0[NB];
  P.read_w(0, wA);
  P.read_a(lds, 0, a0);
  P.decode_b(wA, 0, b0);
  const int nst = P.nst;
  // whole rounds of four stages: a stage past the end only loads (clamped)
  // and waits, so the loop body has no branch around a step.  Batch slots:
  // step 1 of a round stores batch s/2+1 (slot 1), step 3 batch s/2+2 (slot 0).
  for (int s = 0; s < nst; s += 4) {
    P.template step<0>(s, lds, xr, wb0, wA, wB, a0, b0, acc);
    P.template step<1>(s + 1, lds, xr, wb1, wB, wA, a0, b0, acc);
    P.template step<2>(s + 2, lds, xr, wb0, wA, wB, a0, b0, acc);
    P.template step<3>(s + 3, lds, xr, wb0, wB, wA, a0, b0, acc);
  }

  if (p.S > 1) {
    // int32 partial of split sp (exact: the sums of any split order agree)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = n0 + wave * NB * 32 + nb * 32 + l32;
      if (n >= p.N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m < p.M) p.part[((long)sp * p.M + m) * p.N + n] = acc[mb][nb][r] >> 4;
        }
    }
    return;
  }
  // epilogue; 32x32 accumulator layout: lane -> column l32, register r -> row 8*(r/4) + 4*h + r%4.
  // The lane's 16 s_x values per row block are loaded together first, so the
  // stores below never wait on a load (rows past M read 0 and are not stored).
  const __amdgpu_buffer_rsrc_t rsx = make_rsrc(p.sx, (uint32_t)p.M * 4u);
  float sxv[MB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if constexpr (STAGED)
        sxv[mb][r] = qsh[rr];  // this workgroup's own scales (another may still be writing s_x)
      else
        sxv[mb][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsx, (uint32_t)(m0 + rr) * 4u, 0, 0));
    }
  if (m0 + BM <= p.M && p.acc_out == nullptr) {
    // Every row of the tile exists and no accumulators are asked for: the
    // row offset is uniform and goes into the scalar base address, the lane
    // keeps one offset for all its stores, and registers r and r+1 (r even:
    // consecutive rows of one column) are rounded as below and stored as the
    // low and the high half of one word.
    const long N = p.N;
    const int wu = __builtin_amdgcn_readfirstlane(wave);  // (uniform: the base goes in scalar registers)
    const uint64_t yw = reinterpret_cast<uint64_t>(p.y + (long)m0 * N + n0 + wu * NB * 32);
    typedef __attribute__((address_space(1))) unsigned char gbyte;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = n0 + wave * NB * 32 + nb * 32 + l32;
      if (n >= p.N) continue;
      const float swn = f16_bits_to_f32(p.sw[n]);
      const uint32_t lo = (uint32_t)(4 * h * N + nb * 32 + l32) * 2u;  // lane part, bytes
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float v0 = ((float)(acc[mb][nb][r] >> 4) * sxv[mb][r]) * swn;
          const float v1 = ((float)(acc[mb][nb][r + 1] >> 4) * sxv[mb][r + 1]) * swn;
          const uint32_t pk = f32x2_to_f16x2_bits(v0, v1);
          uint64_t r0 = yw + (uint64_t)((mb * 32 + 8 * (r >> 2) + (r & 3)) * N * 2);
          uint64_t r1 = r0 + (uint64_t)(N * 2);
          asm volatile("" : "+s"(r0), "+s"(r1));
          *reinterpret_cast<__attribute__((address_space(1))) uint16_t*>(reinterpret_cast<gbyte*>(r0) + lo) =
              (uint16_t)pk;
          *reinterpret_cast<__attribute__((address_space(1))) uint16_t*>(reinterpret_cast<gbyte*>(r1) + lo) =
              (uint16_t)(pk >> 16);
        }
    }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n0 + wave * NB * 32 + nb * 32 + l32;
    if (n >= p.N) continue;
    const float swn = f16_bits_to_f32(p.sw[n]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + mb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < p.M) {
          const int a = acc[mb][nb][r] >> 4;
          if (p.acc_out) p.acc_out[(long)m * p.N + n] = a;
          p.y[(long)m * p.N + n] = f32_to_f16_bits(((float)a * sxv[mb][r]) * swn);
        }
      }
  }
}

// acc = the sum of the S int32 partials; y and acc_out as in the GEMM epilogue
__global__ __launch_bounds__(256) void w4a8_split_sum_kernel(const int32_t* __restrict__ part, int S, int M, int N,
                                                             const float* __restrict__ sx, const uint16_t* __restrict__ sw,
                                                             uint16_t* __restrict__ y, int32_t* __restrict__ acc_out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long MN = (long)M * N;
  if (i >= MN) return;
  // eight partials in flight at a time (the sum is exact in any order)
  int a = 0, s = 0;
  for (; s + 8 <= S; s += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(long)(s + u) * MN + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) a += v[u];
  }
  for (; s < S; ++s) a += part[(long)s * MN + i];
  const int m = (int)(i / N), n = (int)(i % N);
  if (acc_out) acc_out[i] = a;
  y[i] = f32_to_f16_bits(((float)a * sx[m]) * f16_bits_to_f32(sw[n]));
}

// Sum over the 64 lanes of a wave, exact in int32: rotations inside each row
// of 16 lanes (DPP), then two swaps across rows.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += dpp_i<0x128>(v);  // row_ror:8
  v += dpp_i<0x124>(v);  // row_ror:4
  v += dpp_i<0x122>(v);  // row_ror:2
  v += dpp_i<0x121>(v);  // row_ror:1
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Sums over the 64 lanes of four values at once, exact in int32: two
// permlane32 swaps, one permlane16 swap, four DPP row rotations.  Row q
// (lanes 16q .. 16q+15) of the result holds the total of v[q].
__device__ __forceinline__ int wave_sum4_i32(int v0, int v1, int v2, int v3) {
  auto sw32 = [](int a, int b) {
    const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)a, (uint32_t)b, false, false);
    return (int)r[0] + (int)r[1];
  };
  const int s02 = sw32(v0, v2);  // lanes 0-31: halves of v0, lanes 32-63: halves of v2
  const int s13 = sw32(v1, v3);
  const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)s02, (uint32_t)s13, false, false);
  int t = (int)r[0] + (int)r[1];  // row q: quarters of v[q]
  t += dpp_i<0x128>(t);
  t += dpp_i<0x124>(t);
  t += dpp_i<0x122>(t);
  t += dpp_i<0x121>(t);
  return t;
}

// Maximum over the 64 lanes (every lane gets it): lanes l and l ^ 32, then
// rows 2i and 2i+1 by swaps, then rotations inside each row of 16 lanes.
// For non-NaN values the result does not depend on the order.
__device__ __forceinline__ float wave_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  v = fmaxf(v, __int_as_float(dpp_i<0x128>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i<0x124>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i<0x122>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i<0x121>(__float_as_int(v))));
  return v;
}

// W4A8 for M <= 16: one wave per output column n, lanes over K in chunks of
// 32 codes (16 bytes of packed codes; 32 bytes of x_q per row), the codes
// decoded to int8 (16 v, as in the GEMM) and multiplied with v_dot4_i32_i8;
// exact int32 sums, reduced over the wave, shifted right by 4.  MT rows of
// x_q per launch (rows past M read row M-1 and are dropped).
template <int MT>
__global__ __launch_bounds__(256) void w4a8_gemv_kernel(const int8_t* __restrict__ xq, const float* __restrict__ sx,
                                                        const uint32_t* __restrict__ w, const uint16_t* __restrict__ sw,
                                                        uint16_t* __restrict__ y, int32_t* __restrict__ acc_out, int M,
                                                        int N, int K) {
  const int lane = threadIdx.x & 63;
  // the wave index kept uniform: a row base the compiler took for
  // divergent would put a per-lane loop around every buffer load
  const int n = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (n >= N) return;  // the whole wave
  const int nch = K / 32;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (long)n * (K / 8), (uint32_t)(K / 2));
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xq, (uint32_t)M * (uint32_t)K);
  int acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0;
  for (int c = lane; c < nch; c += 64) {
    const u32x4_t wv = ld128(rw, (uint32_t)c * 16u);
    uint32_t d[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) decode_word(wv[i], d[2 * i], d[2 * i + 1]);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint32_t xo = (uint32_t)min(m, M - 1) * (uint32_t)K + (uint32_t)c * 32u;
      const u32x4_t x0 = ld128(rx, xo), x1 = ld128(rx, xo + 16u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[m] = __builtin_amdgcn_sdot4((int)d[i], (int)x0[i], acc[m], false);
        acc[m] = __builtin_amdgcn_sdot4((int)d[4 + i], (int)x1[i], acc[m], false);
      }
    }
  }
  const float swn = f16_bits_to_f32(sw[n]);
  if constexpr (MT < 4) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int a = wave_sum_i32(acc[m]) >> 4;
      if (lane == m && m < M) {
        if (acc_out) acc_out[(long)m * N + n] = a;
        y[(long)m * N + n] = f32_to_f16_bits(((float)a * sx[m]) * swn);
      }
    }
  } else {
    // four rows at a time: row q of the lanes holds row 4g + q
#pragma unroll
    for (int g = 0; g < MT / 4; ++g) {
      const int a = wave_sum4_i32(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]) >> 4;
      const int m = 4 * g + (lane >> 4);
      if ((lane & 15) == 0 && m < M) {
        if (acc_out) acc_out[(long)m * N + n] = a;
        y[(long)m * N + n] = f32_to_f16_bits(((float)a * sx[m]) * swn);
      }
    }
  }
}

// W4A8 for M <= 16 and K <= 4096 in one launch.  Every workgroup first
// quantizes all M rows of x into LDS, one wave per row with the row's
// 8-value chunks in registers, by the same arithmetic as
// w4a8_quant_rows_kernel (so the codes and scales are the same bits);
// workgroup 0 also writes them to x_q and s_x.  Then each of its four waves
// computes CW adjacent columns as w4a8_gemv_kernel computes one, reading
// x_q from LDS once for all CW.  The weight words are loaded before the
// quantize, so their latency overlaps it.  Every workgroup quantizes again
// (x, at most 128 KiB, comes from L2), so CW grows with N to keep the
// workgroups near one per CU.
constexpr int FUSED_MAX_K = 4096;

template <int MT, int CW>
__global__ __launch_bounds__(256) void w4a8_gemv_fused_kernel(const uint16_t* __restrict__ x,
                                                              const uint32_t* __restrict__ w,
                                                              const uint16_t* __restrict__ sw, uint16_t* __restrict__ y,
                                                              int8_t* __restrict__ xq_out, float* __restrict__ sx_out,
                                                              int32_t* __restrict__ acc_out, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) int8_t xs[MT * FUSED_MAX_K];  // [M][K] codes
  __shared__ float ss[MT];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int n0 = (blockIdx.x * 4 + wave) * CW;
  const int nch = K / 32;  // 32-code chunks: at most 128, two per lane
  // weight words of the wave's columns (a column past N reads zeros)
  u32x4_t wv[CW][2];
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc(w + (long)min(n0 + j, N - 1) * (K / 8), n0 + j < N ? (uint32_t)(K / 2) : 0u);
#pragma unroll
    for (int i = 0; i < 2; ++i) wv[j][i] = ld128(rw, lane + 64 * i < nch ? (uint32_t)(lane + 64 * i) * 16u : OOB);
  }

  const int C = K >> 3;  // 8-value chunks per row: at most 512, eight per lane
  const bool first = blockIdx.x == 0;
  // rows wave, wave + 4, ... two at a time, both rows' loads issued first
  auto load_row = [&](int m, u32x4_t (&v)[8]) __attribute__((always_inline)) {
    const u32x4_t* row = reinterpret_cast<const u32x4_t*>(x + (long)min(m, M - 1) * K);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = lane + 64 * j < C ? row[lane + 64 * j] : u32x4_t{0, 0, 0, 0};
  };
  auto quant_row = [&](int m, const u32x4_t (&v)[8]) __attribute__((always_inline)) {
    f16x2_t am2 = {0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        am2 = __builtin_elementwise_max(am2, __builtin_bit_cast(f16x2_t, v[j][e] & 0x7FFF7FFFu));
    const float am = wave_max(fmaxf((float)am2[0], (float)am2[1]));
    const float s = am / 127.0f;  // correctly rounded division (HIP default)
    float r = 0.f;
    if (am != 0.f) {
      const float r0 = __builtin_amdgcn_rcpf(s);
      r = __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
    }
    if (lane == 0) {
      ss[m] = s;
      if (first) sx_out[m] = s;
    }
    u32x2_t* qrow = reinterpret_cast<u32x2_t*>(xs + m * K);
    u32x2_t* grow = reinterpret_cast<u32x2_t*>(xq_out + (long)m * K);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (lane + 64 * j < C) {
        const u32x2_t q = {quant_word(v[j][0], v[j][1], s, r), quant_word(v[j][2], v[j][3], s, r)};
        qrow[lane + 64 * j] = q;
        if (first) grow[lane + 64 * j] = q;
      }
    }
  };
  for (int m = wave; m < M; m += 8) {
    u32x4_t va[8], vb[8];
    load_row(m, va);
    if (m + 4 < M) load_row(m + 4, vb);  // uniform
    quant_row(m, va);
    if (m + 4 < M) quant_row(m + 4, vb);
  }
  __syncthreads();
  if (n0 >= N) return;  // no barrier follows

  int acc[MT][CW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < CW; ++j) acc[m][j] = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      uint32_t d[CW][8];
#pragma unroll
      for (int j = 0; j < CW; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) decode_word(wv[j][i][q], d[j][2 * q], d[j][2 * q + 1]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int8_t* xr = xs + min(m, M - 1) * K + c * 32;
        const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(xr), x1 = *reinterpret_cast<const u32x4_t*>(xr + 16);
#pragma unroll
        for (int j = 0; j < CW; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[m][j] = __builtin_amdgcn_sdot4((int)d[j][q], (int)x0[q], acc[m][j], false);
            acc[m][j] = __builtin_amdgcn_sdot4((int)d[j][4 + q], (int)x1[q], acc[m][j], false);
          }
      }
    }
  }
  // the MT x CW sums, four at a time (value v = m CW + j): row q of group g
  // holds value 4g + q, written by the row's first lane
  constexpr int V = MT * CW;
  if constexpr (V < 4) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int m = v / CW, n = n0 + v % CW;
      const int a = wave_sum_i32(acc[m][v % CW]) >> 4;
      if (lane == 0 && m < M && n < N) {
        if (acc_out) acc_out[(long)m * N + n] = a;
        y[(long)m * N + n] = f32_to_f16_bits(((float)a * ss[m]) * f16_bits_to_f32(sw[n]));
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < V / 4; ++g) {
      const int t = wave_sum4_i32(acc[(4 * g) / CW][(4 * g) % CW], acc[(4 * g + 1) / CW][(4 * g + 1) % CW],
                                  acc[(4 * g + 2) / CW][(4 * g + 2) % CW], acc[(4 * g + 3) / CW][(4 * g + 3) % CW]) >> 4;
      const int v = 4 * g + (lane >> 4), m = v / CW, n = n0 + v % CW;
      if ((lane & 15) == 0 && m < M && n < N) {
        if (acc_out) acc_out[(long)m * N + n] = t;
        y[(long)m * N + n] = f32_to_f16_bits(((float)t * ss[m]) * f16_bits_to_f32(sw[n]));
      }
    }
  }
}

template <int MT>
void launch_fused_cw(const W4A8Args& a, int M, int N, int K, hipStream_t s) {
  const uint16_t* x = (const uint16_t*)a.x;
  const uint16_t* sw = (const uint16_t*)a.s_w;
  uint16_t* y = (uint16_t*)a.y;
  // columns per wave: as many as keep 256 workgroups (4 waves each)
  const int cw = N >= 4096 ? 4 : (N >= 2048 ? 2 : 1);
  const dim3 grid((unsigned)((N + 4 * cw - 1) / (4 * cw))), b256(256);
  if (cw == 4)
    hipLaunchKernelGGL((w4a8_gemv_fused_kernel<MT, 4>), grid, b256, 0, s, x, a.w, sw, y, a.x_q, a.s_x, a.acc, M, N, K);
  else if (cw == 2)
    hipLaunchKernelGGL((w4a8_gemv_fused_kernel<MT, 2>), grid, b256, 0, s, x, a.w, sw, y, a.x_q, a.s_x, a.acc, M, N, K);
  else
    hipLaunchKernelGGL((w4a8_gemv_fused_kernel<MT, 1>), grid, b256, 0, s, x, a.w, sw, y, a.x_q, a.s_x, a.acc, M, N, K);
}

}  // namespace

struct GemmTile {
  int mb, nb;  // tile (32 mb) x (128 nb)
};

// the quantize kernel: x -> x_q, s_x
static hipError_t launch_quant(const W4A8Args& a, hipStream_t s) {
  // threads per row: one wave up to 512 values, two up to 1024, then four;
  // chunks per thread: 1, 2, 4 or 8 (K <= 16384), else one row per block
  const int M = (int)a.M, K = (int)a.K;
  const uint16_t* x = (const uint16_t*)a.x;
  const int C = K / 8;
  const dim3 b256(256);
  if (C <= 64)
    hipLaunchKernelGGL((w4a8_quant_rows_kernel<1, 1>), dim3((M + 3) / 4), b256, 0, s, x, M, K, a.x_q, a.s_x);
  else if (C <= 128)
    hipLaunchKernelGGL((w4a8_quant_rows_kernel<2, 1>), dim3((M + 1) / 2), b256, 0, s, x, M, K, a.x_q, a.s_x);
  else if (C <= 256)
    hipLaunchKernelGGL((w4a8_quant_rows_kernel<4, 1>), dim3(M), b256, 0, s, x, M, K, a.x_q, a.s_x);
  else if (C <= 512)
    hipLaunchKernelGGL((w4a8_quant_rows_kernel<4, 2>), dim3(M), b256, 0, s, x, M, K, a.x_q, a.s_x);
  else if (C <= 1024)
    hipLaunchKernelGGL((w4a8_quant_rows_kernel<4, 4>), dim3(M), b256, 0, s, x, M, K, a.x_q, a.s_x);
  else if (C <= 2048)
    hipLaunchKernelGGL((w4a8_quant_rows_kernel<4, 8>), dim3(M), b256, 0, s, x, M, K, a.x_q, a.s_x);
  else
    hipLaunchKernelGGL(w4a8_quant_kernel, dim3(M), b256, 0, s, x, K, a.x_q, a.s_x);
  return hipGetLastError();
}

static bool shape_ok(const W4A8Args& a) {
  // K whole 32-code chunks; buffer offsets are 32-bit
  return a.K % 32 == 0 && a.N * a.K / 2 < (int64_t(1) << 31) && a.K * 256 < (int64_t(1) << 31) &&
         a.M * a.K * 2 < (int64_t(1) << 31);
}

// Tile: with K of 16 stages or more, the largest whose grid gives every
// CU a workgroup; with shorter K (a short loop, where more workgroups
// overlap better) 64 x 256 or 64 x 128 if it gives every CU two.  Else
// 32 x 128 (half the MFMA work per fragment read, the most workgroups).
// The sweep of both lowerings and every tile (bench.py --w4a8-sweep) finds
// this choice the fastest, or within 3% of it, on each shape of the set.
static GemmTile auto_tile(int M, int N, int K) {
  auto count = [&](const GemmTile& c) {
    return (long)((M + c.mb * 32 - 1) / (c.mb * 32)) * ((N + c.nb * 128 - 1) / (c.nb * 128));
  };
  const bool long_k = K >= 16 * BK;
  const GemmTile tiles[] = {{4, 2}, {2, 2}, {2, 1}};
  for (const GemmTile& c : tiles) {
    if (!long_k && c.mb == 4) continue;
    if (count(c) >= (long_k ? 256 : 512)) return c;
  }
  return GemmTile{1, 1};
}

// The integer product and epilogue on one tile shape: from x_q (full-K
// lowering, x_q and s_x already written) or from x (staged lowering, which
// writes x_q and s_x itself).
static hipError_t launch_gemm_tile(const W4A8Args& a, bool staged, GemmTile t, hipStream_t s) {
  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  Params p;
  p.xq = a.x_q;
  p.sx = a.s_x;
  p.x = (const uint16_t*)a.x;
  p.xq_out = a.x_q;
  p.sx_out = a.s_x;
  p.w = a.w;
  p.sw = (const uint16_t*)a.s_w;
  p.y = (uint16_t*)a.y;
  p.acc_out = a.acc;
  p.M = M;
  p.N = N;
  p.K = K;
  p.Tm = (M + t.mb * 32 - 1) / (t.mb * 32);
  p.Tn = (N + t.nb * 128 - 1) / (t.nb * 128);
  // K splits when the tiles leave CUs idle and K has at least 16 stages:
  // enough workgroups for every CU, at least 4 whole stages per split,
  // partials within 32-bit sizes.  (Below 16 stages the split's second
  // kernel and partials cost more than the shorter K loop saves.)
  {
    const int nst = (K + BK - 1) / BK, tiles = p.Tm * p.Tn;
    int S = 1;
    if (tiles < 256 && nst >= 16) {
      S = std::min((256 + tiles - 1) / tiles, nst / 4);
      while (S > 1 && (int64_t)S * M * N * 4 >= (int64_t(1) << 31)) --S;
    }
    p.per_split = (nst + S - 1) / S;
    p.S = (nst + p.per_split - 1) / p.per_split;  // no empty split
    p.part = nullptr;
    if (p.S > 1) {
      const hipError_t e2 = stream_workspace(s, (size_t)p.S * M * N * 4, (void**)&p.part);
      if (e2 != hipSuccess) return e2;
    }
  }
  p.per_xcd = (p.Tm * p.Tn * p.S + 7) / 8;
  const dim3 grid(8 * p.per_xcd);
#define QAFF_W4A8_LAUNCH(MB, NB)                                                      \
  if (staged)                                                                        \
    hipLaunchKernelGGL((w4a8_gemm_kernel<MB, NB, true>), grid, dim3(256), 0, s, p);  \
  else                                                                               \
    hipLaunchKernelGGL((w4a8_gemm_kernel<MB, NB, false>), grid, dim3(256), 0, s, p);
  if (t.mb == 4 && t.nb == 2) {
    QAFF_W4A8_LAUNCH(4, 2)
  } else if (t.mb == 2 && t.nb == 2) {
    QAFF_W4A8_LAUNCH(2, 2)
  } else if (t.mb == 2 && t.nb == 1) {
    QAFF_W4A8_LAUNCH(2, 1)
  } else if (t.mb == 1 && t.nb == 1) {
    QAFF_W4A8_LAUNCH(1, 1)
  } else {
    return hipErrorNotSupported;
  }
#undef QAFF_W4A8_LAUNCH
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && p.S > 1) {
    const long MN = (long)M * N;
    hipLaunchKernelGGL(w4a8_split_sum_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, p.part, p.S, M, N,
                       p.sx, p.sw, p.y, p.acc_out);
    e = hipGetLastError();
  }
  return e;
}

// Which lowering runs when the caller does not choose (M > 16): the
// full-K one.  The staged lowering quantizes x once per column tile inside
// the GEMM; on every shape of the sweep that repeated work cost more than
// the x_q round trip it saves (qgemm_w4a8_tiled still runs it).
static bool staged_default(int M, int N, int K) {
  (void)M;
  (void)N;
  (void)K;
  return false;
}

hipError_t launch_w4a8_product(const W4A8Args& a, hipStream_t s) {
  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  if (M <= 16) {
    const dim3 grid((unsigned)((N + 3) / 4));
    const int8_t* xq = a.x_q;
    const uint32_t* w = a.w;
    const uint16_t* sw = (const uint16_t*)a.s_w;
    uint16_t* y = (uint16_t*)a.y;
    if (M == 1)
      hipLaunchKernelGGL(w4a8_gemv_kernel<1>, grid, dim3(256), 0, s, xq, a.s_x, w, sw, y, a.acc, M, N, K);
    else if (M == 2)
      hipLaunchKernelGGL(w4a8_gemv_kernel<2>, grid, dim3(256), 0, s, xq, a.s_x, w, sw, y, a.acc, M, N, K);
    else if (M <= 4)
      hipLaunchKernelGGL(w4a8_gemv_kernel<4>, grid, dim3(256), 0, s, xq, a.s_x, w, sw, y, a.acc, M, N, K);
    else if (M <= 8)
      hipLaunchKernelGGL(w4a8_gemv_kernel<8>, grid, dim3(256), 0, s, xq, a.s_x, w, sw, y, a.acc, M, N, K);
    else
      hipLaunchKernelGGL(w4a8_gemv_kernel<16>, grid, dim3(256), 0, s, xq, a.s_x, w, sw, y, a.acc, M, N, K);
    return hipGetLastError();
  }
  return launch_gemm_tile(a, false, auto_tile(M, N, K), s);
}

hipError_t launch_w4a8(const W4A8Args& a, hipStream_t s) {
  if (!shape_ok(a)) return hipErrorNotSupported;
  const int M = (int)a.M, N = (int)a.N, K = (int)a.K;
  if (M <= 16 && K <= FUSED_MAX_K) {
    if (M == 1) launch_fused_cw<1>(a, M, N, K, s);
    else if (M == 2) launch_fused_cw<2>(a, M, N, K, s);
    else if (M <= 4) launch_fused_cw<4>(a, M, N, K, s);
    else if (M <= 8) launch_fused_cw<8>(a, M, N, K, s);
    else launch_fused_cw<16>(a, M, N, K, s);
    return hipGetLastError();
  }
  if (M <= 16) {
    const hipError_t e = launch_quant(a, s);
    if (e != hipSuccess) return e;
    return launch_w4a8_product(a, s);
  }
  const GemmTile t = auto_tile(M, N, K);
  if (!staged_default(M, N, K)) {
    const hipError_t e = launch_quant(a, s);
    if (e != hipSuccess) return e;
    return launch_gemm_tile(a, false, t, s);
  }
  return launch_gemm_tile(a, true, t, s);
}

hipError_t launch_w4a8_config(const W4A8Args& a, int staged, int bm, int bn, hipStream_t s) {
  if (!shape_ok(a) || a.M <= 16) return hipErrorNotSupported;
  const GemmTile t{bm / 32, bn / 128};
  if (bm % 32 || bn % 128) return hipErrorNotSupported;
  if (!staged) {
    const hipError_t e = launch_quant(a, s);
    if (e != hipSuccess) return e;
  }
  return launch_gemm_tile(a, staged != 0, t, s);
}

}  // namespace qaff
