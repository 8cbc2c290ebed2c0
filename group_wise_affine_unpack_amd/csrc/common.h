// Shared device helpers and launcher declarations of libqaff (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qaff {

enum Dtype : int { BF16 = 0, F16 = 1, F32 = 2 };

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;

// ---- scalar storage formats -------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// element i of a bf16 / f16 / f32 array as float (exact)
__device__ __forceinline__ float load_as_f32(const void* base, long i, int dt) {
  if (dt == BF16) return bf16_bits_to_f32(((const uint16_t*)base)[i]);
  if (dt == F16) return f16_bits_to_f32(((const uint16_t*)base)[i]);
  return ((const float*)base)[i];
}

// float -> 16-bit storage, round to nearest even (v_cvt_pk_bf16_f32 / v_cvt_f16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}
// Two floats rounded to f16 (nearest even) in one word, the first in the low
// half, each exactly as f32_to_f16_bits rounds it on its own: where the value
// is a product, the compiler folds that multiply into the rounding (one
// v_fma_mix, a single rounding of the exact product), and a packed
// conversion of the two fp32 products would round twice (measured to differ
// on about 0.007% of W4A8 outputs).  The barrier keeps the pair from being
// merged into the packed conversion.
__device__ __forceinline__ uint32_t f32x2_to_f16x2_bits(float lo, float hi) {
  uint32_t a = f32_to_f16_bits(lo), b = f32_to_f16_bits(hi);
  asm volatile("" : "+v"(a), "+v"(b));
  return a | (b << 16);
}
__device__ __forceinline__ uint16_t f32_to_act_bits(float v, bool f16) {
  return f16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
}

// ---- buffer resources -----------------------------------------------------
// Raw buffer descriptor over [base, base + bytes): a load whose offset
// (VGPR offset plus immediate) is at or past `bytes` returns zeros.
constexpr uint32_t RSRC_WORD3 = 0x00020000u;  // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)RSRC_WORD3);
}

// ---- wave reduction -----------------------------------------------------
// Sum over the 64 lanes of a wave: rotates inside each row of 16 lanes with
// DPP (every lane of the row ends with the row sum), then two swaps across
// rows.  Every lane returns the full sum.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0x128>(v);  // row_ror:8
  v += dpp_mov<0x124>(v);  // row_ror:4
  v += dpp_mov<0x122>(v);  // row_ror:2
  v += dpp_mov<0x121>(v);  // row_ror:1
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace qaff

// ---- launchers (host side; each returns a hipError_t) ---------------------

namespace qaff {

struct AffineArgs {
  const void* x;
  const uint32_t* w;
  const void* scales;
  const void* biases;
  const int32_t* k_perm;
  void* y;
  int64_t M, N, K;
  int G, bits;
  int act_dt, s_dt, b_dt;
};

// scratch of `bytes` for work on stream s: the stream's cached buffer (see
// workspace.hip); valid until the next call on the same stream
hipError_t stream_workspace(hipStream_t s, size_t bytes, void** out);
// Until scratch_override_end, stream_workspace calls on this thread return
// `p` (cap bytes) instead of a stream buffer, and fail with
// hipErrorOutOfMemory for more; _end returns the largest request seen.
void scratch_override_begin(void* p, size_t cap);
size_t scratch_override_end();
// frees every cached and grown-out workspace buffer of every device;
// *freed = bytes of the cached (current) buffers
hipError_t release_workspaces(size_t* freed);

// workgroups of `kernel` (`block` threads, `lds` bytes of dynamic LDS) that
// the current device holds at once, counting at most max_per_cu per CU:
// resident per CU times the CUs (cached per device, kernel, block and LDS)
hipError_t resident_workgroups(const void* kernel, int block, size_t lds, int max_per_cu, int64_t* out);

// the device address of the no-allocation entry point's fixed scratch array
// on the current device (looked up once per device) and its size
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

hipError_t launch_gemv_affine(const AffineArgs& a, hipStream_t s);
// count problems that share M, G, bits and dtypes, in as few launches as possible
hipError_t launch_gemv_grouped(const AffineArgs* probs, int count, hipStream_t s);
hipError_t launch_gemm_affine(const AffineArgs& a, hipStream_t s);
// y = W (silu(a.x) * up) [+ resid], M <= 16 (a.x is the gate)
hipError_t launch_gemv_silu(const AffineArgs& a, const void* up, const void* resid, hipStream_t s);

// A decode chain (gemv_affine.hip): 4-bit linears at M = 1, in stages; the
// plan holds the device descriptors and counts, each run is one launch.
struct ChainSpec {
  const void* x;      // [K]; with a gate, the up projection
  const void* gate;   // [K] or null
  const void* resid;  // [N] or null
  const void* w;
  const void* scales;
  const void* biases;
  void* y;            // [N]
  int64_t N, K;
  int stage;          // nondecreasing
};
hipError_t chain_plan_create(const ChainSpec* spec, int count, int G, int act_f16, void** out);
hipError_t chain_plan_run(void* plan, hipStream_t s);
hipError_t chain_plan_status(void* plan, int* timed_out);
hipError_t chain_plan_free(void* plan);

struct GptqArgs {
  const void* x;
  const int32_t* qweight;
  const int32_t* qzeros;
  const void* scales;
  const int32_t* g_idx;
  void* y;
  int64_t M, N, K;
  int G;
};
hipError_t launch_gptq_direct(const GptqArgs& a, hipStream_t s);
hipError_t launch_gptq_repack(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                              const int32_t* k_perm_dev, uint32_t* w_out, void* s_out, void* b_out, int bias_dt,
                              int64_t K, int64_t N, int G, hipStream_t s);

struct W4A8Args {
  const void* x;
  const uint32_t* w;
  const void* s_w;
  void* y;
  int8_t* x_q;
  float* s_x;
  int32_t* acc;
  int64_t M, N, K;
};
hipError_t launch_w4a8(const W4A8Args& a, hipStream_t s);
// the integer product and epilogue of W4A8 from x_q and s_x already written
hipError_t launch_w4a8_product(const W4A8Args& a, hipStream_t s);
// M > 16 with a chosen lowering (staged: quantize inside the GEMM; else the
// quantize kernel, then the full-K GEMM) and tile bm x bn
hipError_t launch_w4a8_config(const W4A8Args& a, int staged, int bm, int bn, hipStream_t s);
// SmoothQuant: factors, weight quantization (optional fold), smoothed quantizer
hipError_t launch_smooth_factors(const float* amax, const void* w, int w_dt, int64_t N, int64_t K, double alpha,
                                 float* s, hipStream_t st);
hipError_t launch_w4a8_weights(const void* w, int w_dt, const float* smooth, int64_t N, int64_t K, uint32_t* w_q4,
                               uint16_t* s_w, hipStream_t st);
hipError_t launch_smooth_quant(const void* x, const float* smooth, int64_t M, int64_t K, int8_t* x_q, float* s_x,
                               hipStream_t st);

hipError_t launch_dequant(const uint32_t* w, const void* s, const void* b, void* out, int64_t N, int64_t K, int G,
                          int bits, int sdt, int bdt, int odt, hipStream_t st);

// streaming read of `bytes` (a multiple of 16) by `blocks` x 256 threads;
// sink holds blocks*256 words
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s);

hipError_t launch_quantize_pack(const void* w, int w_dt, uint32_t* packed, void* scales, void* biases, int sb_dt,
                                int64_t N, int64_t K, int G, int bits, hipStream_t s);

}  // namespace qaff
