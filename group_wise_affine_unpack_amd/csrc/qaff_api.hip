// C ABI of libqaff: argument checks, dispatch, error reporting.
// The declarations and their contracts are in include/qaff.h.
#include <stdarg.h>
#include <stdio.h>

#include <string>
#include <vector>

#include "../../include/qaff.h"
#include "common.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return QAFF_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(QAFF_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool act_dtype_ok(int d) { return d == QAFF_BF16 || d == QAFF_F16; }
bool sb_dtype_ok(int d) { return d == QAFF_BF16 || d == QAFF_F16 || d == QAFF_F32; }
bool group_ok(int g) { return g == 32 || g == 64 || g == 128; }

constexpr int64_t kMaxDim = int64_t(1) << 30;  // int32 index arithmetic inside the kernels

int check_affine(const void* x, const uint32_t* w, const void* s, const void* b, const void* y, int64_t M,
                 int64_t N, int64_t K, int G, int bits, int act_dt, int s_dt, int b_dt) {
  if (M < 0 || N < 0 || K <= 0) return fail(QAFF_E_INVAL, "sizes must satisfy M >= 0, N >= 0, K > 0 (got %lld, %lld, %lld)", (long long)M, (long long)N, (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(QAFF_E_UNSUPPORTED, "dimension above 2^30");
  if (!(bits == 2 || bits == 4 || bits == 8)) return fail(QAFF_E_INVAL, "bits must be 2, 4 or 8 (got %d)", bits);
  if (!group_ok(G)) return fail(QAFF_E_INVAL, "group_size must be 32, 64 or 128 (got %d)", G);
  if (K % G != 0) return fail(QAFF_E_INVAL, "K=%lld is not a multiple of group_size=%d", (long long)K, G);
  if (K % (32 / bits) != 0) return fail(QAFF_E_INVAL, "K=%lld is not a multiple of 32/bits=%d", (long long)K, 32 / bits);
  if (!act_dtype_ok(act_dt)) return fail(QAFF_E_INVAL, "act_dtype must be QAFF_BF16 or QAFF_F16 (got %d)", act_dt);
  if (!sb_dtype_ok(s_dt) || !sb_dtype_ok(b_dt)) return fail(QAFF_E_INVAL, "scale/bias dtype must be BF16, F16 or F32");
  if (M == 0 || N == 0) return QAFF_OK;
  if (!x || !w || !s || !b || !y) return fail(QAFF_E_INVAL, "null tensor pointer");
  if (!aligned16(x) || !aligned16(w)) return fail(QAFF_E_ALIGN, "x and w_packed must be 16-byte aligned");
  return QAFF_OK;
}

qaff::AffineArgs affine_args(const void* x, const uint32_t* w, const void* s, const void* b, const int32_t* kp,
                             void* y, int64_t M, int64_t N, int64_t K, int G, int bits, int act_dt, int s_dt,
                             int b_dt) {
  qaff::AffineArgs a;
  a.x = x;
  a.w = w;
  a.scales = s;
  a.biases = b;
  a.k_perm = kp;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  a.G = G;
  a.bits = bits;
  a.act_dt = act_dt;
  a.s_dt = s_dt;
  a.b_dt = b_dt;
  return a;
}

}  // namespace

extern "C" {

const char* qaff_last_error(void) { return g_last_error.c_str(); }

int qaff_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  if (!src || !sink) return fail(QAFF_E_INVAL, "null pointer");
  if (bytes == 0 || bytes % 16) return fail(QAFF_E_INVAL, "bytes must be a positive multiple of 16");
  if (blocks <= 0) return fail(QAFF_E_INVAL, "blocks must be positive");
  if (!aligned16(src)) return fail(QAFF_E_ALIGN, "src must be 16-byte aligned");
  (void)hipGetLastError();
  hipError_t e = qaff::launch_stream_read(src, (size_t)bytes, sink, blocks, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream read launch");
  return ok();
}

int qaff_version(void) { return 200; }

int qaff_release_workspaces(uint64_t* freed_bytes) {
  size_t freed = 0;
  const hipError_t e = qaff::release_workspaces(&freed);
  if (freed_bytes) *freed_bytes = (uint64_t)freed;
  if (e != hipSuccess) return hip_fail(e, "releasing workspaces");
  return ok();
}

int qgemv_affine(const void* x, const uint32_t* w_packed, const void* scales, const void* biases,
                 const int32_t* k_perm, void* y, int64_t M, int64_t N, int64_t K, int32_t group_size,
                 int32_t bits, int32_t act_dtype, int32_t scale_dtype, int32_t bias_dtype, void* stream) {
  int rc = check_affine(x, w_packed, scales, biases, y, M, N, K, group_size, bits, act_dtype, scale_dtype, bias_dtype);
  if (rc != QAFF_OK) return rc;
  if (M > 16) return fail(QAFF_E_INVAL, "qgemv_affine takes M <= 16 (got %lld)", (long long)M);
  if (M == 0 || N == 0) return ok();
  (void)hipGetLastError();
  hipError_t e = qaff::launch_gemv_affine(
      affine_args(x, w_packed, scales, biases, k_perm, y, M, N, K, group_size, bits, act_dtype, scale_dtype, bias_dtype),
      static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "row or activation too large for 32-bit offsets");
  if (e != hipSuccess) return hip_fail(e, "gemv launch");
  return ok();
}

int qgemv_affine_silu_gate(const void* gate, const void* up, const void* resid, const uint32_t* w_packed,
                           const void* scales, const void* biases, void* y, int64_t M, int64_t N, int64_t K,
                           int32_t group_size, int32_t bits, int32_t act_dtype, int32_t scale_dtype,
                           int32_t bias_dtype, void* stream) {
  int rc = check_affine(gate, w_packed, scales, biases, y, M, N, K, group_size, bits, act_dtype, scale_dtype, bias_dtype);
  if (rc != QAFF_OK) return rc;
  if (M > 16) return fail(QAFF_E_INVAL, "qgemv_affine_silu_gate takes M <= 16 (got %lld)", (long long)M);
  if (M == 0 || N == 0) return ok();
  if (!up) return fail(QAFF_E_INVAL, "null tensor pointer (up)");
  if (!aligned16(up)) return fail(QAFF_E_ALIGN, "gate and up must be 16-byte aligned");
  if ((K * bits) % 128 != 0) return fail(QAFF_E_UNSUPPORTED, "the gated GEMV takes rows of whole 16-byte chunks (K*bits %% 128 == 0)");
  (void)hipGetLastError();
  hipError_t e = qaff::launch_gemv_silu(
      affine_args(gate, w_packed, scales, biases, nullptr, y, M, N, K, group_size, bits, act_dtype, scale_dtype, bias_dtype),
      up, resid, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "row or activation too large for 32-bit offsets");
  if (e != hipSuccess) return hip_fail(e, "gated gemv launch");
  return ok();
}

int qgemv_affine_chain_plan(const qaff_chain_linear* linears, int32_t count, int32_t group_size, int32_t bits,
                            int32_t act_dtype, void** plan_out) {
  if (!plan_out) return fail(QAFF_E_INVAL, "null plan_out");
  *plan_out = nullptr;
  if (count < 1 || count > (1 << 20)) return fail(QAFF_E_INVAL, "count must be in [1, 2^20] (got %d)", count);
  if (!linears) return fail(QAFF_E_INVAL, "null linear array");
  if (bits != 4) return fail(QAFF_E_UNSUPPORTED, "the chain takes 4-bit codes (got %d)", bits);
  if (!(act_dtype == QAFF_BF16 || act_dtype == QAFF_F16))
    return fail(QAFF_E_INVAL, "act_dtype must be QAFF_BF16 or QAFF_F16 (got %d)", act_dtype);
  std::vector<qaff::ChainSpec> spec(count);
  for (int32_t i = 0; i < count; ++i) {
    const qaff_chain_linear& l = linears[i];
    int rc = check_affine(l.x, l.w_packed, l.scales, l.biases, l.y, 1, l.N, l.K, group_size, bits, act_dtype,
                          act_dtype, act_dtype);
    if (rc != QAFF_OK) {
      const std::string msg = g_last_error;
      return fail(rc, "linear %d: %s", i, msg.c_str());
    }
    if (l.N < 1) return fail(QAFF_E_INVAL, "linear %d: N must be >= 1", i);
    if (l.K % 32 != 0) return fail(QAFF_E_UNSUPPORTED, "linear %d: K must be a multiple of 32 (got %lld)", i, (long long)l.K);
    if (l.K > 32768) return fail(QAFF_E_UNSUPPORTED, "linear %d: K above 32768 (the input is staged in LDS)", i);
    if (l.gate && !aligned16(l.gate)) return fail(QAFF_E_ALIGN, "linear %d: gate must be 16-byte aligned", i);
    if (l.stage < 0 || (i > 0 && l.stage < linears[i - 1].stage))
      return fail(QAFF_E_INVAL, "linear %d: stages must be >= 0 and nondecreasing", i);
    if (l.N * l.K / 2 >= (int64_t(1) << 31)) return fail(QAFF_E_UNSUPPORTED, "linear %d too large for 32-bit offsets", i);
    spec[i] = qaff::ChainSpec{l.x, l.gate, l.resid, l.w_packed, l.scales, l.biases, l.y, l.N, l.K, l.stage};
  }
  if (linears[count - 1].stage >= (1 << 20)) return fail(QAFF_E_INVAL, "more than 2^20 stages");
  (void)hipGetLastError();
  hipError_t e = qaff::chain_plan_create(spec.data(), count, group_size, act_dtype == QAFF_F16, plan_out);
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "chain too large or kernel not resident");
  if (e != hipSuccess) return hip_fail(e, "chain plan");
  return ok();
}

int qgemv_affine_chain_run(void* plan, void* stream) {
  if (!plan) return fail(QAFF_E_INVAL, "null plan");
  (void)hipGetLastError();
  hipError_t e = qaff::chain_plan_run(plan, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidDevice) return fail(QAFF_E_INVAL, "the plan belongs to another device");
  if (e != hipSuccess) return hip_fail(e, "chain launch");
  return ok();
}

int qgemv_affine_chain_status(void* plan, int32_t* timed_out) {
  if (!plan || !timed_out) return fail(QAFF_E_INVAL, "null plan or timed_out");
  int t = 0;
  hipError_t e = qaff::chain_plan_status(plan, &t);
  if (e != hipSuccess) return hip_fail(e, "chain status");
  *timed_out = t;
  return ok();
}

int qgemv_affine_chain_free(void* plan) {
  if (!plan) return ok();
  hipError_t e = qaff::chain_plan_free(plan);
  if (e != hipSuccess) return hip_fail(e, "chain free");
  return ok();
}

int qgemv_affine_grouped(const qaff_gemv_problem* problems, int32_t count, int64_t M, int32_t group_size,
                         int32_t bits, int32_t act_dtype, int32_t scale_dtype, int32_t bias_dtype, void* stream) {
  if (count < 0 || count > 65536) return fail(QAFF_E_INVAL, "count must be in [0, 65536] (got %d)", count);
  if (count > 0 && problems == nullptr) return fail(QAFF_E_INVAL, "null problem array");
  if (M > 16) return fail(QAFF_E_INVAL, "qgemv_affine_grouped takes M <= 16 (got %lld)", (long long)M);
  std::vector<qaff::AffineArgs> args;
  args.reserve(count);
  for (int32_t i = 0; i < count; ++i) {
    const qaff_gemv_problem& p = problems[i];
    int rc = check_affine(p.x, p.w_packed, p.scales, p.biases, p.y, M, p.N, p.K, group_size, bits, act_dtype,
                          scale_dtype, bias_dtype);
    if (rc != QAFF_OK) {
      const std::string msg = g_last_error;
      return fail(rc, "problem %d: %s", i, msg.c_str());
    }
    if (M > 0 && p.N > 0)
      args.push_back(affine_args(p.x, p.w_packed, p.scales, p.biases, p.k_perm, p.y, M, p.N, p.K, group_size, bits,
                                 act_dtype, scale_dtype, bias_dtype));
  }
  if (args.empty()) return ok();
  (void)hipGetLastError();
  hipError_t e = qaff::launch_gemv_grouped(args.data(), (int)args.size(), static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "a problem is too large for 32-bit offsets");
  if (e != hipSuccess) return hip_fail(e, "grouped gemv launch");
  return ok();
}

int qmm_affine(const void* x, const uint32_t* w_packed, const void* scales, const void* biases,
               const int32_t* k_perm, void* y, int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t bits,
               int32_t act_dtype, int32_t scale_dtype, int32_t bias_dtype, void* stream) {
  int rc = check_affine(x, w_packed, scales, biases, y, M, N, K, group_size, bits, act_dtype, scale_dtype, bias_dtype);
  if (rc != QAFF_OK) return rc;
  if (M == 0 || N == 0) return ok();
  const qaff::AffineArgs a =
      affine_args(x, w_packed, scales, biases, k_perm, y, M, N, K, group_size, bits, act_dtype, scale_dtype, bias_dtype);
  (void)hipGetLastError();
  hipError_t e = (M <= 16) ? qaff::launch_gemv_affine(a, static_cast<hipStream_t>(stream))
                           : qaff::launch_gemm_affine(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "this shape/dtype combination has no kernel");
  if (e != hipSuccess) return hip_fail(e, M <= 16 ? "gemv launch" : "gemm launch");
  return ok();
}

int qmm_affine_noalloc(const void* x, const uint32_t* w_packed, const void* scales, const void* biases,
                       const int32_t* k_perm, void* y, int64_t M, int64_t N, int64_t K, int32_t group_size,
                       int32_t bits, int32_t act_dtype, int32_t scale_dtype, int32_t bias_dtype, void* stream) {
  int rc = check_affine(x, w_packed, scales, biases, y, M, N, K, group_size, bits, act_dtype, scale_dtype, bias_dtype);
  if (rc != QAFF_OK) return rc;
  if (M == 0 || N == 0) return ok();
  const qaff::AffineArgs a =
      affine_args(x, w_packed, scales, biases, k_perm, y, M, N, K, group_size, bits, act_dtype, scale_dtype, bias_dtype);
  void* scratch = nullptr;
  size_t cap = 0;
  hipError_t e = qaff::noalloc_scratch(&scratch, &cap);
  if (e != hipSuccess) return hip_fail(e, "looking up the scratch array");
  (void)hipGetLastError();
  // the launchers take their scratch from the array instead of the stream
  // buffer; a request past its size fails in the launcher
  qaff::scratch_override_begin(scratch, cap);
  e = (M <= 16) ? qaff::launch_gemv_affine(a, static_cast<hipStream_t>(stream))
                : qaff::launch_gemm_affine(a, static_cast<hipStream_t>(stream));
  const size_t need = qaff::scratch_override_end();
  if (need > cap)
    return fail(QAFF_E_UNSUPPORTED, "this call needs %zu bytes of scratch; qmm_affine_noalloc has %zu (use qmm_affine)",
                need, cap);
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "this shape/dtype combination has no kernel");
  if (e != hipSuccess) return hip_fail(e, M <= 16 ? "gemv launch" : "gemm launch");
  return ok();
}

int qmm_gptq(const void* x, const int32_t* qweight, const int32_t* qzeros, const void* scales, const int32_t* g_idx,
             void* y, int64_t M, int64_t N, int64_t K, int32_t group_size, void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return fail(QAFF_E_INVAL, "sizes must satisfy M >= 0, N > 0, K > 0");
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(QAFF_E_UNSUPPORTED, "dimension above 2^30");
  if (!group_ok(group_size)) return fail(QAFF_E_INVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
  if (K % group_size || K % 8 || N % 8) return fail(QAFF_E_INVAL, "need K %% G == 0, K %% 8 == 0, N %% 8 == 0");
  if (M == 0) return ok();
  if (!x || !qweight || !qzeros || !scales || !y) return fail(QAFF_E_INVAL, "null tensor pointer");
  if (!aligned16(x) || !aligned16(qweight)) return fail(QAFF_E_ALIGN, "x and qweight must be 16-byte aligned");
  qaff::GptqArgs a;
  a.x = x;
  a.qweight = qweight;
  a.qzeros = qzeros;
  a.scales = scales;
  a.g_idx = g_idx;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  a.G = group_size;
  (void)hipGetLastError();
  hipError_t e = qaff::launch_gptq_direct(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "this shape has no kernel");
  if (e != hipSuccess) return hip_fail(e, "gptq launch");
  return ok();
}

int qgemm_w4a8(const void* x, const uint32_t* w_q4, const void* s_w, void* y, int8_t* x_q, float* s_x,
               int32_t* acc_out, int64_t M, int64_t N, int64_t K, void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return fail(QAFF_E_INVAL, "sizes must satisfy M >= 0, N > 0, K > 0");
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(QAFF_E_UNSUPPORTED, "dimension above 2^30");
  if (K % 32) return fail(QAFF_E_INVAL, "K must be a multiple of 32 (got %lld)", (long long)K);
  // |acc| <= K * 127 * 8 must fit int32 (also after the x16 nibble placement used on the device)
  if (K > (int64_t(1) << 17)) return fail(QAFF_E_UNSUPPORTED, "K above 131072 could overflow the int32 accumulator");
  if (M == 0) return ok();
  if (!x || !w_q4 || !s_w || !y || !x_q || !s_x) return fail(QAFF_E_INVAL, "null tensor pointer");
  if (!aligned16(x) || !aligned16(w_q4) || !aligned16(x_q)) return fail(QAFF_E_ALIGN, "x, w_q4 and x_q must be 16-byte aligned");
  qaff::W4A8Args a;
  a.x = x;
  a.w = w_q4;
  a.s_w = s_w;
  a.y = y;
  a.x_q = x_q;
  a.s_x = s_x;
  a.acc = acc_out;
  a.M = M;
  a.N = N;
  a.K = K;
  (void)hipGetLastError();
  hipError_t e = qaff::launch_w4a8(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "this shape has no kernel");
  if (e != hipSuccess) return hip_fail(e, "w4a8 launch");
  return ok();
}

int qgemm_w4a8_tiled(const void* x, const uint32_t* w_q4, const void* s_w, void* y, int8_t* x_q, float* s_x,
                     int32_t* acc_out, int64_t M, int64_t N, int64_t K, int32_t staged, int32_t bm, int32_t bn,
                     void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return fail(QAFF_E_INVAL, "sizes must satisfy M >= 0, N > 0, K > 0");
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(QAFF_E_UNSUPPORTED, "dimension above 2^30");
  if (K % 32) return fail(QAFF_E_INVAL, "K must be a multiple of 32 (got %lld)", (long long)K);
  if (K > (int64_t(1) << 17)) return fail(QAFF_E_UNSUPPORTED, "K above 131072 could overflow the int32 accumulator");
  if (staged != 0 && staged != 1) return fail(QAFF_E_INVAL, "staged must be 0 or 1");
  const bool tile_ok = (bm == 32 && bn == 128) || (bm == 64 && bn == 128) || (bm == 64 && bn == 256) ||
                       (bm == 128 && bn == 256);
  if (!tile_ok) return fail(QAFF_E_UNSUPPORTED, "tile %dx%d is not built (32x128, 64x128, 64x256, 128x256)", bm, bn);
  if (M == 0) return ok();
  if (M <= 16) return fail(QAFF_E_UNSUPPORTED, "M <= 16 runs the GEMV paths, which have no tile (use qgemm_w4a8)");
  if (!x || !w_q4 || !s_w || !y || !x_q || !s_x) return fail(QAFF_E_INVAL, "null tensor pointer");
  if (!aligned16(x) || !aligned16(w_q4) || !aligned16(x_q)) return fail(QAFF_E_ALIGN, "x, w_q4 and x_q must be 16-byte aligned");
  qaff::W4A8Args a;
  a.x = x;
  a.w = w_q4;
  a.s_w = s_w;
  a.y = y;
  a.x_q = x_q;
  a.s_x = s_x;
  a.acc = acc_out;
  a.M = M;
  a.N = N;
  a.K = K;
  (void)hipGetLastError();
  hipError_t e = qaff::launch_w4a8_config(a, staged, bm, bn, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "this shape has no kernel");
  if (e != hipSuccess) return hip_fail(e, "w4a8 launch");
  return ok();
}

int qgemm_w4a8_smooth(const void* x, const float* smooth, const uint32_t* w_q4, const void* s_w, void* y,
                      int8_t* x_q, float* s_x, int32_t* acc_out, int64_t M, int64_t N, int64_t K, void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return fail(QAFF_E_INVAL, "sizes must satisfy M >= 0, N > 0, K > 0");
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(QAFF_E_UNSUPPORTED, "dimension above 2^30");
  if (K % 32) return fail(QAFF_E_INVAL, "K must be a multiple of 32 (got %lld)", (long long)K);
  if (K > (int64_t(1) << 17)) return fail(QAFF_E_UNSUPPORTED, "K above 131072 could overflow the int32 accumulator");
  if (M == 0) return ok();
  if (!x || !smooth || !w_q4 || !s_w || !y || !x_q || !s_x) return fail(QAFF_E_INVAL, "null tensor pointer");
  if (!aligned16(x) || !aligned16(w_q4) || !aligned16(x_q)) return fail(QAFF_E_ALIGN, "x, w_q4 and x_q must be 16-byte aligned");
  qaff::W4A8Args a;
  a.x = x;
  a.w = w_q4;
  a.s_w = s_w;
  a.y = y;
  a.x_q = x_q;
  a.s_x = s_x;
  a.acc = acc_out;
  a.M = M;
  a.N = N;
  a.K = K;
  if (N * K / 2 >= (int64_t(1) << 31) || K * 256 >= (int64_t(1) << 31))
    return fail(QAFF_E_UNSUPPORTED, "weight too large for 32-bit offsets");
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = qaff::launch_smooth_quant(x, smooth, M, K, x_q, s_x, st);
  if (e == hipSuccess) e = qaff::launch_w4a8_product(a, st);
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "this shape has no kernel");
  if (e != hipSuccess) return hip_fail(e, "smoothed w4a8 launch");
  return ok();
}

int smoothquant_factors(const float* act_absmax, const void* w, int32_t w_dtype, double alpha, float* smooth_out,
                        int64_t N, int64_t K, void* stream) {
  if (N <= 0 || K <= 0) return fail(QAFF_E_INVAL, "sizes must satisfy N > 0, K > 0");
  if (N > kMaxDim || K > kMaxDim) return fail(QAFF_E_UNSUPPORTED, "dimension above 2^30");
  if (!sb_dtype_ok(w_dtype)) return fail(QAFF_E_INVAL, "w_dtype must be BF16, F16 or F32");
  if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(QAFF_E_INVAL, "alpha must lie in [0, 1]");
  if (!act_absmax || !w || !smooth_out) return fail(QAFF_E_INVAL, "null tensor pointer");
  (void)hipGetLastError();
  hipError_t e = qaff::launch_smooth_factors(act_absmax, w, w_dtype, N, K, alpha, smooth_out,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "smoothing factors launch");
  return ok();
}

int w4a8_quantize_weights(const void* w, int32_t w_dtype, const float* smooth, uint32_t* w_q4_out, void* s_w_out,
                          int64_t N, int64_t K, void* stream) {
  if (N <= 0 || K <= 0) return fail(QAFF_E_INVAL, "sizes must satisfy N > 0, K > 0");
  if (N > kMaxDim || K > kMaxDim) return fail(QAFF_E_UNSUPPORTED, "dimension above 2^30");
  if (K % 8) return fail(QAFF_E_INVAL, "K must be a multiple of 8 (got %lld)", (long long)K);
  if (!sb_dtype_ok(w_dtype)) return fail(QAFF_E_INVAL, "w_dtype must be BF16, F16 or F32");
  if (!w || !w_q4_out || !s_w_out) return fail(QAFF_E_INVAL, "null tensor pointer");
  (void)hipGetLastError();
  hipError_t e = qaff::launch_w4a8_weights(w, w_dtype, smooth, N, K, w_q4_out, static_cast<uint16_t*>(s_w_out),
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "w4a8 weight quantization launch");
  return ok();
}

int gptq_to_affine_repack(const int32_t* qweight, const int32_t* qzeros, const void* scales, const int32_t* g_idx,
                          uint32_t* w_packed_out, void* scales_out, void* biases_out, int32_t bias_dtype,
                          int32_t* k_perm_out, int64_t K, int64_t N, int32_t group_size, void* stream) {
  if (N <= 0 || K <= 0) return fail(QAFF_E_INVAL, "sizes must satisfy N > 0, K > 0");
  if (N > kMaxDim || K > kMaxDim) return fail(QAFF_E_UNSUPPORTED, "dimension above 2^30");
  if (!group_ok(group_size)) return fail(QAFF_E_INVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
  if (K % group_size || K % 8 || N % 8) return fail(QAFF_E_INVAL, "need K %% G == 0, K %% 8 == 0, N %% 8 == 0");
  if (!(bias_dtype == QAFF_F16 || bias_dtype == QAFF_F32)) return fail(QAFF_E_INVAL, "bias_dtype must be F16 or F32");
  if (!qweight || !qzeros || !scales || !w_packed_out || !scales_out || !biases_out || !k_perm_out)
    return fail(QAFF_E_INVAL, "null tensor pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ng = K / group_size;
  // The permutation is built on the host: stable counting sort of 0..K-1 by
  // group, with a check that every group holds exactly G columns.
  std::vector<int32_t> perm(K);
  if (g_idx == nullptr) {
    for (int64_t i = 0; i < K; ++i) perm[i] = (int32_t)i;
  } else {
    std::vector<int32_t> gi(K);
    hipError_t e = hipMemcpyAsync(gi.data(), g_idx, sizeof(int32_t) * K, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading g_idx");
    std::vector<int64_t> count(ng + 1, 0);
    for (int64_t i = 0; i < K; ++i) {
      if (gi[i] < 0 || gi[i] >= ng) return fail(QAFF_E_INVAL, "g_idx[%lld]=%d is outside [0, %lld)", (long long)i, gi[i], (long long)ng);
      ++count[gi[i] + 1];
    }
    for (int64_t g = 0; g < ng; ++g)
      if (count[g + 1] != group_size)
        return fail(QAFF_E_INVAL, "group %lld holds %lld columns, not group_size=%d", (long long)g, (long long)count[g + 1], group_size);
    for (int64_t g = 0; g < ng; ++g) count[g + 1] += count[g];
    for (int64_t i = 0; i < K; ++i) perm[count[gi[i]]++] = (int32_t)i;
  }
  (void)hipGetLastError();
  hipError_t e = hipMemcpyAsync(k_perm_out, perm.data(), sizeof(int32_t) * K, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "writing k_perm");
  e = qaff::launch_gptq_repack(qweight, qzeros, scales, k_perm_out, w_packed_out, scales_out, biases_out, bias_dtype,
                               K, N, group_size, s);
  if (e != hipSuccess) return hip_fail(e, "repack launch");
  // perm lives on this host stack frame: the copy must finish before returning
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "repack");
  return ok();
}

int dequantize_affine(const uint32_t* w_packed, const void* scales, const void* biases, void* out, int64_t N,
                      int64_t K, int32_t group_size, int32_t bits, int32_t scale_dtype, int32_t bias_dtype,
                      int32_t out_dtype, void* stream) {
  if (N < 0 || K <= 0) return fail(QAFF_E_INVAL, "sizes must satisfy N >= 0, K > 0 (got %lld, %lld)", (long long)N, (long long)K);
  if (N > kMaxDim || K > kMaxDim) return fail(QAFF_E_UNSUPPORTED, "dimension above 2^30");
  if (!(bits == 2 || bits == 4 || bits == 8)) return fail(QAFF_E_INVAL, "bits must be 2, 4 or 8 (got %d)", bits);
  if (!group_ok(group_size)) return fail(QAFF_E_INVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
  if (K % group_size != 0) return fail(QAFF_E_INVAL, "K=%lld is not a multiple of group_size=%d", (long long)K, group_size);
  if (!sb_dtype_ok(scale_dtype) || !sb_dtype_ok(bias_dtype) || !sb_dtype_ok(out_dtype))
    return fail(QAFF_E_INVAL, "scale, bias and output dtypes must be BF16, F16 or F32");
  if (N == 0) return ok();
  if (!w_packed || !scales || !biases || !out) return fail(QAFF_E_INVAL, "null tensor pointer");
  if (!aligned16(out)) return fail(QAFF_E_ALIGN, "out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(w_packed) & 3u) != 0) return fail(QAFF_E_ALIGN, "w_packed must be 4-byte aligned");
  (void)hipGetLastError();
  hipError_t e = qaff::launch_dequant(w_packed, scales, biases, out, N, K, group_size, bits, scale_dtype, bias_dtype,
                                      out_dtype, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(QAFF_E_UNSUPPORTED, "weight too large");
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  return ok();
}

int quantize_pack_affine(const void* w, int32_t w_dtype, uint32_t* w_packed_out, void* scales_out, void* biases_out,
                         int32_t sb_dtype, int64_t N, int64_t K, int32_t group_size, int32_t bits, void* stream) {
  if (N < 0 || K <= 0) return fail(QAFF_E_INVAL, "sizes must satisfy N >= 0, K > 0");
  if (N > kMaxDim || K > kMaxDim) return fail(QAFF_E_UNSUPPORTED, "dimension above 2^30");
  if (!(bits == 2 || bits == 4 || bits == 8)) return fail(QAFF_E_INVAL, "bits must be 2, 4 or 8 (got %d)", bits);
  if (!group_ok(group_size)) return fail(QAFF_E_INVAL, "group_size must be 32, 64 or 128 (got %d)", group_size);
  if (K % group_size) return fail(QAFF_E_INVAL, "K is not a multiple of group_size");
  if (!sb_dtype_ok(w_dtype) || !sb_dtype_ok(sb_dtype)) return fail(QAFF_E_INVAL, "dtypes must be BF16, F16 or F32");
  if (N == 0) return ok();
  if (!w || !w_packed_out || !scales_out || !biases_out) return fail(QAFF_E_INVAL, "null tensor pointer");
  (void)hipGetLastError();
  hipError_t e = qaff::launch_quantize_pack(w, w_dtype, w_packed_out, scales_out, biases_out, sb_dtype, N, K,
                                            group_size, bits, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantize_pack launch");
  return ok();
}

}  // extern "C"
