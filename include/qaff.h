/*
 * qaff.h - C ABI of libqaff.so: group-wise affine quantized matmul on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (y = x . W^T with W stored as packed integer codes plus
 * per-group scales and biases) is the fused dequantize + matmul described on:
 *   - "metrale_gpu_runtime/mlx_int8.rs" API page, module docs "Layout"
 *     (uint32 words, lowest column in the low bits, w = code*scale + bias with
 *     group c/G) and the `gemv` / `gemm` docs (y = W x, Y = X W^T);
 *   - Transformers docs, "Metal" quantization page, intro (codes packed in
 *     uint32 with per-group scales and biases, bit widths 2/4/8, configurable
 *     group size, one fused dequant+matmul kernel);
 *   - TinyGPT "Quantization Expansion", section 1 "GPTQReader", "Format"
 *     (GPTQ qweight/qzeros/scales/g_idx and the "+1" zero rule);
 *   - executorch PR #24467 (mlx::int8_int4_gemm), "What this adds" (dynamic
 *     per-token int8 activations x per-channel int4 weights, int32 sums).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (HIP global memory) unless a
 *     comment says otherwise.  Tensors are dense and row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it asynchronously; hot-path calls never synchronize.
 *   - The caller owns every buffer; the library keeps no pointer to them
 *     after the call returns.  Internal scratch (GEMM pre-pass buffers and
 *     split-K partials, GPTQ partials, permuted activations for k_perm) comes
 *     from a buffer the library keeps per (device, stream): calls on one
 *     stream reuse it in stream order, and once it is large enough no call
 *     allocates.  It only grows, and growing is refused (QAFF_E_HIP) while
 *     `stream` is being captured into a graph: capture a call after one
 *     eager call of the same shapes on the same stream.
 *   - Errors are returned as qaff_status codes; no C++ exception crosses the
 *     ABI.  Argument checks run before any HIP call, so a rejected call has
 *     enqueued nothing.  qaff_last_error() gives a message for the calling
 *     thread's last non-OK status.  Faults inside kernels surface at the
 *     caller's next synchronization, as for any HIP work.
 *   - M == 0 (or N == 0) returns QAFF_OK without launching anything.
 *   - Calls are reentrant; overlapping calls that share output buffers race,
 *     as any two kernels writing the same memory would.
 */
#ifndef QAFF_H
#define QAFF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QAFF_OK = 0,
    QAFF_E_INVAL = 1,        /* bad argument: null pointer, negative size, bad bits/G, shape rule */
    QAFF_E_UNSUPPORTED = 2,  /* valid combination that this library does not implement */
    QAFF_E_ALIGN = 3,        /* a pointer is not aligned as the kernels require (16 bytes) */
    QAFF_E_HIP = 4           /* a HIP runtime call or launch failed */
} qaff_status;

typedef enum {
    QAFF_BF16 = 0,
    QAFF_F16 = 1,
    QAFF_F32 = 2
} qaff_dtype;

/*
 * qmm_affine - y[M,N] = x[M,K] . W[N,K]^T with
 *     W[n,k] = q(n,k) * scales[n, k/G] + biases[n, k/G]
 *     q(n,k) = (w_packed[n, k/P] >> (bits * (k % P))) & (2^bits - 1),  P = 32/bits
 * (mlx_int8.rs "Layout" for 8 bits; the same low-bits-first rule for 2 and 4).
 *
 *   x         [M, K]        act_dtype (QAFF_BF16 or QAFF_F16), 16-byte aligned
 *   w_packed  [N, K*bits/32] uint32, 16-byte aligned
 *   scales    [N, K/G]      scale_dtype (BF16, F16 or F32)
 *   biases    [N, K/G]      bias_dtype  (BF16, F16 or F32)
 *   k_perm    [K] int32 or NULL.  When given, x is read as x[m, k_perm[k]]:
 *             column k of W pairs with column k_perm[k] of x.  This is how a
 *             GPTQ act-order layer runs after gptq_to_affine_repack.  Values
 *             must lie in [0, K) (not checked on the device).
 *   y         [M, N]        act_dtype, written with round-to-nearest-even
 *   group_size G in {32, 64, 128}; bits in {2, 4, 8};
 *   K % G == 0 and K*bits % 128 == 0 (whole 16-byte loads per row).
 *
 * Dispatch: M <= 16 runs a memory-bound GEMV kernel (exact fp32 arithmetic
 * on the integer codes; 4-bit codes with 2..16 x rows on the matrix cores,
 * except a narrow call with M <= 4; K split over workgroups, plus a summing
 * pass, when a call gives the matrix-core kernel 64 workgroups or fewer),
 * after one permuting pass over x when k_perm is given.  17 <= M <= 48 with
 * 4-bit codes and scales and biases in the activation dtype runs as 16-row
 * slices of that GEMV.  Otherwise larger M runs a pre-pass plus the MFMA
 * GEMM kernel, with K split over workgroups (and a summing pass) when the
 * output tiles would leave CUs idle.  Accuracy: max|y-ref|/(|ref|+1) <= 1e-2
 * and relative Frobenius error <= 5e-3 against an fp64 evaluation, for
 * finite inputs.
 */
int qmm_affine(const void *x, const uint32_t *w_packed, const void *scales, const void *biases,
               const int32_t *k_perm, void *y, int64_t M, int64_t N, int64_t K,
               int32_t group_size, int32_t bits, int32_t act_dtype, int32_t scale_dtype,
               int32_t bias_dtype, void *stream);

/* qgemv_affine - same arguments and result as qmm_affine, but always runs the
 * GEMV kernel; M must be <= 16 (QAFF_E_INVAL otherwise). */
int qgemv_affine(const void *x, const uint32_t *w_packed, const void *scales, const void *biases,
                 const int32_t *k_perm, void *y, int64_t M, int64_t N, int64_t K,
                 int32_t group_size, int32_t bits, int32_t act_dtype, int32_t scale_dtype,
                 int32_t bias_dtype, void *stream);

/*
 * qgemv_affine_grouped - `count` independent GEMVs y_i = x_i . W_i^T of the
 * qmm_affine form, computed by as few kernel launches as possible (one per
 * 56 problems).  This is the multi-weight decode GEMV: linears that read the
 * same input (q/k/v, gate/up) pass the same x, and each problem keeps its own
 * weights, parameters and output.  It serves decode with M <= 16, where one
 * launch per small matrix costs more time in launch latency than in reading
 * the weights (mlx_int8.rs API page, `gemv`: y = W x over the packed layout).
 *
 *   problems  HOST array of `count` descriptors (read during the call only);
 *             every pointer in it is a device pointer with the meaning,
 *             layout and alignment of the qmm_affine argument of that name
 *   count     0 <= count <= 65536; 0 returns QAFF_OK
 *   M, group_size, bits, act_dtype, scale_dtype, bias_dtype
 *             shared by every problem, with the qmm_affine rules; M <= 16
 *   Each problem is checked as qgemv_affine would check it; the first bad
 *   one fails the whole call before anything is launched.  Outputs of
 *   different problems must not overlap.
 */
typedef struct qaff_gemv_problem {
    const void *x;            /* [M, K] act_dtype */
    const uint32_t *w_packed; /* [N, K*bits/32] */
    const void *scales;       /* [N, K/G] */
    const void *biases;       /* [N, K/G] */
    const int32_t *k_perm;    /* [K] or NULL */
    void *y;                  /* [M, N] act_dtype */
    int64_t N;
    int64_t K;
} qaff_gemv_problem;

int qgemv_affine_grouped(const qaff_gemv_problem *problems, int32_t count, int64_t M,
                         int32_t group_size, int32_t bits, int32_t act_dtype, int32_t scale_dtype,
                         int32_t bias_dtype, void *stream);

/*
 * qmm_gptq - y[M,N] = x[M,K] . W^T for a GPTQ layer in its own layout
 * (TinyGPT "Quantization Expansion", "GPTQReader" / "Format"):
 *     W[n,i] = scales[g, n] * (q - ((qzeros[g, n/8] >> 4*(n%8)) & 15) - 1),
 *     q = (qweight[i/8, n] >> 4*(i%8)) & 15,   g = g_idx[i] (or i/G if NULL)
 *   x       [M, K]    f16, 16-byte aligned;      y [M, N] f16
 *   qweight [K/8, N]  int32 (read as uint32),   qzeros [K/G, N/8] int32
 *   scales  [K/G, N]  f16;                       g_idx [K] int32 or NULL,
 *           values in [0, K/G) (not checked on the device)
 *   K % 8 == 0, K % G == 0, N % 8 == 0, G in {32, 64, 128}; with g_idx, at
 *   most 192 groups (K/G), else QAFF_E_UNSUPPORTED (the per-workgroup table
 *   of scales and zeros for every group must fit in LDS).  A layer without
 *   act-order (g_idx[i] = i/G) should pass g_idx = NULL: then a workgroup's
 *   table holds only the groups of its K slice, and any K/G is taken.
 * Kernels: M < 8 on the VALU (w exact in fp32); M >= 8 on the matrix cores
 * (w as two exact fp16 pieces relative to each column's largest scale in
 * the table) when g_idx is NULL or there are at most 96 groups, else on
 * the VALU; fp32 partial sums over K slices, then one summing pass.
 * Accuracy as for qmm_affine.
 */
int qmm_gptq(const void *x, const int32_t *qweight, const int32_t *qzeros, const void *scales,
             const int32_t *g_idx, void *y, int64_t M, int64_t N, int64_t K, int32_t group_size,
             void *stream);

/*
 * qgemm_w4a8 - int8 dynamic-activation x int4 per-channel-weight GEMM
 * (executorch PR #24467, "What this adds"):
 *     s_x[m]   = max_k |x[m,k]| / 127                 (IEEE fp32 division)
 *     x_q[m,k] = clamp(rint(x[m,k] / s_x[m]), -127, 127), round half to even;
 *                an all-zero row gives s_x = 0 and codes 0
 *     acc[m,n] = sum_k x_q[m,k] * v[n,k]             (exact int32)
 *     y[m,n]   = f16( (float(acc) * s_x[m]) * s_w[n] )
 *   x       [M, K]    f16
 *   w_q4    [N, K/8]  uint32; nibble k%8 of word k/8 is v[n,k] in two's
 *                     complement, range [-8, 7]; 16-byte aligned
 *   s_w     [N]       f16
 *   y       [M, N]    f16 (output)
 *   x_q     [M, K]    int8 (output, caller-owned; the quantized activations)
 *   s_x     [M]       f32  (output, caller-owned)
 *   acc_out [M, N]    int32 or NULL (output; the accumulators, for checking)
 *   K % 32 == 0.  Launches on `stream`: for M <= 16 and K <= 4096 one kernel
 *   (every workgroup quantizes x into LDS, workgroup 0 also writes x_q and
 *   s_x, then a dot4 GEMV); otherwise quantize, then the integer product (a
 *   dot4 GEMV for M <= 16, else the int8 MFMA GEMM, plus a summing pass over
 *   int32 partials when K is split).
 */
int qgemm_w4a8(const void *x, const uint32_t *w_q4, const void *s_w, void *y, int8_t *x_q, float *s_x,
               int32_t *acc_out, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * gptq_to_affine_repack - rewrite a GPTQ layer in the affine layout
 * (setup call; it MAY SYNCHRONIZE `stream`: it reads g_idx back to the host
 * to build the permutation and to check it).
 *     perm          = stable sort of 0..K-1 by g_idx (ties keep column order)
 *     w_packed_out  [N, K/8] uint32, code j of row n = q(perm[j], n)
 *     scales_out    [N, K/G] f16,  scales_out[n, g] = scales[g, n]
 *     biases_out    [N, K/G] bias_dtype (F32 exact, or F16 rounded to nearest
 *                   even): -scales[g, n] * (z_stored[g, n] + 1)
 *     k_perm_out    [K] int32, = perm; pass it as k_perm to qmm_affine
 * Then code*scale + bias reproduces scale*(q - zero) of the GPTQ recipe.
 * QAFF_E_INVAL if some group does not hold exactly G columns or a g_idx value
 * is out of range.  g_idx NULL means g_idx[i] = i/G (perm = identity).
 */
int gptq_to_affine_repack(const int32_t *qweight, const int32_t *qzeros, const void *scales,
                          const int32_t *g_idx, uint32_t *w_packed_out, void *scales_out,
                          void *biases_out, int32_t bias_dtype, int32_t *k_perm_out, int64_t K,
                          int64_t N, int32_t group_size, void *stream);

/*
 * quantize_pack_affine - quantize a dense weight into the affine layout
 * (the on-load quantization of the Transformers "Metal" page; the page gives
 * no formula, this is the min/max affine rule):
 *   per row n and group g, in IEEE fp32:
 *     scale = (max - min) / (2^bits - 1), stored in sb_dtype (nearest even)
 *     bias  = min, stored in sb_dtype
 *     q     = clamp(rint((w - bias_stored) / scale_stored), 0, 2^bits - 1),
 *             0 when scale_stored == 0
 *   w            [N, K] w_dtype (BF16, F16 or F32)
 *   w_packed_out [N, K*bits/32] uint32;  scales_out, biases_out [N, K/G] sb_dtype
 */
int quantize_pack_affine(const void *w, int32_t w_dtype, uint32_t *w_packed_out, void *scales_out,
                         void *biases_out, int32_t sb_dtype, int64_t N, int64_t K, int32_t group_size,
                         int32_t bits, void *stream);

/* Message for the calling thread's last non-OK status ("" if none).  The
 * string is owned by the library and valid until the thread's next call. */
const char *qaff_last_error(void);

/* Library version, as major*10000 + minor*100 + patch. */
int qaff_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QAFF_H */
