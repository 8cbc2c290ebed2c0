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
 *     split-K partials, GPTQ partials and tables, permuted activations for
 *     k_perm) comes from a buffer the library keeps per (device, stream):
 *     calls on one stream reuse it in stream order, and once it is large
 *     enough no call allocates.  It only grows, and growing is refused
 *     (QAFF_E_HIP) while `stream` is being captured into a graph: capture a
 *     call after one eager call of the same shapes on the same stream.
 *     A captured graph keeps addressing the scratch of the stream it was
 *     captured on, whatever stream it is later replayed on.  So every graph
 *     captured on one stream (torch.cuda.graph captures on one shared
 *     stream by default), and every eager call on that stream, share one
 *     scratch buffer: their executions must not overlap in time, or they
 *     race and give wrong outputs.  Replay such graphs in stream order on
 *     one stream, or capture them on different streams.
 *     qaff_release_workspaces() frees the scratch; qmm_affine_noalloc() is
 *     the one entry point that never allocates.
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
 *   K % G == 0 (so K % (32/bits) == 0: a row is whole words).  Rows that
 *   are not whole 16-byte chunks (K*bits % 128 != 0: 2-bit codes with G = 32
 *   and K an odd multiple of 32) run a plain one-wave-per-row GEMV, also
 *   for M > 16 (in 16-row slices), slower than the main kernels.
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

/*
 * qmm_affine_noalloc - qmm_affine for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, dispatch, kernels and result as
 * qmm_affine (bit for bit), but its scratch (GEMM pre-pass buffers, split-K
 * partials, permuted x for k_perm) is a fixed device array of
 * QAFF_NOALLOC_SCRATCH_BYTES inside the library, one per device, held from
 * the library's loading until the process ends.  The call never allocates
 * or frees device memory and so may also be captured into a graph without
 * an eager call first.
 *   A call needing more scratch than the array holds returns
 *   QAFF_E_UNSUPPORTED (the message gives the size it needed); it may have
 *   enqueued kernels that wrote only the array, never y.  The 4-bit prefill
 *   at M = 2048, K = 4096 needs about 26 MiB; M <= 16 needs at most
 *   M*K*2 bytes (k_perm) plus split-K partials.
 *   Every call on a device shares that device's array, and it keeps the
 *   last call's contents (no kernel relies on it starting at zero): calls
 *   whose executions overlap on one device (other streams, concurrent
 *   graph replays) race on it and give wrong outputs.  Serialize them.
 */
#define QAFF_NOALLOC_SCRATCH_BYTES (64u << 20)
int qmm_affine_noalloc(const void *x, const uint32_t *w_packed, const void *scales, const void *biases,
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
 * qgemv_affine_silu_gate - the down projection of a gated MLP in one launch,
 * with the gated activation never written to memory (mlx_int8.rs API page,
 * `gemv_silu_gate` and `gemv_silu_gate_resid`):
 *     h[m,k]  = silu(gate[m,k]) * up[m,k],   silu(t) = t / (1 + e^-t)
 *     y[m,n]  = sum_k W[n,k] * h[m,k]  (+ resid[m,n] when resid != NULL)
 * with W as in qmm_affine.
 *   gate, up  [M, K] act_dtype (BF16 or F16), 16-byte aligned
 *   resid     [M, N] act_dtype or NULL; y may be the same buffer as resid
 *             (the residual update y += W h in place)
 *   y         [M, N] act_dtype; w_packed, scales, biases as in qmm_affine
 *   M <= 16 (QAFF_E_INVAL otherwise); K*bits % 128 == 0 (QAFF_E_UNSUPPORTED
 *   otherwise).
 * h is formed in registers in fp32 (exp and a hardware reciprocal, about
 * 1 ulp) and rounded to f16 for the dot products, so |h| must stay below
 * 65504; the codes then take the f16 path whatever act_dtype is.  Accuracy
 * as for qmm_affine.  Runs the dot2 GEMV kernel at every M.
 */
int qgemv_affine_silu_gate(const void *gate, const void *up, const void *resid, const uint32_t *w_packed,
                           const void *scales, const void *biases, void *y, int64_t M, int64_t N, int64_t K,
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
 * qgemv_affine_chain_* - the linears of a decode step (one x row) in
 * dependency order, in one launch.  A decoder layer reads its hidden state
 * in q/k/v, their result in o, o's in gate/up, and silu(gate) * up in
 * down; the fused inputs are those of the mlx_int8.rs API page
 * (`gemv_gate_up`: linears sharing one x; `gemv_silu_gate`,
 * `gemv_silu_gate_resid`: the gated input and the residual).  Each linear
 * is y = W h (+ resid) with W as in qmm_affine and
 *     h = x                        (gate == NULL)
 *     h = silu(gate) * x           (as qgemv_affine_silu_gate, x = up)
 * and its `stage`: linears of one stage run together, a stage starts when
 * every linear of every earlier stage has written y, so a linear may read
 * (as x, gate or resid) the y of any linear of an earlier stage, or any
 * buffer the caller filled.  No linear may write a buffer that a linear of
 * its own or a later stage reads, other than its own resid (y == resid is
 * the in-place residual update).
 *   x, gate  [K] act_dtype, 16-byte aligned; resid, y [N] act_dtype
 *   w_packed [N, K/8] (bits = 4 only), 16-byte aligned; scales, biases
 *            [N, K/G] in act_dtype (BF16 or F16; other combinations:
 *            QAFF_E_UNSUPPORTED); K % 32 == 0, K <= 32768, G in
 *            {32, 64, 128}
 *   stage    >= 0, nondecreasing along the array
 * qgemv_affine_chain_plan copies the descriptors to the device (it
 * synchronizes the device; the pointers are kept, not the data) and returns
 * a plan for the current device.  qgemv_affine_chain_run launches it on
 * stream (one cooperative launch, two workgroups per CU; runs of one plan
 * must not overlap).  qgemv_affine_chain_status synchronizes and sets
 * *timed_out when a run's wait between stages gave up (after about a
 * second; it cannot happen while every workgroup is resident, which the
 * cooperative launch guarantees).  qgemv_affine_chain_free releases the
 * plan (the caller's buffers are untouched).  Accuracy per linear as for
 * qmm_affine and qgemv_affine_silu_gate, each y rounded once to act_dtype.
 * On MI355X the same stages as one qgemv_affine_grouped call each, replayed
 * from a HIP graph, are faster: meeting between stages across the XCDs
 * inside a launch costs more than a launch boundary there.
 */
typedef struct qaff_chain_linear {
    const void *x;            /* [K] act_dtype; with a gate: the up projection */
    const void *gate;         /* [K] act_dtype or NULL */
    const void *resid;        /* [N] act_dtype or NULL */
    const uint32_t *w_packed; /* [N, K/8] */
    const void *scales;       /* [N, K/G] act_dtype */
    const void *biases;       /* [N, K/G] act_dtype */
    void *y;                  /* [N] act_dtype */
    int64_t N;
    int64_t K;
    int32_t stage;
} qaff_chain_linear;

int qgemv_affine_chain_plan(const qaff_chain_linear *linears, int32_t count, int32_t group_size, int32_t bits,
                            int32_t act_dtype, void **plan_out);
int qgemv_affine_chain_run(void *plan, void *stream);
int qgemv_affine_chain_status(void *plan, int32_t *timed_out);
int qgemv_affine_chain_free(void *plan);

/*
 * qmm_gptq - y[M,N] = x[M,K] . W^T for a GPTQ layer in its own layout
 * (TinyGPT "Quantization Expansion", "GPTQReader" / "Format"):
 *     W[n,i] = scales[g, n] * (q - ((qzeros[g, n/8] >> 4*(n%8)) & 15) - 1),
 *     q = (qweight[i/8, n] >> 4*(i%8)) & 15,   g = g_idx[i] (or i/G if NULL)
 *   x       [M, K]    f16, 16-byte aligned;      y [M, N] f16
 *   qweight [K/8, N]  int32 (read as uint32),   qzeros [K/G, N/8] int32
 *   scales  [K/G, N]  f16;                       g_idx [K] int32 or NULL,
 *           values in [0, K/G) (not checked on the device)
 *   K % 8 == 0, K % G == 0, N % 8 == 0, G in {32, 64, 128}.  With g_idx,
 *   each workgroup keeps a table of (scale, bias) for every group in LDS
 *   when it fits; with more groups than that, a pre-pass writes the table to
 *   library scratch and the kernel reads it through L2 (slower).  A layer
 *   without act-order (g_idx[i] = i/G) should pass g_idx = NULL: then a
 *   workgroup's table holds only the groups of its K slice.
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
 * qgemm_w4a8_tiled - qgemm_w4a8 for M > 16 with the lowering and the tile
 * chosen by the caller, for tile sweeps and tests (executorch PR #24467,
 * "What this adds": the two lowerings and their tile template parameters).
 *   staged = 0: the full-K lowering, as qgemm_w4a8 runs it: the per-token
 *     quantize kernel writes x_q and s_x, then the int8 x int4 GEMM reads
 *     them.
 *   staged = 1: one kernel.  Each workgroup takes the maxima of its rows of
 *     x, then quantizes x one 128-code K tile at a time into LDS on its way
 *     to the matrix cores (the workgroups of the first column tile also
 *     store x_q and s_x).  No x_q round trip through memory; the quantize
 *     work is repeated once per column tile.
 *   bm x bn: the output tile, one of 32x128, 64x128, 64x256, 128x256 (the
 *     K tile is 128 codes).
 * Outputs are the same bits for every lowering and tile (x_q, s_x and acc
 * exact; y the same f16 rounding of the same products), as qgemm_w4a8
 * defines them.  Other tiles and M <= 16 (the GEMV paths) return
 * QAFF_E_UNSUPPORTED; the other arguments and errors as for qgemm_w4a8.
 */
int qgemm_w4a8_tiled(const void *x, const uint32_t *w_q4, const void *s_w, void *y, int8_t *x_q, float *s_x,
                     int32_t *acc_out, int64_t M, int64_t N, int64_t K, int32_t staged, int32_t bm, int32_t bn,
                     void *stream);

/*
 * SmoothQuant ahead of W4A8 (TinyGPT "Quantization Expansion", section 3
 * "SmoothQuant"): a per-input-channel factor s moves activation range into
 * the weights, y = (x / s) . (s W)^T, so that outlier channels of x no
 * longer set the per-token int8 scale.  Three calls:
 *
 * smoothquant_factors - setup:  smooth_out[k] = act_absmax[k]^alpha /
 *     max_n |w[n,k]|^(1 - alpha), computed in fp64, stored fp32; a channel
 *     whose activation or weight maximum is 0 gets 1.
 *   act_absmax [K] f32: max over calibration tokens of |x[:, k]|, gathered
 *              by the caller; w [N, K] w_dtype (BF16, F16, F32), the dense
 *              weight before quantization; alpha in [0, 1] (0.5 usually).
 *
 * w4a8_quantize_weights - setup: the per-channel int4 weight of W4A8 from a
 *     dense weight, with the smoothing folded in when smooth != NULL:
 *       W'[n,k]  = W[n,k] * smooth[k]                (fp32, nearest even)
 *       s_w[n]   = f16( max_k |W'[n,k]| / 7 )        (fp32 division, then RNE)
 *       v[n,k]   = clamp(rint(W'[n,k] / s_w[n]), -8, 7)   (s_w as stored)
 *   w [N, K] w_dtype; smooth [K] f32 or NULL; w_q4_out [N, K/8] uint32
 *   (the qgemm_w4a8 layout); s_w_out [N] f16.  K % 8 == 0.  A row of zeros
 *   gets s_w = 0 and codes 0.  Bit-exact (IEEE divisions, rint to even).
 *
 * qgemm_w4a8_smooth - qgemm_w4a8 on the smoothed activations:
 *       xs[m,k] = f32(x[m,k]) / smooth[k]             (IEEE division)
 *     then s_x, x_q, acc and y exactly as qgemm_w4a8 defines them, with xs
 *     in place of x (w_q4 and s_w from w4a8_quantize_weights with the same
 *     smooth).  smooth [K] f32, finite and nonzero; the other arguments as
 *     for qgemm_w4a8.  Two launches: the smoothed quantizer, then the
 *     integer product.
 */
int smoothquant_factors(const float *act_absmax, const void *w, int32_t w_dtype, double alpha, float *smooth_out,
                        int64_t N, int64_t K, void *stream);
int w4a8_quantize_weights(const void *w, int32_t w_dtype, const float *smooth, uint32_t *w_q4_out, void *s_w_out,
                          int64_t N, int64_t K, void *stream);
int qgemm_w4a8_smooth(const void *x, const float *smooth, const uint32_t *w_q4, const void *s_w, void *y,
                      int8_t *x_q, float *s_x, int32_t *acc_out, int64_t M, int64_t N, int64_t K, void *stream);

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

/*
 * dequantize_affine - write the whole weight as a dense array (the
 * standalone dequantization of the mlx_int8.rs API page, `dequantize_to`,
 * which writes BF16; Transformers "Metal" page, "Dequantize"):
 *     out[n, k] = RNE_out( q(n,k) * scales[n, k/G] + biases[n, k/G] )
 * with q as in qmm_affine and the product and sum evaluated exactly (fp64)
 * before the one rounding to out_dtype (round to nearest, ties to even).
 *   w_packed [N, K*bits/32] uint32, 4-byte aligned
 *   scales, biases [N, K/G] in scale_dtype / bias_dtype (BF16, F16, F32)
 *   out      [N, K] out_dtype (BF16, F16 or F32), 16-byte aligned
 *   group_size in {32, 64, 128}; bits in {2, 4, 8}; K % G == 0.
 * Asynchronous on `stream`; allocates nothing.  Memory-bound: reads
 * N*K*bits/8 + parameter bytes, writes N*K*sizeof(out).
 */
int dequantize_affine(const uint32_t *w_packed, const void *scales, const void *biases, void *out, int64_t N,
                      int64_t K, int32_t group_size, int32_t bits, int32_t scale_dtype, int32_t bias_dtype,
                      int32_t out_dtype, void *stream);

/*
 * qaff_release_workspaces - free all scratch the library holds: the buffer
 * kept per (device, stream) and every buffer grown out of since the last
 * release, on every device.  This is the release half of the caller-frees-
 * once convention of the mlx_int8.rs API page (`release` frees a weight's
 * buffers exactly once): scratch has no other owner, so the caller decides
 * when it goes.
 *   Safe only when (1) no work enqueued through this library is still
 *   pending on any stream (synchronize first), and (2) no captured graph
 *   that contains a call of this library will be replayed again (destroy
 *   such graphs first): their kernels hold the freed addresses.
 *   The next call that needs scratch allocates again.
 *   freed_bytes (HOST pointer, may be NULL) receives the bytes of the
 *   per-stream buffers that were cached (grown-out ones not counted).
 *   Returns QAFF_OK, or QAFF_E_HIP if a hipFree failed (every buffer is
 *   still forgotten, and the rest are freed).  Not to be called while other
 *   threads make library calls.
 */
int qaff_release_workspaces(uint64_t *freed_bytes);

/* Message for the calling thread's last non-OK status ("" if none).  The
 * string is owned by the library and valid until the thread's next call. */
const char *qaff_last_error(void);

/*
 * qaff_stream_read - measurement helper, not part of the matmul path: read
 * `bytes` (a positive multiple of 16) at `src` with non-temporal 16-byte
 * loads by `blocks` workgroups of 256 threads, and write one word per
 * thread to `sink` (blocks*256 uint32).  Timing it over a buffer much larger
 * than the last-level cache gives the device's achievable streaming-read
 * rate, the ceiling quoted beside the published HBM peak.
 */
int qaff_stream_read(const void *src, uint64_t bytes, uint32_t *sink, int32_t blocks, void *stream);

/* Library version, as major*10000 + minor*100 + patch. */
int qaff_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QAFF_H */
