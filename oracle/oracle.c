/*
 * Reference CPU implementation of the group-wise affine dequant + matmul path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP kernels are
 * checked against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load it.  It shares no code, header, table or helper with the
 * HIP library; the library never loads it.
 *
 * Everything is plain and slow on purpose: fp64 dequantization of every
 * weight, then a triple loop y[m,n] = sum_k x[m,k] * w[n,k] with k ascending.
 * OpenMP splits the output columns n across threads; it does not change any
 * sum.  Build with -O2 -fno-fast-math -ffp-contract=off so that float code
 * below is evaluated exactly as written (IEEE single/double, round to nearest
 * even, no fused multiply-add).
 *
 * Sources (page title, then section):
 *   [MLX8]  metrale_gpu_runtime mlx_int8.rs API page: module docs "Layout"
 *           (uint32 words, low byte = lowest column; dequant byte*scale+bias
 *           with group c/G), `gemm` doc (Y = X W^T).
 *   [METAL] Transformers docs, "Metal" quantization: intro (uint32-packed
 *           codes with per-group scales and biases, bits 2/4/8, fused
 *           dequant+matmul), "Dequantize" section (packed -> float).
 *   [GPTQ]  TinyGPT "Quantization Expansion", section 1 "GPTQReader":
 *           "Format" (qweight/scales/qzeros/g_idx shapes) and the dequant
 *           recipe with the "+1" zero convention.
 *   [W4A8]  executorch PR #24467 (mlx::int8_int4_gemm), "What this adds":
 *           dynamic symmetric per-token int8 activations x symmetric
 *           per-channel int4 weights, int32 accumulation.
 *   [QAT]   TinyGPT "Quantization Expansion", section 4 "Fake-quant + STE":
 *           symmetric scale = max|row| / qMax, round, clip to +-qMax.
 *
 * Readings where the pages are silent are marked READING and listed in the
 * design notes.  Pinned by tests/test_oracle_pins.py; no function here is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* storage dtype tags used by this file's API */
enum { OR_BF16 = 0, OR_F16 = 1, OR_F32 = 2 };

/* error returns */
enum { OR_OK = 0, OR_EARG = -1, OR_EGROUP = -2, OR_ERANGE = -3, OR_EMEM = -4 };

/* ---------------------------------------------------------------------- */
/* IEEE storage formats, from their definitions                           */

/* bfloat16 is the top half of an IEEE single. */
static double bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                  /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);      /* (1.m) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a double to binary16, round-to-nearest-even. */
static uint16_t f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7e00);
    if (a >= 65520.0)                 /* 65504 + half an ulp rounds to even = inf */
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {        /* subnormal grid: multiples of 2^-24 */
        double m = nearbyint(a * 16777216.0);
        return (uint16_t)(sign | (uint16_t)m);   /* m == 1024 is the smallest normal */
    }
    int e;
    double f = frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
    double m = nearbyint(ldexp(f, 11)); /* 11 significant bits, in [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    int biased = e - 1 + 15;
    if (biased >= 31)
        return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)((int)m - 1024));
}

/* Round an IEEE single to bfloat16, round-to-nearest-even on the 16 dropped bits. */
static uint16_t f32_to_bf16(float v)
{
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);  /* quiet NaN */
    uint32_t keep = u >> 16, rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u)))
        keep += 1;                                /* carries into the exponent as it should */
    return (uint16_t)keep;
}

/* element i of a bf16 / f16 / f32 array, widened to double (exact) */
static double load_f64(const void *base, int64_t i, int dtype)
{
    switch (dtype) {
    case OR_BF16: return bf16_to_f64(((const uint16_t *)base)[i]);
    case OR_F16:  return f16_to_f64(((const uint16_t *)base)[i]);
    default:      return (double)((const float *)base)[i];
    }
}

static int dtype_ok(int d) { return d == OR_BF16 || d == OR_F16 || d == OR_F32; }

/* exported conversions, so the tests can pin them against library converters */
void oracle_to_f64(const void *src, int dtype, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = load_f64(src, i, dtype);
}

void oracle_f64_to_f16(const double *src, int64_t n, uint16_t *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = f64_to_f16(src[i]);
}

void oracle_f32_to_bf16(const float *src, int64_t n, uint16_t *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = f32_to_bf16(src[i]);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing of the oracle as a CPU baseline;
 * no result depends on the thread count). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------------- */
/* O1  affine code unpack  [MLX8 "Layout"; METAL intro]                    */
/*                                                                        */
/* A row of K codes of `bits` bits is stored in K*bits/32 uint32 words,    */
/* P = 32/bits codes per word, code k in bits [bits*(k%P), bits*(k%P+1))   */
/* of word k/P: the lowest column sits in the low bits.  The 8-bit rule is */
/* printed on [MLX8]; READING: 2- and 4-bit follow the same rule.           */

static inline unsigned code_at(const uint32_t *row, int64_t k, int bits)
{
    int per = 32 / bits;
    uint32_t word = row[k / per];
    unsigned shift = (unsigned)(bits * (k % per));
    return (unsigned)((word >> shift) & ((1u << bits) - 1u));
}

static int affine_args_ok(int64_t N, int64_t K, int G, int bits)
{
    if (!(bits == 2 || bits == 4 || bits == 8)) return 0;
    if (N < 0 || K < 0 || G <= 0) return 0;
    if (K % G != 0) return 0;
    if ((K * bits) % 32 != 0) return 0;
    return 1;
}

int oracle_unpack_affine(const uint32_t *packed, int64_t N, int64_t K, int bits, uint8_t *codes)
{
    if (!(bits == 2 || bits == 4 || bits == 8) || (K * bits) % 32) return OR_EARG;
    int64_t wpr = K * bits / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)code_at(packed + n * wpr, k, bits);
    return OR_OK;
}

/* O2  dequantize one row to fp64:  w[k] = q(k) * scale[k/G] + bias[k/G]   */
/* [MLX8 "Layout"; METAL intro and "Dequantize"].  q*scale has at most     */
/* 8+24 significant bits and the sum with the bias is exact in fp64 for    */
/* every bf16/f16 scale and bias; f32 scales are within one fp64 rounding.  */
static void dequant_affine_row(const uint32_t *packed_row, const void *scales, int s_dtype,
                               const void *biases, int b_dtype, int64_t n, int64_t K, int G, int bits,
                               double *w)
{
    int64_t ng = K / G;
    for (int64_t k = 0; k < K; ++k) {
        double q = (double)code_at(packed_row, k, bits);
        double s = load_f64(scales, n * ng + k / G, s_dtype);
        double b = load_f64(biases, n * ng + k / G, b_dtype);
        w[k] = q * s + b;
    }
}

int oracle_dequant_affine(const uint32_t *packed, const void *scales, int s_dtype, const void *biases,
                          int b_dtype, int64_t N, int64_t K, int G, int bits, double *w)
{
    if (!affine_args_ok(N, K, G, bits) || !dtype_ok(s_dtype) || !dtype_ok(b_dtype)) return OR_EARG;
    int64_t wpr = K * bits / 32;
    for (int64_t n = 0; n < N; ++n)
        dequant_affine_row(packed + n * wpr, scales, s_dtype, biases, b_dtype, n, K, G, bits, w + n * K);
    return OR_OK;
}

/* O3  y[m,n] = sum_{k ascending} x[m, kp(k)] * w[n,k]   [MLX8 `gemm` doc] */
/* kp = k_perm when given (x read through a column permutation, which is   */
/* how a GPTQ act-order layer looks after repacking), else identity.       */
int oracle_qmm_affine(const void *x, int act_dtype, const uint32_t *packed, const void *scales,
                      int s_dtype, const void *biases, int b_dtype, const int32_t *k_perm,
                      int64_t M, int64_t N, int64_t K, int G, int bits, double *y)
{
    if (!affine_args_ok(N, K, G, bits) || M < 0 || !dtype_ok(s_dtype) || !dtype_ok(b_dtype) ||
        !dtype_ok(act_dtype))
        return OR_EARG;
    if (k_perm)
        for (int64_t k = 0; k < K; ++k)
            if (k_perm[k] < 0 || k_perm[k] >= K) return OR_ERANGE;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    if (!xd) return OR_EMEM;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            xd[m * K + k] = load_f64(x, m * K + (k_perm ? k_perm[k] : k), act_dtype);
    int64_t wpr = K * bits / 32;
    int fail = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(K + 1));
        if (!w) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            if (!w) continue;
            dequant_affine_row(packed + n * wpr, scales, s_dtype, biases, b_dtype, n, K, G, bits, w);
            for (int64_t m = 0; m < M; ++m) {
                const double *xr = xd + m * K;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += xr[k] * w[k];
                y[m * N + n] = acc;
            }
        }
        free(w);
    }
    free(xd);
    return fail ? OR_EMEM : OR_OK;
}

/* ---------------------------------------------------------------------- */
/* G1  GPTQ dequant  [GPTQ "Format" and the dequant recipe]                */
/*                                                                        */
/* qweight int32 [K/8, N]: 8 codes per word along K, code i in nibble i%8. */
/* qzeros  int32 [K/G, N/8]: 8 zero points per word along N, stored as     */
/*         zero-1 (the "+1" convention).  scales f16 [K/G, N].            */
/* g_idx   int32 [K] or NULL (then i/G).                                  */
/* W[o,i] = scale[g,o] * (q - (z_stored + 1)), g = g_idx[i].              */
/* READING: words are read as uint32 before shifting (the sign bit of an   */
/* int32 word is just the top nibble's high bit).                         */

static inline unsigned nib(int32_t word, int j)
{
    return (unsigned)(((uint32_t)word >> (4 * j)) & 0xFu);
}

static int gptq_args_ok(int64_t K, int64_t N, int G)
{
    return K > 0 && N > 0 && G > 0 && K % G == 0 && K % 8 == 0 && N % 8 == 0;
}

static int gidx_ok(const int32_t *g_idx, int64_t K, int G)
{
    if (!g_idx) return 1;
    for (int64_t i = 0; i < K; ++i)
        if (g_idx[i] < 0 || g_idx[i] >= K / G) return 0;
    return 1;
}

static void dequant_gptq_row(const int32_t *qweight, const int32_t *qzeros, const uint16_t *scales,
                             const int32_t *g_idx, int64_t K, int64_t N, int G, int64_t o, double *w)
{
    for (int64_t i = 0; i < K; ++i) {
        double q = (double)nib(qweight[(i / 8) * N + o], (int)(i % 8));
        int64_t g = g_idx ? g_idx[i] : i / G;
        double s = f16_to_f64(scales[g * N + o]);
        double z = (double)nib(qzeros[g * (N / 8) + o / 8], (int)(o % 8)) + 1.0;
        w[i] = s * (q - z);
    }
}

int oracle_dequant_gptq(const int32_t *qweight, const int32_t *qzeros, const uint16_t *scales,
                        const int32_t *g_idx, int64_t K, int64_t N, int G, double *w)
{
    if (!gptq_args_ok(K, N, G)) return OR_EARG;
    if (!gidx_ok(g_idx, K, G)) return OR_ERANGE;
    for (int64_t o = 0; o < N; ++o)
        dequant_gptq_row(qweight, qzeros, scales, g_idx, K, N, G, o, w + o * K);
    return OR_OK;
}

/* y[m,o] = sum_i x[m,i] * W[o,i]; x f16 [M, K] */
int oracle_qmm_gptq(const uint16_t *x, const int32_t *qweight, const int32_t *qzeros, const uint16_t *scales,
                    const int32_t *g_idx, int64_t M, int64_t K, int64_t N, int G, double *y)
{
    if (!gptq_args_ok(K, N, G) || M < 0) return OR_EARG;
    if (!gidx_ok(g_idx, K, G)) return OR_ERANGE;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    if (!xd) return OR_EMEM;
    for (int64_t i = 0; i < M * K; ++i)
        xd[i] = f16_to_f64(x[i]);
    int fail = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(K + 1));
        if (!w) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static)
        for (int64_t o = 0; o < N; ++o) {
            if (!w) continue;
            dequant_gptq_row(qweight, qzeros, scales, g_idx, K, N, G, o, w);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t i = 0; i < K; ++i)
                    acc += xd[m * K + i] * w[i];
                y[m * N + o] = acc;
            }
        }
        free(w);
    }
    free(xd);
    return fail ? OR_EMEM : OR_OK;
}

/* G2  GPTQ -> affine repack.                                              */
/* perm = stable sort of 0..K-1 by g_idx (ties by position); every group   */
/* must hold exactly G columns, else OR_EGROUP.  Then                      */
/*   code_aff[n, j]  = q(perm[j], n)        packed 8 per word along j      */
/*   scale_aff[n, g] = scale[g, n]          (f16 bits copied)              */
/*   bias_aff[n, g]  = -scale[g, n] * (z_stored[g, n] + 1)                 */
/*   k_perm[j]       = perm[j]                                             */
/* so that code_aff*scale_aff + bias_aff = scale*(q - zero) term by term   */
/* [GPTQ recipe].  The bias is exact in f32 (11-bit scale times a 5-bit    */
/* integer); bias_dtype OR_F16 rounds it to nearest even.                  */
int oracle_gptq_to_affine_repack(const int32_t *qweight, const int32_t *qzeros, const uint16_t *scales,
                                 const int32_t *g_idx, int64_t K, int64_t N, int G, int bias_dtype,
                                 uint32_t *packed_out, uint16_t *scales_out, void *biases_out,
                                 int32_t *k_perm_out)
{
    if (!gptq_args_ok(K, N, G) || !(bias_dtype == OR_F16 || bias_dtype == OR_F32)) return OR_EARG;
    if (!gidx_ok(g_idx, K, G)) return OR_ERANGE;
    int64_t ng = K / G;
    /* stable selection: walk the groups in order, and within a group the columns in order */
    int64_t j = 0;
    for (int64_t g = 0; g < ng; ++g) {
        int64_t count = 0;
        for (int64_t i = 0; i < K; ++i) {
            int64_t gi = g_idx ? g_idx[i] : i / G;
            if (gi == g) {
                if (count == G) return OR_EGROUP;
                k_perm_out[j++] = (int32_t)i;
                ++count;
            }
        }
        if (count != G) return OR_EGROUP;
    }
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t w = 0; w < K / 8; ++w) {
            uint32_t word = 0;
            for (int e = 0; e < 8; ++e) {
                int64_t i = k_perm_out[w * 8 + e];
                word |= (uint32_t)nib(qweight[(i / 8) * N + n], (int)(i % 8)) << (4 * e);
            }
            packed_out[n * (K / 8) + w] = word;
        }
        for (int64_t g = 0; g < ng; ++g) {
            uint16_t sb = scales[g * N + n];
            double s = f16_to_f64(sb);
            double zs = (double)nib(qzeros[g * (N / 8) + n / 8], (int)(n % 8));
            double b = -s * (zs + 1.0);
            scales_out[n * ng + g] = sb;
            if (bias_dtype == OR_F32)
                ((float *)biases_out)[n * ng + g] = (float)b;
            else
                ((uint16_t *)biases_out)[n * ng + g] = f64_to_f16(b);
        }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------- */
/* W4A8  [W4A8 "What this adds"; symmetric rule as in QAT]                 */
/*                                                                        */
/* Q1 amax[m] = max_k |x[m,k]|           (f16 -> f32 is exact)            */
/* Q2 s_x[m]  = amax / 127               (IEEE single division)           */
/* Q3 q[m,k]  = clamp(rint(x / s_x), -127, 127), rint = nearest even;     */
/*    READING: an all-zero row has s_x = 0 and codes 0.                   */
int oracle_w4a8_quantize_act(const uint16_t *x, int64_t M, int64_t K, int8_t *q, float *s_x)
{
    if (M < 0 || K <= 0) return OR_EARG;
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf((float)f16_to_f64(x[m * K + k]));
            if (a > amax) amax = a;
        }
        float s = amax / 127.0f;
        s_x[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)f16_to_f64(x[m * K + k]);
            float t = 0.0f;
            if (s != 0.0f) {
                t = rintf(v / s);
                if (t > 127.0f) t = 127.0f;
                if (t < -127.0f) t = -127.0f;
            }
            q[m * K + k] = (int8_t)t;
        }
    }
    return OR_OK;
}

/* Q4 weight nibble -> two's complement value in [-8, 7]                   */
/* READING: w_q4 is [N, K/8] uint32, nibble k%8 of word k/8 = column k.   */
static inline int s4_at(const uint32_t *row, int64_t k)
{
    int v = (int)((row[k / 8] >> (4 * (k % 8))) & 0xFu);
    return v >= 8 ? v - 16 : v;
}

/* Q5 acc[m,n] = sum_k q[m,k] * v[n,k], exact in int64 */
int oracle_w4a8_acc(const int8_t *q, const uint32_t *w_q4, int64_t M, int64_t N, int64_t K, int64_t *acc)
{
    if (M < 0 || N < 0 || K <= 0 || K % 8) return OR_EARG;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t *row = w_q4 + n * (K / 8);
        for (int64_t m = 0; m < M; ++m) {
            int64_t a = 0;
            for (int64_t k = 0; k < K; ++k)
                a += (int64_t)q[m * K + k] * (int64_t)s4_at(row, k);
            acc[m * N + n] = a;
        }
    }
    return OR_OK;
}

/* Q1..Q6: codes, scales, int64 accumulators, and y = acc * s_x * s_w in fp64 */
int oracle_w4a8(const uint16_t *x, const uint32_t *w_q4, const uint16_t *s_w, int64_t M, int64_t N, int64_t K,
                int8_t *q, float *s_x, int64_t *acc, double *y)
{
    int rc = oracle_w4a8_quantize_act(x, M, K, q, s_x);
    if (rc) return rc;
    rc = oracle_w4a8_acc(q, w_q4, M, N, K, acc);
    if (rc) return rc;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t a = acc[m * N + n];
            if (a > INT32_MAX || a < INT32_MIN) return OR_ERANGE;
            y[m * N + n] = (double)a * (double)s_x[m] * f16_to_f64(s_w[n]);
        }
    return OR_OK;
}

/* ---------------------------------------------------------------------- */
/* A1..A3  quantize_pack_affine  [METAL "quantize on the fly"]             */
/*                                                                        */
/* READING (the pages give no formula; plainest min/max affine):          */
/* per row n and group g, in IEEE single:                                 */
/*   lo = min, hi = max over the group                                    */
/*   scale = (hi - lo) / (2^bits - 1), rounded to sb_dtype                 */
/*   bias  = lo, rounded to sb_dtype                                       */
/*   q     = clamp(rint((w - bias) / scale), 0, 2^bits - 1), or 0 when the */
/*           stored scale is 0                                             */
/* then codes are packed as in O1.                                         */
static float round_to(float v, int dtype)
{
    if (dtype == OR_BF16) {
        uint16_t h = f32_to_bf16(v);
        return (float)bf16_to_f64(h);
    }
    if (dtype == OR_F16)
        return (float)f16_to_f64(f64_to_f16((double)v));
    return v;
}

static void store_as(void *base, int64_t i, int dtype, float v)
{
    if (dtype == OR_BF16)
        ((uint16_t *)base)[i] = f32_to_bf16(v);
    else if (dtype == OR_F16)
        ((uint16_t *)base)[i] = f64_to_f16((double)v);
    else
        ((float *)base)[i] = v;
}

int oracle_quantize_pack_affine(const void *w, int w_dtype, int64_t N, int64_t K, int G, int bits,
                                int sb_dtype, uint32_t *packed, void *scales, void *biases)
{
    if (!affine_args_ok(N, K, G, bits) || !dtype_ok(w_dtype) || !dtype_ok(sb_dtype)) return OR_EARG;
    int64_t ng = K / G, wpr = K * bits / 32;
    int per = 32 / bits;
    float qmax = (float)((1 << bits) - 1);
    memset(packed, 0, sizeof(uint32_t) * (size_t)(N * wpr));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < ng; ++g) {
            float lo = INFINITY, hi = -INFINITY;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float v = (float)load_f64(w, n * K + k, w_dtype);
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            float range = hi - lo;
            float s = range / qmax;
            float s_r = round_to(s, sb_dtype);
            float b_r = round_to(lo, sb_dtype);
            store_as(scales, n * ng + g, sb_dtype, s);
            store_as(biases, n * ng + g, sb_dtype, lo);
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float v = (float)load_f64(w, n * K + k, w_dtype);
                float t = 0.0f;
                if (s_r != 0.0f) {
                    float d = v - b_r;
                    t = rintf(d / s_r);
                    if (t < 0.0f) t = 0.0f;
                    if (t > qmax) t = qmax;
                }
                uint32_t code = (uint32_t)t;
                packed[n * wpr + k / per] |= code << (bits * (k % per));
            }
        }
    return OR_OK;
}

/* ---------------------------------------------------------------------- */
/* D1  dequantize to a storage type  [MLX8 `dequantize_to` (the whole      */
/*     weight written out as BF16); METAL "Dequantize"]                    */
/*                                                                        */
/* Each weight is the exact fp64 value of O2, rounded ONCE to the output   */
/* type, nearest even.  READING: the output type is BF16 (as on [MLX8]),   */
/* F16 or F32.                                                            */

/* Round a double to bfloat16 (8 significant bits, the exponent range of   */
/* an IEEE single), nearest even, from the definition of the format.       */
static uint16_t f64_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7fc0);
    if (a < ldexp(1.0, -126)) {       /* subnormal grid: multiples of 2^-133 */
        double m = nearbyint(ldexp(a, 133));
        return (uint16_t)(sign | (uint16_t)m);   /* m == 128 is the smallest normal */
    }
    int e;
    double f = frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
    double m = nearbyint(ldexp(f, 8));  /* 8 significant bits, in [128, 256] */
    if (m == 256.0) {
        m = 128.0;
        e += 1;
    }
    int biased = e - 1 + 127;
    if (biased >= 255)
        return (uint16_t)(sign | 0x7f80);
    return (uint16_t)(sign | (uint16_t)(biased << 7) | (uint16_t)((int)m - 128));
}

void oracle_f64_to_bf16(const double *src, int64_t n, uint16_t *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = f64_to_bf16(src[i]);
}

int oracle_dequant_affine_to(const uint32_t *packed, const void *scales, int s_dtype, const void *biases,
                             int b_dtype, int64_t N, int64_t K, int G, int bits, int out_dtype, void *out)
{
    if (!affine_args_ok(N, K, G, bits) || !dtype_ok(s_dtype) || !dtype_ok(b_dtype) || !dtype_ok(out_dtype))
        return OR_EARG;
    int64_t wpr = K * bits / 32;
    double *w = (double *)malloc(sizeof(double) * (size_t)(K + 1));
    if (!w) return OR_EMEM;
    for (int64_t n = 0; n < N; ++n) {
        dequant_affine_row(packed + n * wpr, scales, s_dtype, biases, b_dtype, n, K, G, bits, w);
        for (int64_t k = 0; k < K; ++k) {
            if (out_dtype == OR_BF16)
                ((uint16_t *)out)[n * K + k] = f64_to_bf16(w[k]);
            else if (out_dtype == OR_F16)
                ((uint16_t *)out)[n * K + k] = f64_to_f16(w[k]);
            else
                ((float *)out)[n * K + k] = (float)w[k];
        }
    }
    free(w);
    return OR_OK;
}

/* ---------------------------------------------------------------------- */
/* S1  SiLU-gated input  [MLX8 `gemv_silu_gate`, `gemv_silu_gate_resid`]   */
/*                                                                        */
/*   h[m,k] = silu(gate[m,k]) * up[m,k],   silu(t) = t / (1 + e^-t)        */
/*   y[m,n] = sum_{k ascending} h[m,k] * w[n,k]   (+ resid[m,n] if given)  */
/* all in fp64 from the stored gate, up and resid values; w as in O2.     */
static double silu(double t)
{
    return t / (1.0 + exp(-t));
}

void oracle_silu(const double *src, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = silu(src[i]);
}

int oracle_qmm_affine_silu_gate(const void *gate, const void *up, const void *resid, int act_dtype,
                                const uint32_t *packed, const void *scales, int s_dtype, const void *biases,
                                int b_dtype, int64_t M, int64_t N, int64_t K, int G, int bits, double *y)
{
    if (!affine_args_ok(N, K, G, bits) || M < 0 || !dtype_ok(s_dtype) || !dtype_ok(b_dtype) ||
        !dtype_ok(act_dtype))
        return OR_EARG;
    double *hd = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    if (!hd) return OR_EMEM;
    for (int64_t i = 0; i < M * K; ++i)
        hd[i] = silu(load_f64(gate, i, act_dtype)) * load_f64(up, i, act_dtype);
    int64_t wpr = K * bits / 32;
    int fail = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(K + 1));
        if (!w) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            if (!w) continue;
            dequant_affine_row(packed + n * wpr, scales, s_dtype, biases, b_dtype, n, K, G, bits, w);
            for (int64_t m = 0; m < M; ++m) {
                const double *hr = hd + m * K;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += hr[k] * w[k];
                if (resid)
                    acc += load_f64(resid, m * N + n, act_dtype);
                y[m * N + n] = acc;
            }
        }
        free(w);
    }
    free(hd);
    return fail ? OR_EMEM : OR_OK;
}

/* ---------------------------------------------------------------------- */
/* SQ  SmoothQuant ahead of W4A8  [GPTQ page, section 3 "SmoothQuant":     */
/*     "Trick" (y = (x / s) . (s W), per input channel) and Xiao et al.'s  */
/*     rule for s quoted there]                                           */
/*                                                                        */
/* SQ1 s[k] = act_absmax[k]^alpha / max_n |W[n,k]|^(1 - alpha), in fp64,   */
/*     stored as fp32 (nearest even).  act_absmax[k] = max over the        */
/*     calibration tokens of |x[:,k]|, gathered by the caller.            */
/*     READING: a channel whose activation or weight maximum is 0 gets     */
/*     s = 1 (the formula gives 0, inf or 0/0 there; 1 leaves it as is).   */
int oracle_smooth_factors(const float *act_absmax, const void *w, int w_dtype, int64_t N, int64_t K, double alpha,
                          float *s)
{
    if (N <= 0 || K <= 0 || !dtype_ok(w_dtype) || !(alpha >= 0.0 && alpha <= 1.0)) return OR_EARG;
    for (int64_t k = 0; k < K; ++k) {
        double wmax = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double a = fabs(load_f64(w, n * K + k, w_dtype));
            if (a > wmax) wmax = a;
        }
        double amax = (double)act_absmax[k];
        if (!(amax > 0.0) || !(wmax > 0.0))
            s[k] = 1.0f;
        else
            s[k] = (float)(pow(amax, alpha) / pow(wmax, 1.0 - alpha));
    }
    return OR_OK;
}

/* SQ2 W' = W diag(s) in our [N, K] layout (column k times s[k]), each     */
/*     product rounded to fp32; then the per-channel int4 quantization of   */
/*     W4A8 [W4A8 "What this adds"; symmetric rule as in QAT]:              */
/*       s_w[n] = f16( max_k |W'[n,k]| / 7 )   (fp32 division, then RNE)   */
/*       v[n,k] = clamp(rint(W'[n,k] / s_w[n]), -8, 7)  (fp32, s_w as stored)*/
/*     packed as Q4 (two's complement nibbles, lowest k in the low bits).  */
/*     smooth == NULL means s = 1 (plain W4A8 weight quantization).        */
/*     READING: a row with max 0 (or s_w rounding to 0) gets codes 0.       */
int oracle_w4a8_quantize_weights(const void *w, int w_dtype, const float *smooth, int64_t N, int64_t K,
                                 uint32_t *w_q4, uint16_t *s_w)
{
    if (N <= 0 || K <= 0 || K % 8 || !dtype_ok(w_dtype)) return OR_EARG;
    memset(w_q4, 0, sizeof(uint32_t) * (size_t)(N * (K / 8)));
    for (int64_t n = 0; n < N; ++n) {
        float wmax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)load_f64(w, n * K + k, w_dtype);
            if (smooth) v = v * smooth[k];
            float a = fabsf(v);
            if (a > wmax) wmax = a;
        }
        float sc = wmax / 7.0f;
        uint16_t h = f64_to_f16((double)sc);
        s_w[n] = h;
        float sr = (float)f16_to_f64(h);
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)load_f64(w, n * K + k, w_dtype);
            if (smooth) v = v * smooth[k];
            float t = 0.0f;
            if (sr != 0.0f) {
                t = rintf(v / sr);
                if (t > 7.0f) t = 7.0f;
                if (t < -8.0f) t = -8.0f;
            }
            uint32_t nibv = (uint32_t)((int)t & 0xF);
            w_q4[n * (K / 8) + k / 8] |= nibv << (4 * (k % 8));
        }
    }
    return OR_OK;
}

/* SQ3 the smoothed activations meet the W4A8 quantizer: per token,        */
/*       xs[m,k] = fp32(x[m,k]) / s[k]           (IEEE single division)     */
/*     then Q1..Q6 on xs in place of x.                                    */
int oracle_w4a8_smooth(const uint16_t *x, const float *smooth, const uint32_t *w_q4, const uint16_t *s_w, int64_t M,
                       int64_t N, int64_t K, int8_t *q, float *s_x, int64_t *acc, double *y)
{
    if (M < 0 || N < 0 || K <= 0 || K % 8) return OR_EARG;
    float *xs = (float *)malloc(sizeof(float) * (size_t)(M * K + 1));
    if (!xs) return OR_EMEM;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            xs[m * K + k] = (float)f16_to_f64(x[m * K + k]) / smooth[k];
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(xs[m * K + k]);
            if (a > amax) amax = a;
        }
        float sc = amax / 127.0f;
        s_x[m] = sc;
        for (int64_t k = 0; k < K; ++k) {
            float t = 0.0f;
            if (sc != 0.0f) {
                t = rintf(xs[m * K + k] / sc);
                if (t > 127.0f) t = 127.0f;
                if (t < -127.0f) t = -127.0f;
            }
            q[m * K + k] = (int8_t)t;
        }
    }
    free(xs);
    int rc = oracle_w4a8_acc(q, w_q4, M, N, K, acc);
    if (rc) return rc;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t a = acc[m * N + n];
            if (a > INT32_MAX || a < INT32_MIN) return OR_ERANGE;
            y[m * N + n] = (double)a * (double)s_x[m] * f16_to_f64(s_w[n]);
        }
    return OR_OK;
}
