/*
 * NVFP4 oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU definition of what the NVFP4 prefill path computes.  Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or helper with the
 * HIP library in nvfp4_prefill_gemm_amd/csrc, and the product path never
 * calls it.
 *
 * Source of the method: "Quantized Prefilling, Precise Decoding for Agentic
 * LLMs" (Mix-Quant), Section 3.3 "NVFP4 Microscaling Quantization for
 * Prefilling", Eq. (2) (element quantization / dequantization) and Eq. (3)
 * (amax-based E4M3 block scale), with g = 16 elements per block.
 *
 * Readings taken where the page is silent (all listed in the design doc):
 *   - tensor scale alpha = amax(|x|) / (6 * 448) computed in FP32;
 *   - Eq. (3) evaluated in FP32 as  s = amax_b / (alpha * 6),  then rounded
 *     to the E4M3 (OCP "FN": bias 7, max 448) grid, nearest, ties to even,
 *     saturating at 448;
 *   - Eq. (2) evaluated in FP32 as  v = x / (alpha * sigma),  then rounded to
 *     the E2M1 grid, nearest, ties to even, clipped to +-6, sign kept (so -0
 *     and small negatives give the negative-zero code 0x8);
 *   - a block whose alpha*sigma is zero gets signed-zero codes;
 *   - codes are packed two per byte, element 2j in the low nibble;
 *     scales are one byte per block, row-major [rows, cols/16].
 *
 * Every rounding here is done the slow, obvious way: search the finite value
 * table (built from the format's bit fields) for the nearest value and break
 * exact ties toward the code whose mantissa LSB is zero.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC -pthread
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_ABI_VERSION 1

int oracle_abi_version(void) { return ORACLE_ABI_VERSION; }

/* ------------------------------------------------------------------------ */
/* Formats, decoded from their bit fields.                                   */
/* ------------------------------------------------------------------------ */

/* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no Inf/NaN.
 * exponent field 0 is subnormal: value = m * 0.5.                          */
double oracle_e2m1_value(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return s ? -mag : mag;
}

/* E4M3 (OCP "FN"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no Inf.    */
double oracle_e4m3_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -mag : mag;
}

/* Nearest entry of an ascending table of non-negative values, ties broken
 * toward the even index (= mantissa LSB 0 in both formats, whose
 * non-negative codes are ordered by value).  a must be finite, >= 0.     */
static int nearest_even(double a, const double *table, int n) {
    int best = 0;
    double bd = fabs(a - table[0]);
    for (int c = 1; c < n; ++c) {
        double d = fabs(a - table[c]);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return best;
}

static double E2M1_POS[8];   /* codes 0..7   */
static double E4M3_POS[127]; /* codes 0..126 */
static pthread_once_t tables_once = PTHREAD_ONCE_INIT;
static void build_tables(void) {
    for (int c = 0; c < 8; ++c) E2M1_POS[c] = oracle_e2m1_value(c);
    for (int c = 0; c < 127; ++c) E4M3_POS[c] = oracle_e4m3_value(c);
}
static void tables(void) { pthread_once(&tables_once, build_tables); }

/* Pi_FP4 of Eq. (2): nearest E2M1 value with clipping; returns the 4-bit code
 * with the sign of v (v = -0.0 gives 0x8).                                  */
int oracle_e2m1_encode(float v) {
    tables();
    int sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (!(a <= 6.0)) return sign | 7; /* clip: beyond the largest magnitude */
    return sign | nearest_even(a, E2M1_POS, 8);
}

/* Pi_E4M3 of Eq. (3) for a non-negative scale: nearest E4M3 value, ties to
 * even, saturating at 448 (code 0x7E).                                      */
int oracle_e4m3_encode(float s) {
    tables();
    double a = (double)s;
    if (!(a <= 448.0)) return 0x7E;
    if (a <= 0.0) return 0;
    return nearest_even(a, E4M3_POS, 127);
}

void oracle_e2m1_encode_n(const float *v, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e2m1_encode(v[i]);
}
void oracle_e4m3_encode_n(const float *s, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e4m3_encode(s[i]);
}

/* ------------------------------------------------------------------------ */
/* Threading over rows (arithmetic is independent of the split).             */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void *ctx, int64_t r0, int64_t r1);
typedef struct { row_fn fn; void *ctx; int64_t r0, r1; } row_job;
static void *row_thread(void *p) {
    row_job *j = (row_job *)p;
    j->fn(j->ctx, j->r0, j->r1);
    return NULL;
}
int oracle_default_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}
static void parallel_rows(row_fn fn, void *ctx, int64_t rows, int nthreads) {
    if (nthreads <= 0) nthreads = oracle_default_threads();
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
    if (nthreads <= 1) { fn(ctx, 0, rows); return; }
    pthread_t th[256];
    row_job jobs[256];
    int64_t per = (rows + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t r0 = t * per, r1 = r0 + per > rows ? rows : r0 + per;
        if (r0 >= r1) break;
        jobs[t] = (row_job){fn, ctx, r0, r1};
        if (pthread_create(&th[t], NULL, row_thread, &jobs[t]) != 0) { fn(ctx, r0, r1); continue; }
        started = t + 1;
    }
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Quantization (Eq. 2 and Eq. 3).                                           */
/* ------------------------------------------------------------------------ */

static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* max |x| over a BF16 matrix with row stride ld (elements). */
float oracle_amax_bf16(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld) {
    float m = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float a = fabsf(bf16_to_float(x[r * ld + c]));
            if (a > m) m = a;
        }
    return m;
}

/* Tensor-level scale: alpha = amax / (q_max * E4M3 max) = amax / (6 * 448). */
float oracle_tensor_alpha(float amax) { return amax / (6.0f * 448.0f); }

/* One 16-element block v (FP32 values) with tensor scale alpha: Eq. (3) for
 * its E4M3 scale code, Eq. (2) for its 16 E2M1 codes, packed two per byte
 * (element 2j in the low nibble) into codes8[0..7].                         */
static void quant_block(const float v[16], float alpha, uint8_t *scale, uint8_t codes8[8]) {
    float amax_b = 0.0f;
    for (int i = 0; i < 16; ++i) {
        float a = fabsf(v[i]);
        if (a > amax_b) amax_b = a;
    }
    /* Eq. (3): sigma = Pi_E4M3( amax_b / (alpha * q_max) ) */
    float t = alpha * 6.0f;
    float s = (t > 0.0f) ? amax_b / t : 0.0f;
    int sc = oracle_e4m3_encode(s);
    float sigma = (float)oracle_e4m3_value(sc);
    *scale = (uint8_t)sc;
    /* Eq. (2): q_i = Pi_FP4( x_i / (alpha * sigma) ) */
    float d = alpha * sigma;
    uint8_t codes[16];
    for (int i = 0; i < 16; ++i) {
        float y = (d > 0.0f) ? v[i] / d : copysignf(0.0f, v[i]);
        codes[i] = (uint8_t)oracle_e2m1_encode(y);
    }
    for (int j = 0; j < 8; ++j) codes8[j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
}

typedef struct {
    const uint16_t *x;   /* BF16 input, or NULL */
    const float *xf;     /* FP32 input, or NULL */
    int64_t cols, ld;
    float alpha;
    uint8_t *codes, *scales;
} quant_ctx;

static void quant_rows(void *p, int64_t r0, int64_t r1) {
    quant_ctx *q = (quant_ctx *)p;
    const int64_t nb = q->cols / 16;
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            float v[16];
            for (int i = 0; i < 16; ++i)
                v[i] = q->x ? bf16_to_float(q->x[r * q->ld + b * 16 + i]) : q->xf[r * q->ld + b * 16 + i];
            quant_block(v, q->alpha, &q->scales[r * nb + b], &q->codes[r * (q->cols / 2) + b * 8]);
        }
    }
}

/* x: BF16 bits [rows, ld]; codes: [rows, cols/2]; scales: [rows, cols/16].
 * alpha_mode 0: alpha = amax/2688 is computed and stored to *alpha;
 * alpha_mode 1: *alpha is used as given (static tensor scale).
 * Returns 0, or -1 when cols is not a multiple of 16 or ld < cols.         */
int oracle_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, int alpha_mode,
                    float *alpha, uint8_t *codes, uint8_t *scales, int nthreads) {
    if (cols % 16 != 0 || ld < cols || rows < 0) return -1;
    tables();
    if (alpha_mode == 0) *alpha = oracle_tensor_alpha(oracle_amax_bf16(x, rows, cols, ld));
    quant_ctx q = {x, NULL, cols, ld, *alpha, codes, scales};
    parallel_rows(quant_rows, &q, rows, nthreads);
    return 0;
}

/* The same Eq. (3) / Eq. (2) steps on an FP32 tensor (a GEMM output that is
 * quantized for the next linear layer), each value taken as it is (no
 * rounding to BF16 first).  alpha_mode as in oracle_quantize; the dynamic
 * amax is max |x| over the FP32 values.                                    */
int oracle_quantize_f32(const float *x, int64_t rows, int64_t cols, int64_t ld, int alpha_mode, float *alpha,
                        uint8_t *codes, uint8_t *scales, int nthreads) {
    if (cols % 16 != 0 || ld < cols || rows < 0) return -1;
    tables();
    if (alpha_mode == 0) {
        float m = 0.0f;
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t c = 0; c < cols; ++c) {
                float a = fabsf(x[r * ld + c]);
                if (a > m) m = a;
            }
        *alpha = oracle_tensor_alpha(m);
    }
    quant_ctx q = {NULL, x, cols, ld, *alpha, codes, scales};
    parallel_rows(quant_rows, &q, rows, nthreads);
    return 0;
}

/* x_hat = alpha * sigma * q  (Eq. 2), in float64: sigma*q is exact and the
 * product with alpha is rounded once.                                       */
void oracle_dequantize(const uint8_t *codes, const uint8_t *scales, float alpha, int64_t rows,
                       int64_t cols, double *out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = codes[r * (cols / 2) + c / 2];
            int code = (c & 1) ? (byte >> 4) : (byte & 15);
            double sigma = oracle_e4m3_value(scales[r * (cols / 16) + c / 16]);
            out[r * cols + c] = (double)alpha * (sigma * oracle_e2m1_value(code));
        }
}

/* ------------------------------------------------------------------------ */
/* GEMM  Y[m,n] = sum_k xhatA[m,k] * xhatW[n,k]   (y = x W^T).              */
/* ------------------------------------------------------------------------ */

/* Exact form.  With x_hat = alpha*sigma*q, every 2q is an integer in
 * [-12, 12] and every 512*sigma is an integer in [0, 229376], so
 *   Y = alphaA*alphaW * 2^-20 * sum_b (512 sA)(512 sW) sum_{k in b} (2qA)(2qW)
 * is an exact int64 sum (|term| < 2^43, fine for K below ~10^6), scaled once
 * in float64 at the end.                                                    */
typedef struct {
    int8_t *q2;   /* [rows, K]  2*q     */
    int32_t *s512; /* [rows, K/16] 512*sigma */
} decoded;

static int decode_operand(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                          decoded *d) {
    d->q2 = (int8_t *)malloc((size_t)(rows * K > 0 ? rows * K : 1));
    d->s512 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(rows * (K / 16) > 0 ? rows * (K / 16) : 1));
    if (!d->q2 || !d->s512) { free(d->q2); free(d->s512); return -1; }
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = codes[r * (K / 2) + k / 2];
            int code = (k & 1) ? (byte >> 4) : (byte & 15);
            d->q2[r * K + k] = (int8_t)lrint(2.0 * oracle_e2m1_value(code));
        }
        for (int64_t b = 0; b < K / 16; ++b) {
            double s = oracle_e4m3_value(scales[r * (K / 16) + b]);
            d->s512[r * (K / 16) + b] = (int32_t)lrint(512.0 * s);
        }
    }
    return 0;
}

static double exact_dot(const decoded *A, int64_t m, const decoded *W, int64_t n, int64_t K) {
    const int8_t *qa = A->q2 + m * K, *qw = W->q2 + n * K;
    const int32_t *sa = A->s512 + m * (K / 16), *sw = W->s512 + n * (K / 16);
    int64_t acc = 0;
    for (int64_t b = 0; b < K / 16; ++b) {
        int64_t p = 0;
        for (int i = 0; i < 16; ++i) p += (int64_t)qa[b * 16 + i] * qw[b * 16 + i];
        acc += p * (int64_t)sa[b] * (int64_t)sw[b];
    }
    return (double)acc;
}

typedef struct {
    const decoded *A, *W;
    int64_t N, K;
    double scale;
    double *out;
    const int64_t *mi, *ni;
} gemm_ctx;

static void exact_rows(void *p, int64_t r0, int64_t r1) {
    gemm_ctx *g = (gemm_ctx *)p;
    for (int64_t m = r0; m < r1; ++m)
        for (int64_t n = 0; n < g->N; ++n)
            g->out[m * g->N + n] = exact_dot(g->A, m, g->W, n, g->K) * g->scale;
}
static void exact_pairs(void *p, int64_t i0, int64_t i1) {
    gemm_ctx *g = (gemm_ctx *)p;
    for (int64_t i = i0; i < i1; ++i) g->out[i] = exact_dot(g->A, g->mi[i], g->W, g->ni[i], g->K) * g->scale;
}

int oracle_gemm_exact(const uint8_t *a_codes, const uint8_t *a_scales, float a_alpha,
                      const uint8_t *w_codes, const uint8_t *w_scales, float w_alpha, int64_t M,
                      int64_t N, int64_t K, double *out, int nthreads) {
    if (K % 16 != 0) return -1;
    decoded A, W;
    if (decode_operand(a_codes, a_scales, M, K, &A)) return -2;
    if (decode_operand(w_codes, w_scales, N, K, &W)) { free(A.q2); free(A.s512); return -2; }
    gemm_ctx g = {&A, &W, N, K, ldexp(1.0, -20) * (double)a_alpha * (double)w_alpha, out, NULL, NULL};
    parallel_rows(exact_rows, &g, M, nthreads);
    free(A.q2); free(A.s512); free(W.q2); free(W.s512);
    return 0;
}

/* Same definition at selected (m, n) pairs, for full-size spot checks.  The
 * operands are decoded whole (rows [0, M) and [0, N)).                      */
int oracle_gemm_exact_pairs(const uint8_t *a_codes, const uint8_t *a_scales, float a_alpha,
                            const uint8_t *w_codes, const uint8_t *w_scales, float w_alpha,
                            int64_t M, int64_t N, int64_t K, const int64_t *mi, const int64_t *ni,
                            int64_t npairs, double *out, int nthreads) {
    if (K % 16 != 0) return -1;
    decoded A, W;
    if (decode_operand(a_codes, a_scales, M, K, &A)) return -2;
    if (decode_operand(w_codes, w_scales, N, K, &W)) { free(A.q2); free(A.s512); return -2; }
    gemm_ctx g = {&A, &W, N, K, ldexp(1.0, -20) * (double)a_alpha * (double)w_alpha, out, mi, ni};
    parallel_rows(exact_pairs, &g, npairs, nthreads);
    free(A.q2); free(A.s512); free(W.q2); free(W.s512);
    return 0;
}

/* Literal FP32 form: x_hat rounded to float (alpha * (sigma*q)), float
 * products, float sums in increasing k.                                     */
typedef struct {
    const float *xa, *xw;
    int64_t N, K;
    float *out;
} fp32_ctx;
static void fp32_rows(void *p, int64_t r0, int64_t r1) {
    fp32_ctx *g = (fp32_ctx *)p;
    for (int64_t m = r0; m < r1; ++m)
        for (int64_t n = 0; n < g->N; ++n) {
            float acc = 0.0f;
            for (int64_t k = 0; k < g->K; ++k) {
                float prod = g->xa[m * g->K + k] * g->xw[n * g->K + k];
                acc = acc + prod;
            }
            g->out[m * g->N + n] = acc;
        }
}
static float *dequant_f32(const uint8_t *codes, const uint8_t *scales, float alpha, int64_t rows,
                          int64_t K) {
    float *x = (float *)malloc(sizeof(float) * (size_t)(rows * K > 0 ? rows * K : 1));
    if (!x) return NULL;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = codes[r * (K / 2) + k / 2];
            int code = (k & 1) ? (byte >> 4) : (byte & 15);
            float sq = (float)(oracle_e4m3_value(scales[r * (K / 16) + k / 16]) * oracle_e2m1_value(code));
            x[r * K + k] = alpha * sq;
        }
    return x;
}
int oracle_gemm_fp32(const uint8_t *a_codes, const uint8_t *a_scales, float a_alpha,
                     const uint8_t *w_codes, const uint8_t *w_scales, float w_alpha, int64_t M,
                     int64_t N, int64_t K, float *out, int nthreads) {
    if (K % 16 != 0) return -1;
    float *xa = dequant_f32(a_codes, a_scales, a_alpha, M, K);
    float *xw = dequant_f32(w_codes, w_scales, w_alpha, N, K);
    if (!xa || !xw) { free(xa); free(xw); return -2; }
    fp32_ctx g = {xa, xw, N, K, out};
    parallel_rows(fp32_rows, &g, M, nthreads);
    free(xa); free(xw);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* BF16 GEMM of the decode path: float64 products and sums.                  */
/* ------------------------------------------------------------------------ */
typedef struct {
    const uint16_t *a, *w;
    int64_t N, K;
    double *out;
    const int64_t *mi, *ni;
} bf16_ctx;
static double bf16_dot(const uint16_t *a, const uint16_t *w, int64_t K) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += (double)bf16_to_float(a[k]) * (double)bf16_to_float(w[k]);
    return acc;
}
static void bf16_rows(void *p, int64_t r0, int64_t r1) {
    bf16_ctx *g = (bf16_ctx *)p;
    for (int64_t m = r0; m < r1; ++m)
        for (int64_t n = 0; n < g->N; ++n)
            g->out[m * g->N + n] = bf16_dot(g->a + m * g->K, g->w + n * g->K, g->K);
}
static void bf16_pairs(void *p, int64_t i0, int64_t i1) {
    bf16_ctx *g = (bf16_ctx *)p;
    for (int64_t i = i0; i < i1; ++i) g->out[i] = bf16_dot(g->a + g->mi[i] * g->K, g->w + g->ni[i] * g->K, g->K);
}
void oracle_bf16_gemm(const uint16_t *a, const uint16_t *w, int64_t M, int64_t N, int64_t K,
                      double *out, int nthreads) {
    bf16_ctx g = {a, w, N, K, out, NULL, NULL};
    parallel_rows(bf16_rows, &g, M, nthreads);
}
void oracle_bf16_gemm_pairs(const uint16_t *a, const uint16_t *w, int64_t K, const int64_t *mi,
                            const int64_t *ni, int64_t npairs, double *out, int nthreads) {
    bf16_ctx g = {a, w, 0, K, out, mi, ni};
    parallel_rows(bf16_pairs, &g, npairs, nthreads);
}

/* ------------------------------------------------------------------------ */
/* MXFP4: E2M1 elements with one E8M0 (power-of-two) scale per 32 elements. */
/* Mix-Quant Section 3.3 names MXFP4 as the coarser microscaling format with  */
/* larger groups and power-of-two scales.  The pages give no rounding rule;   */
/* the reading taken is the OCP Microscaling (MX) v1.0 conversion: shared     */
/* exponent = floor(log2(max |x|)) - 2 (2 = largest E2M1 exponent), clamped   */
/* to E8M0's [-127, 127]; an all-zero block takes the smallest scale 2^-127;  */
/* elements are x / 2^shared rounded to E2M1 nearest-even with saturation.   */
/* ------------------------------------------------------------------------ */

/* E8M0 code -> value 2^(code - 127); code 255 is NaN. */
double oracle_e8m0_value(int code) {
    if ((code & 255) == 255) return NAN;
    return ldexp(1.0, (code & 255) - 127);
}

typedef struct {
    const uint16_t *x;
    int64_t cols, ld;
    uint8_t *codes, *scales;
} mx_ctx;

static void mx_rows(void *p, int64_t r0, int64_t r1) {
    mx_ctx *q = (mx_ctx *)p;
    const int64_t nb = q->cols / 32;
    for (int64_t r = r0; r < r1; ++r) {
        const uint16_t *xr = q->x + r * q->ld;
        for (int64_t b = 0; b < nb; ++b) {
            double v[32], amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                v[i] = (double)bf16_to_float(xr[b * 32 + i]);
                if (fabs(v[i]) > amax) amax = fabs(v[i]);
            }
            int shared = -127;
            if (amax > 0.0) {
                int e;
                frexp(amax, &e);   /* amax = m * 2^e, m in [0.5, 1): floor(log2 amax) = e - 1 */
                shared = (e - 1) - 2;
                if (shared < -127) shared = -127;
                if (shared > 127) shared = 127;
            }
            q->scales[r * nb + b] = (uint8_t)(shared + 127);
            uint8_t codes[32];
            for (int i = 0; i < 32; ++i) {
                double y = ldexp(v[i], -shared); /* exact */
                codes[i] = (uint8_t)oracle_e2m1_encode((float)y);
            }
            for (int j = 0; j < 16; ++j)
                q->codes[r * (q->cols / 2) + b * 16 + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
        }
    }
}

/* x: BF16 bits [rows, ld]; codes [rows, cols/2]; scales [rows, cols/32] E8M0.
 * Returns 0, or -1 when cols % 32 != 0 or ld < cols.                         */
int oracle_mx_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *codes,
                       uint8_t *scales, int nthreads) {
    if (cols % 32 != 0 || ld < cols || rows < 0) return -1;
    tables();
    mx_ctx q = {x, cols, ld, codes, scales};
    parallel_rows(mx_rows, &q, rows, nthreads);
    return 0;
}

/* x_hat = 2^shared * q, float64 (exact). */
void oracle_mx_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                          double *out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = codes[r * (cols / 2) + c / 2];
            int code = (c & 1) ? (byte >> 4) : (byte & 15);
            out[r * cols + c] = oracle_e8m0_value(scales[r * (cols / 32) + c / 32]) * oracle_e2m1_value(code);
        }
}

/* Y[m,n] = sum_b 2^(sA[m,b] + sW[n,b]) * sum_{k in b} qA qW.  Each block sum is
 * an exact integer (in quarter units) times an exact power of two; the block
 * terms are added in float64 in increasing b.                                */
typedef struct {
    const uint8_t *ac, *as, *wc, *ws;
    int64_t N, K;
    double *out;
    const int64_t *mi, *ni;
} mxg_ctx;
static double mx_dot(const mxg_ctx *g, int64_t m, int64_t n) {
    const int64_t nb = g->K / 32;
    double acc = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        int64_t p = 0;
        for (int i = 0; i < 32; ++i) {
            int64_t k = b * 32 + i;
            uint8_t ba = g->ac[m * (g->K / 2) + k / 2], bw = g->wc[n * (g->K / 2) + k / 2];
            int ca = (k & 1) ? (ba >> 4) : (ba & 15), cw = (k & 1) ? (bw >> 4) : (bw & 15);
            p += (int64_t)lrint(2.0 * oracle_e2m1_value(ca)) * (int64_t)lrint(2.0 * oracle_e2m1_value(cw));
        }
        int e = ((int)g->as[m * nb + b] - 127) + ((int)g->ws[n * nb + b] - 127) - 2;
        acc += ldexp((double)p, e);
    }
    return acc;
}
static void mxg_rows(void *p, int64_t r0, int64_t r1) {
    mxg_ctx *g = (mxg_ctx *)p;
    for (int64_t m = r0; m < r1; ++m)
        for (int64_t n = 0; n < g->N; ++n) g->out[m * g->N + n] = mx_dot(g, m, n);
}
static void mxg_pairs(void *p, int64_t i0, int64_t i1) {
    mxg_ctx *g = (mxg_ctx *)p;
    for (int64_t i = i0; i < i1; ++i) g->out[i] = mx_dot(g, g->mi[i], g->ni[i]);
}
int oracle_mx_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_codes,
                   const uint8_t *w_scales, int64_t M, int64_t N, int64_t K, double *out, int nthreads) {
    if (K % 32 != 0) return -1;
    tables();
    mxg_ctx g = {a_codes, a_scales, w_codes, w_scales, N, K, out, NULL, NULL};
    parallel_rows(mxg_rows, &g, M, nthreads);
    return 0;
}
int oracle_mx_gemm_pairs(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_codes,
                         const uint8_t *w_scales, int64_t K, const int64_t *mi, const int64_t *ni,
                         int64_t npairs, double *out, int nthreads) {
    if (K % 32 != 0) return -1;
    tables();
    mxg_ctx g = {a_codes, a_scales, w_codes, w_scales, 0, K, out, mi, ni};
    parallel_rows(mxg_pairs, &g, npairs, nthreads);
    return 0;
}
