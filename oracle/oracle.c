/*
 * CPU oracle for the decode-phase weight-only-quantized GEMM
 *     y[m, n] = sum_k x[m, k] * w[n, k]
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, includes or calls
 * this file; only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark load it.  It shares no code, header, table or constant with the
 * GPU path.
 *
 * Plain and slow on purpose: every value is decoded exactly from its bit
 * pattern by the format's closed form, every product and sum is taken in IEEE
 * binary64, one accumulator per output walks k = 0 .. K-1 in increasing order,
 * and nothing is blocked, fused or reordered.  Threads split the output
 * columns n only, so the result does not depend on the thread count.
 *
 * Where the method's result is defined:
 *   - FP8 weights: E4M3 codes with one FP32 scale per 128x128 block of W
 *     (arc PR "FP8 bank conflict + the dispatch threshold's provenance",
 *     section "The threshold": weight_block_size [128, 128]; atlas "Module
 *     m16_tc", section NUMERICS: the 128-K block scale).  The plain definition
 *     w[n,k] = e4m3(q[n,k]) * s[n/128][k/128] is used; the GPU folds the scale
 *     once per 128-K block, which is the same value up to rounding.
 *   - 3-bit LUT weights: w[n,k] = fp16_rne(qmap[c[n,k]] * g[n][k/128])
 *     (FLUTE "Add optimized_w3", "Core contributions" item 1 -- the learned
 *     8-entry map -- and "Results": the dequant rounds to fp16 before the
 *     accumulate).
 *   - E4M3 is read as OCP E4M3FN (bias 7, no infinities, S.1111.111 is NaN),
 *     the pages being silent on the flavour.
 *   - W8A8 (both operands FP8): the arc PR's "Worth a separate change" section
 *     notes that block-scaled FP8 GEMMs need the activations in FP8 too, i.e.
 *     an activation quantiser, which it does not specify; the atlas ladder
 *     ("ARM ORDER", rung 6) puts a W8A8 block-scaled tier above the decode
 *     band.  Reading used here: one FP32 scale per (row, 128-wide K group),
 *     s = amax / 448 in binary32 (s = 1 for an all-zero group), code =
 *     E4M3 nearest-even of clamp(x / s, -448, 448) with the division in
 *     binary32 -- the same rule as the weights' 128x128 block quantiser.  The
 *     product is then y[m,n] = sum_k (e4m3(xq[m,k]) sx[m][k/128]) *
 *     (e4m3(q[n,k]) s[n/128][k/128]).
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC -pthread.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define WQO_BLOCK 128

/* ---------------------------------------------------------------- decoding */

/* OCP E4M3FN: sign s, exponent e (4 bits, bias 7), mantissa m (3 bits).
 * e == 0 is subnormal: m * 2^-9.  e == 15 && m == 7 is NaN.  No infinity. */
double wqo_e4m3_value(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(8.0 + (double)m, e - 7 - 3);
    return s ? -v : v;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa. */
double wqo_f16_value(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp(1024.0 + (double)m, e - 15 - 10);
    return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa. */
double wqo_bf16_value(uint16_t b)
{
    int s = b >> 15, e = (b >> 7) & 255, m = b & 127;
    double v;
    if (e == 255)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -126 - 7);
    else
        v = ldexp(128.0 + (double)m, e - 127 - 7);
    return s ? -v : v;
}

/* ---------------------------------------------------------------- rounding */

/* Round a binary64 value to a binary format with `p` significand bits
 * (hidden bit included), exponent bias `bias`, `ebits` exponent bits, to
 * nearest with ties to even, with gradual underflow and overflow to infinity.
 * Returns the bit pattern. */
static uint32_t round_to_format(double v, int p, int ebits, int bias)
{
    uint32_t sign = signbit(v) ? 1u : 0u;
    uint32_t emax_field = (1u << ebits) - 1u;
    uint32_t mbits = (uint32_t)(p - 1);
    uint32_t out;
    if (isnan(v))
        return (sign << (ebits + mbits)) | (emax_field << mbits) | (1u << (mbits - 1));
    double a = fabs(v);
    int emin = 1 - bias;                   /* exponent of the smallest normal */
    int emax = (int)emax_field - 1 - bias; /* exponent of the largest finite  */
    if (isinf(a)) {
        out = emax_field << mbits;
    } else if (a < ldexp(1.0, emin)) {
        /* subnormal range: integer multiple of 2^(emin - (p-1)) */
        double q = nearbyint(ldexp(a, (p - 1) - emin)); /* exact scaling, RNE */
        out = (uint32_t)q;                  /* q == 2^(p-1) encodes the min normal */
    } else {
        int e;
        (void)frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
        e -= 1;                             /* a in [2^e, 2^(e+1))        */
        double q = nearbyint(ldexp(a, (p - 1) - e)); /* in [2^(p-1), 2^p] */
        if (q == ldexp(1.0, p)) {
            q = ldexp(1.0, p - 1);
            e += 1;
        }
        if (e > emax) {
            out = emax_field << mbits;      /* overflow -> infinity */
        } else {
            uint32_t field = (uint32_t)(e + bias);
            out = (field << mbits) | ((uint32_t)q - (1u << mbits));
        }
    }
    return (sign << (ebits + mbits)) | out;
}

uint16_t wqo_f16_rne(double v) { return (uint16_t)round_to_format(v, 11, 5, 15); }
uint16_t wqo_bf16_rne(double v) { return (uint16_t)round_to_format(v, 8, 8, 127); }

void wqo_f16_rne_array(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = wqo_f16_rne(v[i]);
}

void wqo_bf16_rne_array(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = wqo_bf16_rne(v[i]);
}

void wqo_e4m3_value_array(const uint8_t* b, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = wqo_e4m3_value(b[i]);
}

void wqo_f16_value_array(const uint16_t* h, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = wqo_f16_value(h[i]);
}

void wqo_bf16_value_array(const uint16_t* h, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = wqo_bf16_value(h[i]);
}

/* ----------------------------------------------------------- weight values */

/* FP8 row: w[k] = e4m3(q[n,k]) * s[n/128][k/128]   (exact in binary64). */
static void fp8_row(const uint8_t* q, int64_t ldq, const float* s, int64_t K,
                    int64_t n, double* w)
{
    int64_t kb = K / WQO_BLOCK;
    for (int64_t k = 0; k < K; ++k)
        w[k] = wqo_e4m3_value(q[n * ldq + k]) * (double)s[(n / WQO_BLOCK) * kb + k / WQO_BLOCK];
}

/* LUT3 row: w[k] = fp16_rne(qmap[c] * g[n][k/128]); the product of two binary16
 * values is exact in binary64, so this is one rounding of the exact product. */
static int lut3_row(const uint8_t* c, int64_t ldc, const uint16_t* qmap, const uint16_t* g,
                    int64_t K, int64_t n, double* w)
{
    int64_t kg = K / WQO_BLOCK;
    for (int64_t k = 0; k < K; ++k) {
        uint8_t code = c[n * ldc + k];
        if (code > 7) return -1;
        double p = wqo_f16_value(qmap[code]) * wqo_f16_value(g[n * kg + k / WQO_BLOCK]);
        w[k] = wqo_f16_value(wqo_f16_rne(p));
    }
    return 0;
}

int wqo_dequant_fp8(const uint8_t* q, int64_t ldq, const float* s, int64_t N, int64_t K,
                    double* w)
{
    if (N % WQO_BLOCK || K % WQO_BLOCK) return -2;
    for (int64_t n = 0; n < N; ++n) fp8_row(q, ldq, s, K, n, w + n * K);
    return 0;
}

int wqo_dequant_lut3(const uint8_t* c, int64_t ldc, const uint16_t* qmap, const uint16_t* g,
                     int64_t N, int64_t K, double* w)
{
    if (K % WQO_BLOCK) return -2;
    for (int64_t n = 0; n < N; ++n)
        if (lut3_row(c, ldc, qmap, g, K, n, w + n * K)) return -1;
    return 0;
}

/* --------------------------------------------------------------------- GEMM */

typedef struct {
    int fmt;                 /* 0 = fp8, 1 = lut3 */
    const double* x;         /* decoded activations [M][K] */
    const uint8_t* w;        /* codes [N][ldw] */
    int64_t ldw;
    const float* s8;         /* fp8 block scales */
    const uint16_t* qmap;    /* lut3 map */
    const uint16_t* g;       /* lut3 group scales */
    int64_t M, N, K;
    const int64_t* cols;     /* optional column subset */
    int64_t ncols;
    double* y;               /* [M][ncols] */
    int nthreads, tid;
    int err;
} job_t;

static void* gemm_worker(void* arg)
{
    job_t* j = (job_t*)arg;
    double* wrow = (double*)malloc(sizeof(double) * (size_t)j->K);
    if (!wrow) { j->err = -3; return NULL; }
    for (int64_t ci = j->tid; ci < j->ncols; ci += j->nthreads) {
        int64_t n = j->cols ? j->cols[ci] : ci;
        if (j->fmt == 0) {
            fp8_row(j->w, j->ldw, j->s8, j->K, n, wrow);
        } else if (lut3_row(j->w, j->ldw, j->qmap, j->g, j->K, n, wrow)) {
            j->err = -1;
            break;
        }
        for (int64_t m = 0; m < j->M; ++m) {
            const double* xr = j->x + m * j->K;
            double acc = 0.0;
            for (int64_t k = 0; k < j->K; ++k)
                acc += xr[k] * wrow[k];
            j->y[m * j->ncols + ci] = acc;
        }
    }
    free(wrow);
    return NULL;
}

static int run_gemm(job_t proto, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    job_t jobs[256];
    int started = 0, err = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].nthreads = nthreads;
        jobs[t].tid = t;
        jobs[t].err = 0;
        if (pthread_create(&th[t], NULL, gemm_worker, &jobs[t]) == 0) {
            started++;
        } else {
            /* fall back: run this share on the calling thread */
            gemm_worker(&jobs[t]);
            th[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t) {
        if (th[t]) pthread_join(th[t], NULL);
        if (jobs[t].err) err = jobs[t].err;
    }
    (void)started;
    return err;
}

/* ------------------------------------------------ activation quantiser (W8A8) */

/* Nearest OCP E4M3FN code to a finite binary32 value v with |v| <= 448, ties
 * to the even code.  The E4M3 grid: m * 2^-9 below 2^-6 (m = 0..7, and m = 8
 * is the smallest normal, code 0x08), (1 + m/8) * 2^(e-7) above.  Everything
 * is exact in binary64; nearbyint() rounds half to even. */
static uint8_t e4m3_rne_code(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a < ldexp(1.0, -6)) {
        double m = nearbyint(ldexp(a, 9));         /* 0 .. 8 */
        return (uint8_t)(sign | (uint8_t)m);
    }
    int e2;
    (void)frexp(a, &e2);                           /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                                /* a in [2^E, 2^(E+1)) */
    double q = nearbyint(ldexp(a, 3 - E));         /* 8 .. 16 */
    if (q == 16.0) {
        q = 8.0;
        E += 1;
    }
    return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)(q - 8.0));
}

uint8_t wqo_e4m3_rne(float v) { return e4m3_rne_code(v); }

/* codes [M][K] and scales [M][K/128] of BF16 x [M][ldx]:
 * s = amax/448 (binary32; 1 for an all-zero group), code = e4m3_rne(clamp(x/s)).
 * A group holding an infinity or a NaN has no finite amax; reading taken (the
 * pages define no quantiser, let alone for non-finite input): its scale is NaN
 * and every code of the group is the E4M3 NaN 0x7F, so every product that
 * uses the group is NaN, as an infinite or NaN activation makes the
 * weight-only paths' sums non-finite. */
int wqo_quantize_x_fp8(const uint16_t* x_bf16, int64_t ldx, int64_t M, int64_t K,
                       uint8_t* codes, float* scales)
{
    if (K % WQO_BLOCK || ldx < K) return -2;
    int64_t kb_n = K / WQO_BLOCK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t kb = 0; kb < kb_n; ++kb) {
            const uint16_t* xr = x_bf16 + m * ldx + kb * WQO_BLOCK;
            float amax = 0.0f;
            int nonfinite = 0;
            for (int i = 0; i < WQO_BLOCK; ++i) {
                float a = fabsf((float)wqo_bf16_value(xr[i]));
                if (!isfinite(a)) nonfinite = 1;
                else if (a > amax) amax = a;
            }
            if (nonfinite) {
                scales[m * kb_n + kb] = NAN;
                for (int i = 0; i < WQO_BLOCK; ++i) codes[m * K + kb * WQO_BLOCK + i] = 0x7F;
                continue;
            }
            float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            scales[m * kb_n + kb] = s;
            for (int i = 0; i < WQO_BLOCK; ++i) {
                float q = (float)wqo_bf16_value(xr[i]) / s;
                if (q > 448.0f) q = 448.0f;
                if (q < -448.0f) q = -448.0f;
                codes[m * K + kb * WQO_BLOCK + i] = e4m3_rne_code(q);
            }
        }
    }
    return 0;
}

/* x_bits: [M][ldx] BF16 (x_is_f16 == 0) or FP16 (x_is_f16 == 1). */
static double* decode_x(const uint16_t* x_bits, int64_t ldx, int64_t M, int64_t K, int is_f16)
{
    double* x = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    if (!x) return NULL;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            x[m * K + k] = is_f16 ? wqo_f16_value(x_bits[m * ldx + k])
                                  : wqo_bf16_value(x_bits[m * ldx + k]);
    return x;
}

/* y64[m][ci] = sum_k x[m,k] * e4m3(q[n,k]) * s[n/128][k/128], n = cols[ci]
 * (cols == NULL: all N columns, ncols ignored). */
int wqo_gemm_fp8(const uint16_t* x_bf16, int64_t ldx, const uint8_t* q, int64_t ldq,
                 const float* s, int64_t M, int64_t N, int64_t K,
                 const int64_t* cols, int64_t ncols, double* y, int nthreads)
{
    if (N % WQO_BLOCK || K % WQO_BLOCK || ldx < K || ldq < K) return -2;
    double* x = decode_x(x_bf16, ldx, M, K, 0);
    if (!x) return -3;
    job_t j = {0, x, q, ldq, s, NULL, NULL, M, N, K, cols, cols ? ncols : N, y, 1, 0, 0};
    int err = run_gemm(j, nthreads);
    free(x);
    return err;
}

/* y64[m][ci] = sum_k x[m,k] * fp16_rne(qmap[c[n,k]] * g[n][k/128]). */
int wqo_gemm_lut3(const uint16_t* x_f16, int64_t ldx, const uint8_t* c, int64_t ldc,
                  const uint16_t* qmap, const uint16_t* g, int64_t M, int64_t N, int64_t K,
                  const int64_t* cols, int64_t ncols, double* y, int nthreads)
{
    if (K % WQO_BLOCK || ldx < K || ldc < K) return -2;
    double* x = decode_x(x_f16, ldx, M, K, 1);
    if (!x) return -3;
    job_t j = {1, x, c, ldc, NULL, qmap, g, M, N, K, cols, cols ? ncols : N, y, 1, 0, 0};
    int err = run_gemm(j, nthreads);
    free(x);
    return err;
}

/* y64[m][ci] = sum_k e4m3(xq[m,k]) * sx[m][k/128] * e4m3(q[n,k]) * s[n/128][k/128]:
 * both operands are decoded exactly into binary64 and summed as in
 * wqo_gemm_fp8 (one accumulator, k increasing). */
int wqo_gemm_w8a8(const uint8_t* xq, int64_t ldxq, const float* sx, const uint8_t* q, int64_t ldq,
                  const float* s, int64_t M, int64_t N, int64_t K,
                  const int64_t* cols, int64_t ncols, double* y, int nthreads)
{
    if (N % WQO_BLOCK || K % WQO_BLOCK || ldxq < K || ldq < K) return -2;
    int64_t kb_n = K / WQO_BLOCK;
    double* x = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    if (!x) return -3;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            x[m * K + k] = wqo_e4m3_value(xq[m * ldxq + k]) * (double)sx[m * kb_n + k / WQO_BLOCK];
    job_t j = {0, x, q, ldq, s, NULL, NULL, M, N, K, cols, cols ? ncols : N, y, 1, 0, 0};
    int err = run_gemm(j, nthreads);
    free(x);
    return err;
}
