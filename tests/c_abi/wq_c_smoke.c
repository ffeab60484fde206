/*
 * C-only use of the libwq boundary (test infrastructure): a plain C program,
 * with no Python and no torch, allocates device memory with the HIP runtime,
 * packs FP8 block-scaled and 3-bit LUT matrices through the C ABI of
 * include/wq.h, runs the GEMMs on both FP8 paths and both LUT layouts, and
 * checks every output against the CPU oracle (liboracle, linked here as the
 * reference the outputs are compared with) with the comparison rule of the
 * tests: within 2 BF16 ULP of
 * the FP64 result rounded to BF16, or within 1e-3*sqrt(K)*max|x|*max|w| of it.
 * It also checks a few validation errors that need no device work.
 *
 * With --selftest it checks only its own acceptance rule, on the CPU.
 *
 * Exit status 0: every check passed; 1: a check failed; 2: no usable device.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "wq.h"

/* the CPU oracle (oracle/oracle.c) */
int wqo_gemm_fp8(const uint16_t* x_bf16, int64_t ldx, const uint8_t* q, int64_t ldq, const float* s, int64_t M,
                 int64_t N, int64_t K, const int64_t* cols, int64_t ncols, double* y, int nthreads);
int wqo_gemm_lut3(const uint16_t* x_f16, int64_t ldx, const uint8_t* c, int64_t ldc, const uint16_t* qmap,
                  const uint16_t* g, int64_t M, int64_t N, int64_t K, const int64_t* cols, int64_t ncols, double* y,
                  int nthreads);
int wqo_dequant_fp8(const uint8_t* q, int64_t ldq, const float* s, int64_t N, int64_t K, double* w);
int wqo_dequant_lut3(const uint8_t* c, int64_t ldc, const uint16_t* qmap, const uint16_t* g, int64_t N, int64_t K,
                     double* w);
uint16_t wqo_bf16_rne(double v);
double wqo_bf16_value(uint16_t b);
double wqo_f16_value(uint16_t h);

static int failures = 0;

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fprintf(stderr, "\n");                        \
            ++failures;                                   \
        }                                                 \
    } while (0)

#define HIP_OK(call)                                                        \
    do {                                                                    \
        hipError_t e_ = (call);                                             \
        if (e_ != hipSuccess) {                                             \
            fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            exit(1);                                                        \
        }                                                                   \
    } while (0)

/* splitmix64: deterministic inputs */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double uniform(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

/* the BF16 bits of a float by truncation (any bit pattern is a valid input) */
static uint16_t bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* an FP16 bit pattern for a value in [-1, 1] (normal numbers, exponent 14 down to 10) */
static uint16_t f16_bits_unit(void)
{
    const uint16_t sign = (uint16_t)((next_u64() & 1) << 15);
    const uint16_t exp = (uint16_t)(10 + next_u64() % 5);
    const uint16_t man = (uint16_t)(next_u64() & 0x3FF);
    return (uint16_t)(sign | (exp << 10) | man);
}

static int64_t bf16_ord(uint16_t b) { return (b & 0x8000) ? -(int64_t)(b & 0x7FFF) : (int64_t)b; }

/* the absolute floor of the acceptance rule: 1e-3 * sqrt(K) * max|x| * max|w| */
static double abs_floor(int64_t K, double xmax, double wmax) { return 1e-3 * sqrt((double)K) * xmax * wmax; }

/* one output: finite, and within 2 BF16 ULP of bf16(y64) or within the floor of y64 */
static int element_ok(uint16_t gb, int is_f16, double r, double floor_abs)
{
    const double g = is_f16 ? wqo_f16_value(gb) : wqo_bf16_value(gb);
    const uint16_t g16 = is_f16 ? wqo_bf16_rne(g) : gb;
    const int ulp_ok = llabs(bf16_ord(g16) - bf16_ord(wqo_bf16_rne(r))) <= 2;
    const int abs_ok = fabs(g - r) <= floor_abs;
    return isfinite(g) && (ulp_ok || abs_ok);
}

static void grade(const char* what, const uint16_t* y_bits, int is_f16, const double* y64, int64_t M, int64_t N,
                  int64_t ldy, double floor_abs)
{
    int64_t bad = 0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            if (!element_ok(y_bits[m * ldy + n], is_f16, y64[m * N + n], floor_abs)) ++bad;
    CHECK(bad == 0, "%s: %lld of %lld outputs outside the tolerance", what, (long long)bad, (long long)(M * N));
}

/* CPU self-test of the rule above (no device): the floor at points where it
 * is a short decimal, and the element rule on both sides of the floor and of
 * the 2-ULP budget.  BF16 1.0 = 0x3F80; one ULP there is 2^-7. */
static int selftest(void)
{
    static const double pts[][4] = {  /* K, max|x|, max|w|, floor */
        {10000, 2.0, 0.5, 0.1}, {1, 1.0, 1.0, 0.001}, {16, 1.0, 1.0, 0.004},
        {256, 3.0, 0.25, 0.012}, {4, 0.5, 8.0, 0.008}, {1024, 1.0, 1.0, 0.032},
    };
    for (size_t i = 0; i < sizeof(pts) / sizeof(pts[0]); ++i) {
        const double f = abs_floor((int64_t)pts[i][0], pts[i][1], pts[i][2]);
        CHECK(fabs(f - pts[i][3]) <= 1e-15 * pts[i][3], "floor(%g, %g, %g) = %.17g, want %g", pts[i][0], pts[i][1],
              pts[i][2], f, pts[i][3]);
    }
    CHECK(element_ok(0x3F82, 0, 1.0, 0.0), "2 ULP above 1.0 must pass");
    CHECK(!element_ok(0x3F83, 0, 1.0, 0.0), "3 ULP above 1.0 must fail with no floor");
    const double e10 = 10.0 / 128.0;           /* 0x3F8A = 1 + 10 * 2^-7 */
    CHECK(element_ok(0x3F8A, 0, 1.0, e10 / 0.99), "10 ULP inside the floor must pass");
    CHECK(element_ok(0x3F8A, 0, 1.0, e10), "10 ULP at the floor must pass");
    CHECK(!element_ok(0x3F8A, 0, 1.0, e10 / 1.01), "10 ULP outside the floor must fail");
    CHECK(!element_ok(0x7F80, 0, 1.0, 1e30), "an infinity must fail");
    CHECK(!element_ok(0x7F80, 0, INFINITY, 1e30), "an infinity must fail where the sum is infinite too");
    CHECK(element_ok(0x3C00, 1, 1.0, 0.0), "FP16 1.0 must pass");
    CHECK(element_ok(0x3C08, 1, 1.0, 0.0), "FP16 1 + 8 ULP (1 BF16 ULP) must pass");
    CHECK(!element_ok(0x3C28, 1, 1.0, 0.0), "FP16 1 + 40 ULP (5 BF16 ULP) must fail");
    printf("%s: %d failed checks (self-test)\n", failures ? "FAIL" : "OK", failures);
    return failures ? 1 : 0;
}

static void test_fp8(void)
{
    const int64_t N = 256, K = 1024, MMAX = 32;
    uint8_t* codes = malloc(N * K);
    float* scales = malloc((N / 128) * (K / 128) * sizeof(float));
    uint16_t* x = malloc(MMAX * K * 2);
    for (int64_t i = 0; i < N * K; ++i) {
        uint8_t b = (uint8_t)(next_u64() & 0xFF);
        if ((b & 0x7F) == 0x7F) b ^= 1; /* no NaN codes */
        codes[i] = b;
    }
    for (int64_t i = 0; i < (N / 128) * (K / 128); ++i) scales[i] = (float)(0.0005 + 0.001 * uniform());
    double xmax = 0;
    for (int64_t i = 0; i < MMAX * K; ++i) {
        x[i] = bf16_bits((float)(2.0 * uniform() - 1.0));
        if (fabs(wqo_bf16_value(x[i])) > xmax) xmax = fabs(wqo_bf16_value(x[i]));
    }
    double* w = malloc(N * K * sizeof(double));
    wqo_dequant_fp8(codes, K, scales, N, K, w);
    double wmax = 0;
    for (int64_t i = 0; i < N * K; ++i)
        if (fabs(w[i]) > wmax) wmax = fabs(w[i]);
    free(w);
    const double floor_abs = abs_floor(K, xmax, wmax);

    uint8_t *d_codes, *d_packed;
    float* d_scales;
    uint16_t *d_x, *d_y;
    const size_t pbytes = wq_fp8_block_packed_bytes(N, K);
    CHECK(pbytes == (size_t)(N * K + 4 * (N / 128) * (K / 128)), "packed bytes %zu", pbytes);
    HIP_OK(hipMalloc((void**)&d_codes, N * K));
    HIP_OK(hipMalloc((void**)&d_scales, (N / 128) * (K / 128) * sizeof(float)));
    HIP_OK(hipMalloc((void**)&d_packed, pbytes));
    HIP_OK(hipMalloc((void**)&d_x, MMAX * K * 2));
    HIP_OK(hipMalloc((void**)&d_y, MMAX * N * 2));
    HIP_OK(hipMemcpy(d_codes, codes, N * K, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_scales, scales, (N / 128) * (K / 128) * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x, MMAX * K * 2, hipMemcpyHostToDevice));
    CHECK(wq_pack_fp8_block(d_codes, K, d_scales, N, K, d_packed, NULL) == WQ_OK, "pack fp8");

    const int64_t Ms[] = {1, 4, 5, 16, 32};
    uint16_t* y = malloc(MMAX * N * 2);
    double* y64 = malloc(MMAX * N * sizeof(double));
    for (int i = 0; i < 5; ++i) {
        const int64_t M = Ms[i];
        wqo_gemm_fp8(x, K, codes, K, scales, M, N, K, NULL, 0, y64, 4);
        for (int path = WQ_PATH_AUTO; path <= WQ_PATH_MFMA; ++path) {
            if (path == WQ_PATH_GEMV && M > 4) continue;
            HIP_OK(hipMemset(d_y, 0xFF, MMAX * N * 2));
            const wq_status st = wq_gemm_fp8_block_path(d_packed, N, K, d_x, K, d_y, N, M, NULL, 0, path, NULL);
            CHECK(st == WQ_OK, "gemm fp8 M=%lld path=%d: %s", (long long)M, path, wq_status_str(st));
            HIP_OK(hipDeviceSynchronize());
            HIP_OK(hipMemcpy(y, d_y, M * N * 2, hipMemcpyDeviceToHost));
            char what[64];
            snprintf(what, sizeof what, "fp8 M=%lld path=%d", (long long)M, path);
            grade(what, y, 0, y64, M, N, N, floor_abs);
        }
    }
    /* validation needs no device work */
    CHECK(wq_gemm_fp8_block(d_packed, N, K, d_x, K, d_y, N, 33, NULL, 0, NULL) == WQ_ERR_SHAPE, "M=33");
    CHECK(wq_gemm_fp8_block(NULL, N, K, d_x, K, d_y, N, 1, NULL, 0, NULL) == WQ_ERR_NULL, "NULL packed");
    CHECK(wq_gemm_fp8_block(d_packed, N, K, d_x, K - 8, d_y, N, 1, NULL, 0, NULL) == WQ_ERR_LD, "ldx < K");
    CHECK(wq_gemm_fp8_block(d_packed, N, 1000, d_x, K, d_y, N, 1, NULL, 0, NULL) == WQ_ERR_SHAPE, "K %% 128");
    CHECK(wq_gemm_fp8_block(d_packed, N, K, d_x, K, d_y, N, 0, NULL, 0, NULL) == WQ_OK, "M=0");
    free(codes), free(scales), free(x), free(y), free(y64);
    hipFree(d_codes), hipFree(d_scales), hipFree(d_packed), hipFree(d_x), hipFree(d_y);
}

static void test_lut3(int dense)
{
    const int64_t N = 96, K = 640, MMAX = 20;
    uint8_t* codes = malloc(N * K);
    uint16_t qmap[8], *g = malloc(N * (K / 128) * 2), *x = malloc(MMAX * K * 2);
    for (int64_t i = 0; i < N * K; ++i) codes[i] = (uint8_t)(next_u64() & 7);
    for (int i = 0; i < 8; ++i) qmap[i] = f16_bits_unit();
    for (int64_t i = 0; i < N * (K / 128); ++i) g[i] = (uint16_t)((8u << 10) | (next_u64() & 0x3FF)); /* ~0.008..0.016 */
    double xmax = 0;
    for (int64_t i = 0; i < MMAX * K; ++i) {
        x[i] = f16_bits_unit();
        if (fabs(wqo_f16_value(x[i])) > xmax) xmax = fabs(wqo_f16_value(x[i]));
    }
    double* w = malloc(N * K * sizeof(double));
    wqo_dequant_lut3(codes, K, qmap, g, N, K, w);
    double wmax = 0;
    for (int64_t i = 0; i < N * K; ++i)
        if (fabs(w[i]) > wmax) wmax = fabs(w[i]);
    free(w);
    const double floor_abs = abs_floor(K, xmax, wmax);

    const size_t pbytes = dense ? wq_lut3_dense_packed_bytes(N, K) : wq_lut3_packed_bytes(N, K);
    uint8_t *d_codes, *d_packed;
    uint16_t *d_qmap, *d_g, *d_x, *d_y;
    HIP_OK(hipMalloc((void**)&d_codes, N * K));
    HIP_OK(hipMalloc((void**)&d_qmap, 16));
    HIP_OK(hipMalloc((void**)&d_g, N * (K / 128) * 2));
    HIP_OK(hipMalloc((void**)&d_packed, pbytes));
    HIP_OK(hipMalloc((void**)&d_x, MMAX * K * 2));
    HIP_OK(hipMalloc((void**)&d_y, MMAX * N * 2));
    HIP_OK(hipMemcpy(d_codes, codes, N * K, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_qmap, qmap, 16, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_g, g, N * (K / 128) * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x, MMAX * K * 2, hipMemcpyHostToDevice));
    const wq_status ps = dense ? wq_pack_lut3_dense(d_codes, K, d_qmap, d_g, N, K, d_packed, NULL)
                               : wq_pack_lut3(d_codes, K, d_qmap, d_g, N, K, d_packed, NULL);
    CHECK(ps == WQ_OK, "pack lut3 dense=%d: %s", dense, wq_status_str(ps));

    const int64_t Ms[] = {1, 7, 16, 20};
    uint16_t* y = malloc(MMAX * N * 2);
    double* y64 = malloc(MMAX * N * sizeof(double));
    for (int i = 0; i < 4; ++i) {
        const int64_t M = Ms[i];
        wqo_gemm_lut3(x, K, codes, K, qmap, g, M, N, K, NULL, 0, y64, 4);
        HIP_OK(hipMemset(d_y, 0xFF, MMAX * N * 2));
        const wq_status st = dense ? wq_gemm_lut3_dense(d_packed, N, K, d_x, K, d_y, N, M, NULL, 0, NULL)
                                   : wq_gemm_lut3(d_packed, N, K, d_x, K, d_y, N, M, NULL, 0, NULL);
        CHECK(st == WQ_OK, "gemm lut3 dense=%d M=%lld: %s", dense, (long long)M, wq_status_str(st));
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(y, d_y, M * N * 2, hipMemcpyDeviceToHost));
        char what[64];
        snprintf(what, sizeof what, "lut3 dense=%d M=%lld", dense, (long long)M);
        grade(what, y, 1, y64, M, N, N, floor_abs);
    }
    /* a code above 7 is refused by the packer */
    uint8_t bad = 9;
    HIP_OK(hipMemcpy(d_codes + 5, &bad, 1, hipMemcpyHostToDevice));
    const wq_status cs = dense ? wq_pack_lut3_dense(d_codes, K, d_qmap, d_g, N, K, d_packed, NULL)
                               : wq_pack_lut3(d_codes, K, d_qmap, d_g, N, K, d_packed, NULL);
    CHECK(cs == WQ_ERR_CODE, "code 9 accepted: %s", wq_status_str(cs));
    free(codes), free(g), free(x), free(y), free(y64);
    hipFree(d_codes), hipFree(d_qmap), hipFree(d_g), hipFree(d_packed), hipFree(d_x), hipFree(d_y);
}

int main(int argc, char** argv)
{
    if (argc > 1 && !strcmp(argv[1], "--selftest")) return selftest();
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
        fprintf(stderr, "no HIP device\n");
        return 2;
    }
    printf("libwq packed format version %d\n", wq_packed_format_version());
    test_fp8();
    test_lut3(0);
    test_lut3(1);
    printf("%s: %d failed checks\n", failures ? "FAIL" : "OK", failures);
    return failures ? 1 : 0;
}
