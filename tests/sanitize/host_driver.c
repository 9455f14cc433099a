/* Host-code sanitizer driver: the oracle's and the input generators' C code
 * built with AddressSanitizer and UndefinedBehaviorSanitizer (see
 * tests/test_host_sanitizers.py) and run over every entry point on small
 * shapes of every weight format, f32 and bf16 activations, full and sampled
 * outputs.  Any out-of-bounds access, use after free, leak or undefined
 * operation aborts the run; the driver also checks that a sampled GEMM equals
 * the same entries of the full one bit for bit, and that every output is
 * finite.  Exit status 0 and "ok" on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle/oracle.c */
void oracle_dequant(int fmt, const uint8_t *W, int64_t N, int64_t K, double *w);
void oracle_quantize_act(const void *x, int x_dtype, int64_t M, int64_t K, int8_t *q, float *d,
                         int32_t *S);
void oracle_block_partials(int fmt, const uint8_t *W, const int8_t *qx, int64_t M, int64_t N,
                           int64_t K, int32_t *out);
int oracle_gemm(int fmt, const uint8_t *W, const void *x, int x_dtype, int64_t M, int64_t N,
                int64_t K, const int64_t *rows, int64_t nrows, const int64_t *cols, int64_t ncols,
                double *y);
void oracle_x_to_f16(const void *x, int x_dtype, int64_t M, int64_t K, uint16_t *x16);
void oracle_dequant_f16(int fmt, const uint8_t *W, int64_t N, int64_t K, uint16_t *w16);
int oracle_gemm_deq_f16(int fmt, const uint8_t *W, const void *x, int x_dtype, int64_t M,
                        int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
                        const int64_t *cols, int64_t ncols, double *y, double *yabs);
void oracle_quantize_act256(const void *x, int x_dtype, int64_t M, int64_t K, int8_t *q,
                            float *d256, int32_t *S32);
int oracle_gemm_a256(const uint8_t *W, const void *x, int x_dtype, int64_t M, int64_t N, int64_t K,
                     const int64_t *rows, int64_t nrows, const int64_t *cols, int64_t ncols,
                     double *y);
void oracle_rms_scale(const void *x, int x_dtype, int64_t M, int64_t K, float eps, float *r32,
                      float *r32_lo, float *r32_hi);
void oracle_rmsnorm(const void *x, int x_dtype, const float *g, const float *r32, int64_t M,
                    int64_t K, float *xn);
void oracle_swiglu(const double *gate, const double *up, int64_t n, double *h);

/* synth/synth.c */
void synth_normal_f32(uint64_t seed, int64_t n, double mean, double std, float *out);
void synth_student_t4_f32(uint64_t seed, int64_t n, float *out);
void synth_f32_to_bf16(const float *in, int64_t n, uint16_t *out);
void synth_pack_q4k(const float *w, int64_t N, int64_t K, uint8_t *out);
void synth_pack_q5k(const float *w, int64_t N, int64_t K, uint8_t *out);
void synth_pack_q6k(const float *w, int64_t N, int64_t K, uint8_t *out);
void synth_pack_q80(const float *w, int64_t N, int64_t K, uint8_t *out);
void synth_random_blocks(uint64_t seed, int fmt, int64_t nblocks, int emin, int emax,
                         int allow_negative, uint8_t *out);

static const int kBytes[4] = {144, 210, 176, 272}; /* Q4_K, Q6_K, Q5_K, Q8_0 per 256 values */

static int fail(const char *what) {
    fprintf(stderr, "FAIL: %s\n", what);
    return 1;
}

static int finite_all(const double *v, int64_t n) {
    for (int64_t i = 0; i < n; i++)
        if (!isfinite(v[i])) return 0;
    return 1;
}

static int run_format(int fmt, int64_t M, int64_t N, int64_t K, int packed) {
    const int64_t wbytes = N * (K / 256) * kBytes[fmt];
    uint8_t *W = malloc((size_t)wbytes);
    float *wf = malloc(sizeof(float) * (size_t)(N * K));
    synth_normal_f32(11 + fmt, N * K, 0.0, 0.02, wf);
    if (packed) {
        if (fmt == 0) synth_pack_q4k(wf, N, K, W);
        else if (fmt == 1) synth_pack_q6k(wf, N, K, W);
        else if (fmt == 2) synth_pack_q5k(wf, N, K, W);
        else synth_pack_q80(wf, N, K, W);
    } else {
        synth_random_blocks(21 + fmt, fmt, N * (K / 256), 1, 14, 1, W);
    }
    float *xf = malloc(sizeof(float) * (size_t)(M * K));
    synth_student_t4_f32(31 + fmt, M * K, xf);
    uint16_t *xb = malloc(sizeof(uint16_t) * (size_t)(M * K));
    synth_f32_to_bf16(xf, M * K, xb);

    double *w = malloc(sizeof(double) * (size_t)(N * K));
    oracle_dequant(fmt, W, N, K, w);
    if (!finite_all(w, N * K)) return fail("dequant");

    int8_t *q = malloc((size_t)(M * K));
    float *d = malloc(sizeof(float) * (size_t)(M * K / 32));
    int32_t *S = malloc(sizeof(int32_t) * (size_t)(M * K / 32));
    oracle_quantize_act(xb, 1, M, K, q, d, S);
    oracle_quantize_act(xf, 0, M, K, q, d, S);
    const int64_t per = fmt == 1 ? K / 16 : K / 32;
    int32_t *part = malloc(sizeof(int32_t) * (size_t)(M * N * per));
    oracle_block_partials(fmt, W, q, M, N, K, part);

    double *y = malloc(sizeof(double) * (size_t)(M * N));
    if (oracle_gemm(fmt, W, xb, 1, M, N, K, NULL, 0, NULL, 0, y)) return fail("gemm alloc");
    if (!finite_all(y, M * N)) return fail("gemm");
    const int64_t rows[2] = {M - 1, 0}, cols[3] = {N - 1, 1, 0};
    double ys[6];
    if (oracle_gemm(fmt, W, xb, 1, M, N, K, rows, 2, cols, 3, ys)) return fail("gemm sampled alloc");
    for (int i = 0; i < 2; i++)
        for (int j = 0; j < 3; j++)
            if (memcmp(&ys[i * 3 + j], &y[rows[i] * N + cols[j]], sizeof(double)) != 0)
                return fail("sampled gemm differs from the full one");

    if (fmt == 0 || fmt == 1) {
        uint16_t *x16 = malloc(sizeof(uint16_t) * (size_t)(M * K));
        uint16_t *w16 = malloc(sizeof(uint16_t) * (size_t)(N * K));
        oracle_x_to_f16(xb, 1, M, K, x16);
        oracle_dequant_f16(fmt, W, N, K, w16);
        double *ya = malloc(sizeof(double) * (size_t)(M * N));
        if (oracle_gemm_deq_f16(fmt, W, xb, 1, M, N, K, NULL, 0, NULL, 0, y, ya)) return fail("f16 alloc");
        if (!finite_all(y, M * N) || !finite_all(ya, M * N)) return fail("gemm_deq_f16");
        free(x16);
        free(w16);
        free(ya);
    }
    if (fmt == 0) {
        float *d256 = malloc(sizeof(float) * (size_t)(M * K / 256));
        oracle_quantize_act256(xb, 1, M, K, q, d256, S);
        if (oracle_gemm_a256(W, xb, 1, M, N, K, rows, 2, cols, 3, ys)) return fail("a256 alloc");
        if (!finite_all(ys, 6)) return fail("gemm_a256");
        free(d256);
    }
    free(W);
    free(wf);
    free(xf);
    free(xb);
    free(w);
    free(q);
    free(d);
    free(S);
    free(part);
    free(y);
    return 0;
}

int main(void) {
    for (int fmt = 0; fmt < 4; fmt++)
        for (int packed = 0; packed < 2; packed++)
            if (run_format(fmt, 3, 5, 512, packed)) return 1;
    /* RMSNorm pieces and SwiGLU */
    const int64_t M = 2, K = 256;
    float *x = malloc(sizeof(float) * (size_t)(M * K)), *g = malloc(sizeof(float) * (size_t)K);
    float *xn = malloc(sizeof(float) * (size_t)(M * K));
    float r32[2], lo[2], hi[2];
    synth_normal_f32(41, M * K, 0.0, 1.0, x);
    synth_normal_f32(42, K, 1.0, 0.1, g);
    oracle_rms_scale(x, 0, M, K, 1e-6f, r32, lo, hi);
    oracle_rmsnorm(x, 0, g, r32, M, K, xn);
    double gate[4] = {-3.0, -0.5, 0.25, 7.0}, up[4] = {1.0, 2.0, -1.0, 0.5}, h[4];
    oracle_swiglu(gate, up, 4, h);
    if (!finite_all(h, 4)) return fail("swiglu");
    free(x);
    free(g);
    free(xn);
    printf("ok\n");
    return 0;
}
