/*
 * oracle.c -- plain CPU reference for the Q4_K / Q6_K x int8 prefill GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test-suite, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source, header, table or helper with the
 * GPU library.
 *
 * What it computes (each step cites the page it follows):
 *
 *  - The method: a batched prefill matmul y[M x N] = x[M x K] . W[N x K]^T in
 *    which the weights stay in their GGUF Q4_K / Q6_K super-blocks, are decoded
 *    to small integers in place, the activation rows are quantised to int8, the
 *    contraction is an int8 x int8 -> int32 dot product and the block scales are
 *    applied afterwards.  Pages: sparkinfer PR #464 "fused Q4K/Q6K->int8 dequant
 *    + token-parallel GDN conv + lane-parallel fallback attention", section
 *    "Summary" (decode super-blocks in registers, int8 tensor-core GEMM);
 *    aprender issue #5475 "Qwen3.5 on CPU prefills one token at a time",
 *    section "Ask" (the row-batched fused Q4_K x int8-activation kernel, as
 *    opposed to dequantising a tile to F32); aprender issue #5305 "Qwen3.5
 *    speed: prefill and decode parity with llama.cpp", sub-ticket #4313 (int8
 *    MMQ prefill matmul plus the LM head on the last token only).
 *  - Activation encoding: per 32 consecutive values of a row, int8 codes with
 *    one fp32 scale and the int32 sum of the codes, the q8_1-style block the
 *    CRUX parity issue #4220 ranks as technique 5 (quantised-activation GEMV,
 *    "q8_1 + dp4a").  The pages give no formula; the plainest symmetric reading
 *    is taken: scale d = amax/127 in fp32, codes rint(x * (1/d)) with ties to
 *    even, clamped to [-127, 127], code 0 wherever x = 0.
 *  - Block layout: the public GGUF K-quant layout (the pages name Q4_K / Q6_K
 *    but do not print their bytes):
 *      Q4_K, 144 B / 256 values: fp16 d, fp16 dmin, 12 bytes of 6-bit sub-block
 *        scales sc[8] and mins m[8], 128 bytes of 4-bit codes q in [0, 15];
 *        w = d*sc[j]*q - dmin*m[j] for sub-block j = v/32.
 *      Q6_K, 210 B / 256 values: ql[128] low nibbles, qh[64] high bit pairs,
 *        16 int8 sub-block scales (16 values each), fp16 d;
 *        w = d*sc[v/16]*(q6 - 32), q6 in [0, 63].
 *      Q5_K, 176 B / 256 values (named beside Q4_K / Q6_K in aprender issue
 *        #5305's decode-GEMV ticket #5221, where it is the slowest format): the
 *        Q4_K header (fp16 d, dmin, the same 12 bytes of 6-bit sc[8] / m[8]),
 *        qh[32] holding the fifth bit of every code, 128 bytes of low nibbles
 *        placed as Q4_K's codes; q5 = low | 16*((qh[v % 32] >> (v / 32)) & 1)
 *        in [0, 31]; w = d*sc[j]*q5 - dmin*m[j] for sub-block j = v/32.
 *      Q8_0, 34 B / 32 values (named on aprender issue #5475's page among the
 *        formats its CPU path runs row by row): fp16 d, then 32 int8 codes q;
 *        w = d*q.  No mins.
 *
 * The combine is done in fp64 in ascending block order.  Integer partials are
 * exact int32.  All floating point here is IEEE binary32/binary64 with no
 * contraction (built with -ffp-contract=off, no fast-math), so the fp32 steps
 * of the activation quantiser are the correctly rounded ones.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_Q4_K = 0, ORACLE_Q6_K = 1, ORACLE_Q5_K = 2, ORACLE_Q8_0 = 3 };
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Threads an OpenMP region of this library runs on (for reporting the CPU
 * baseline's core count; no arithmetic). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* IEEE binary16 bit pattern -> exact double (normals, subnormals, inf, nan). */
double oracle_half_to_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)f, -24);                 /* 0 or subnormal: f * 2^-24 */
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(f | 0x400), e - 25);           /* (1024 + f) * 2^(e-25) */
    return sign ? -v : v;
}

static inline uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ---------------------------------------------------------------- Q4_K decode */

/* The 16-byte header Q4_K and Q5_K share: the two binary16 super-scales as
 * doubles and the six-bit scales sc[8] and mins m[8]. */
static void decode_k_header(const uint8_t *blk, uint8_t *sc, uint8_t *m, double *d, double *dmin) {
    *d = oracle_half_to_double(rd16(blk));
    *dmin = oracle_half_to_double(rd16(blk + 2));
    const uint8_t *s = blk + 4;
    for (int j = 0; j < 8; j++) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            m[j] = s[j + 4] & 63;
        } else {
            /* low 4 bits from byte j+4 (scale: low nibble, min: high nibble),
             * high 2 bits from the top of byte j-4 (scale) or byte j (min) */
            sc[j] = (uint8_t)((s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4));
            m[j] = (uint8_t)((s[j + 4] >> 4) | ((s[j] >> 6) << 4));
        }
    }
}

/* Low four bits of the 256 codes from the 128 nibble bytes qs: value v sits in
 * byte 32*(v/64) + v%32, the low nibble for the first 32 values of each 64. */
static void decode_nibbles(const uint8_t *qs, uint8_t *q) {
    for (int v = 0; v < 256; v++) {
        uint8_t byte = qs[32 * (v / 64) + (v % 32)];
        q[v] = (v % 64) < 32 ? (byte & 0x0F) : (byte >> 4);
    }
}

/* Decode one Q4_K block into codes q[256] (0..15), scales sc[8], mins m[8],
 * and the two binary16 super-scales as doubles. */
static void decode_q4k_block(const uint8_t *blk, uint8_t *q, uint8_t *sc, uint8_t *m,
                             double *d, double *dmin) {
    decode_k_header(blk, sc, m, d, dmin);
    decode_nibbles(blk + 16, q);
}

/* Decode one Q5_K block into codes q[256] (0..31), scales, mins and super-scales
 * (the Q4_K header; qh at bytes 16-47, nibbles at 48-175). */
static void decode_q5k_block(const uint8_t *blk, uint8_t *q, uint8_t *sc, uint8_t *m,
                             double *d, double *dmin) {
    decode_k_header(blk, sc, m, d, dmin);
    const uint8_t *qh = blk + 16;
    decode_nibbles(blk + 48, q);
    for (int v = 0; v < 256; v++) q[v] = (uint8_t)(q[v] | (((qh[v % 32] >> (v / 32)) & 1) << 4));
}

/* Decode W [N x K] Q4_K: q [N*K], sc, m [N*K/32], d, dmin [N*K/256]. */
void oracle_decode_q4k(const uint8_t *W, int64_t N, int64_t K, uint8_t *q, uint8_t *sc,
                       uint8_t *m, double *d, double *dmin) {
    int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N * nb; i++)
        decode_q4k_block(W + i * 144, q + i * 256, sc + i * 8, m + i * 8, d + i, dmin + i);
}

/* Decode W [N x K] Q5_K: q [N*K] (0..31), sc, m [N*K/32], d, dmin [N*K/256]. */
void oracle_decode_q5k(const uint8_t *W, int64_t N, int64_t K, uint8_t *q, uint8_t *sc,
                       uint8_t *m, double *d, double *dmin) {
    int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N * nb; i++)
        decode_q5k_block(W + i * 176, q + i * 256, sc + i * 8, m + i * 8, d + i, dmin + i);
}

/* ---------------------------------------------------------------- Q8_0 decode */

/* Decode W [N x K] Q8_0 (K % 32 == 0): q [N*K] int8, d [N*K/32]. */
void oracle_decode_q80(const uint8_t *W, int64_t N, int64_t K, int8_t *q, double *d) {
    int64_t nb = N * (K / 32);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nb; i++) {
        const uint8_t *blk = W + i * 34;
        d[i] = oracle_half_to_double(rd16(blk));
        for (int t = 0; t < 32; t++) q[i * 32 + t] = (int8_t)blk[2 + t];
    }
}

/* ---------------------------------------------------------------- Q6_K decode */

/* Decode one Q6_K block into 6-bit codes q6[256] (0..63), scales sc[16], d. */
static void decode_q6k_block(const uint8_t *blk, uint8_t *q6, int8_t *sc, double *d) {
    const uint8_t *ql = blk, *qh = blk + 128;
    for (int v = 0; v < 256; v++) {
        int half = v / 128, r = v % 128, quarter = r / 32, l = r % 32;
        uint8_t lowbyte = ql[64 * half + 32 * (quarter % 2) + l];
        int lo = quarter < 2 ? (lowbyte & 0x0F) : (lowbyte >> 4);
        int hi = (qh[32 * half + l] >> (2 * quarter)) & 3;
        q6[v] = (uint8_t)(lo | (hi << 4));
    }
    for (int s = 0; s < 16; s++) sc[s] = (int8_t)blk[192 + s];
    *d = oracle_half_to_double(rd16(blk + 208));
}

/* Decode W [N x K] Q6_K: q6 [N*K], sc [N*K/16], d [N*K/256]. */
void oracle_decode_q6k(const uint8_t *W, int64_t N, int64_t K, uint8_t *q6, int8_t *sc,
                       double *d) {
    int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N * nb; i++)
        decode_q6k_block(W + i * 210, q6 + i * 256, sc + i * 16, d + i);
}

/* Dequantised weights w [N x K] in fp64 (brute-force reference values). */
void oracle_dequant(int fmt, const uint8_t *W, int64_t N, int64_t K, double *w) {
    if (fmt == ORACLE_Q8_0) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < N * (K / 32); i++) {
            double d = oracle_half_to_double(rd16(W + i * 34));
            for (int t = 0; t < 32; t++) w[i * 32 + t] = d * (double)(int8_t)W[i * 34 + 2 + t];
        }
        return;
    }
    int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N * nb; i++) {
        uint8_t q[256];
        double *o = w + i * 256;
        if (fmt == ORACLE_Q4_K || fmt == ORACLE_Q5_K) {
            uint8_t sc[8], m[8];
            double d, dmin;
            if (fmt == ORACLE_Q4_K) decode_q4k_block(W + i * 144, q, sc, m, &d, &dmin);
            else decode_q5k_block(W + i * 176, q, sc, m, &d, &dmin);
            for (int v = 0; v < 256; v++) o[v] = d * sc[v / 32] * q[v] - dmin * m[v / 32];
        } else {
            int8_t sc[16];
            double d;
            decode_q6k_block(W + i * 210, q, sc, &d);
            for (int v = 0; v < 256; v++) o[v] = d * sc[v / 16] * ((int)q[v] - 32);
        }
    }
}

/* ------------------------------------------------------- activation quantiser */

static inline float load_x(const void *x, int x_dtype, int64_t i) {
    if (x_dtype == ORACLE_F32) return ((const float *)x)[i];
    uint32_t u = (uint32_t)((const uint16_t *)x)[i] << 16; /* bf16 -> f32 is exact */
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* One 32-value block: amax, d = amax/127 (fp32 division), id = 1/d (fp32
 * division), q = rint(x*id) (one fp32 multiply, ties to even) clamped to
 * [-127, 127]; q = 0 where x = 0; S = sum q.  All-zero block: d = 0, q = 0. */
static void quantize_block(const float *xf, int8_t *q, float *d_out, int32_t *S_out) {
    float amax = 0.0f;
    for (int t = 0; t < 32; t++) {
        float a = fabsf(xf[t]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        memset(q, 0, 32);
        *d_out = 0.0f;
        *S_out = 0;
        return;
    }
    float d = amax / 127.0f;
    float id = 1.0f / d;
    int32_t S = 0;
    for (int t = 0; t < 32; t++) {
        int qi = 0;
        if (xf[t] != 0.0f) {
            float v = xf[t] * id;
            float r = rintf(v);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            qi = (int)r;
        }
        q[t] = (int8_t)qi;
        S += qi;
    }
    *d_out = d;
    *S_out = S;
}

/* x [M x K] (fp32 or bf16 bits) -> q int8 [M x K], d fp32 [M x K/32], S int32 [M x K/32]. */
void oracle_quantize_act(const void *x, int x_dtype, int64_t M, int64_t K, int8_t *q,
                         float *d, int32_t *S) {
    int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; r++) {
        float xf[32];
        for (int64_t b = 0; b < nb; b++) {
            for (int t = 0; t < 32; t++) xf[t] = load_x(x, x_dtype, r * K + 32 * b + t);
            quantize_block(xf, q + r * K + 32 * b, d + r * nb + b, S + r * nb + b);
        }
    }
}

/* ----------------------------------------------------- integer block partials */

/* Q4_K, Q5_K, Q8_0: out[m][n][b] = sum_{t<32} q_w[n][32b+t] * q_x[m][32b+t] (K/32 per pair)
 * Q6_K: out[m][n][s] = sum_{t<16} (q6[n][16s+t] - 32) * q_x[m][16s+t] (K/16 per pair) */
void oracle_block_partials(int fmt, const uint8_t *W, const int8_t *qx, int64_t M, int64_t N,
                           int64_t K, int32_t *out) {
    uint8_t *qw = (uint8_t *)malloc((size_t)(N * K));
    int64_t nb = K / 256;
    if (fmt == ORACLE_Q8_0) {
        int8_t *q8 = malloc((size_t)(N * K));
        double *d = malloc(sizeof(double) * (size_t)(N * K / 32));
        oracle_decode_q80(W, N, K, q8, d);
        int64_t nblk = K / 32;
#pragma omp parallel for collapse(2) schedule(static)
        for (int64_t mi = 0; mi < M; mi++)
            for (int64_t n = 0; n < N; n++)
                for (int64_t b = 0; b < nblk; b++) {
                    int32_t acc = 0;
                    for (int t = 0; t < 32; t++)
                        acc += (int32_t)q8[n * K + b * 32 + t] * (int32_t)qx[mi * K + b * 32 + t];
                    out[(mi * N + n) * nblk + b] = acc;
                }
        free(q8); free(d); free(qw);
        return;
    }
    if (fmt == ORACLE_Q4_K || fmt == ORACLE_Q5_K) {
        uint8_t *sc = malloc((size_t)(N * K / 32)), *m = malloc((size_t)(N * K / 32));
        double *d = malloc(sizeof(double) * (size_t)(N * nb)), *dm = malloc(sizeof(double) * (size_t)(N * nb));
        if (fmt == ORACLE_Q4_K) oracle_decode_q4k(W, N, K, qw, sc, m, d, dm);
        else oracle_decode_q5k(W, N, K, qw, sc, m, d, dm);
        free(sc); free(m); free(d); free(dm);
    } else {
        int8_t *sc = malloc((size_t)(N * K / 16));
        double *d = malloc(sizeof(double) * (size_t)(N * nb));
        oracle_decode_q6k(W, N, K, qw, sc, d);
        free(sc); free(d);
    }
    int L = fmt == ORACLE_Q6_K ? 16 : 32, off = fmt == ORACLE_Q6_K ? 32 : 0;
    int64_t nblk = K / L;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t mi = 0; mi < M; mi++)
        for (int64_t n = 0; n < N; n++)
            for (int64_t b = 0; b < nblk; b++) {
                int32_t acc = 0;
                for (int t = 0; t < L; t++)
                    acc += ((int32_t)qw[n * K + b * L + t] - off) * (int32_t)qx[mi * K + b * L + t];
                out[(mi * N + n) * nblk + b] = acc;
            }
    free(qw);
}

/* ------------------------------------------------------------------- the GEMM */

/* y[i][j] for the selected rows m = rows[i] of x and columns n = cols[j] of W
 * (rows == NULL: all M rows; cols == NULL: all N columns).  y is fp64
 * [nrows x ncols].  Steps: quantise the activation rows, decode the weight
 * rows, form every per-block int32 dot product, then combine in fp64 in
 * ascending block order:
 *   Q4_K, Q5_K: y = sum_b dx[b] * ( d*sc[b]*I[b] - dmin*m[b]*S[b] )
 *   Q8_0: y = sum_b dx[b] * d[b] * I[b]  (d the weight block's own scale)
 *   Q6_K: y = sum_b dx[b] * d * ( sc[2b]*I16[2b] + sc[2b+1]*I16[2b+1] )
 * where b runs over 32-value activation blocks and d, dmin belong to the
 * super-block holding b.  Returns 0, or -1 on allocation failure. */
int oracle_gemm(int fmt, const uint8_t *W, const void *x, int x_dtype, int64_t M, int64_t N,
                int64_t K, const int64_t *rows, int64_t nrows, const int64_t *cols, int64_t ncols,
                double *y) {
    if (!rows) nrows = M;
    if (!cols) ncols = N;
    int64_t nb32 = K / 32, nsb = K / 256;
    int64_t bbytes = fmt == ORACLE_Q4_K ? 144 : fmt == ORACLE_Q5_K ? 176 : fmt == ORACLE_Q8_0 ? 272 : 210;

    int8_t *qx = malloc((size_t)(nrows * K));
    float *dx = malloc(sizeof(float) * (size_t)(nrows * nb32));
    int32_t *Sx = malloc(sizeof(int32_t) * (size_t)(nrows * nb32));
    uint8_t *qw = malloc((size_t)(ncols * K));
    uint8_t *scw = malloc((size_t)(ncols * K / 16));   /* Q4_K uses K/32 of it */
    uint8_t *mw = malloc((size_t)(ncols * nb32));
    double *dw = malloc(sizeof(double) * (size_t)(ncols * nb32));   /* Q8_0: one per 32 values */
    double *dmw = malloc(sizeof(double) * (size_t)(ncols * nsb));
    if (!qx || !dx || !Sx || !qw || !scw || !mw || !dw || !dmw) {
        free(qx); free(dx); free(Sx); free(qw); free(scw); free(mw); free(dw); free(dmw);
        return -1;
    }

    /* 1. quantise the selected activation rows */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; i++) {
        int64_t r = rows ? rows[i] : i;
        float xf[32];
        for (int64_t b = 0; b < nb32; b++) {
            for (int t = 0; t < 32; t++) xf[t] = load_x(x, x_dtype, r * K + 32 * b + t);
            quantize_block(xf, qx + i * K + 32 * b, dx + i * nb32 + b, Sx + i * nb32 + b);
        }
    }
    /* 2. decode the selected weight rows */
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < ncols; j++) {
        int64_t n = cols ? cols[j] : j;
        if (fmt == ORACLE_Q8_0) {
            oracle_decode_q80(W + n * nsb * bbytes, 1, K, (int8_t *)qw + j * K, dw + j * nb32);
            continue;
        }
        for (int64_t sb = 0; sb < nsb; sb++) {
            const uint8_t *blk = W + (n * nsb + sb) * bbytes;
            if (fmt == ORACLE_Q4_K)
                decode_q4k_block(blk, qw + j * K + 256 * sb, scw + j * nb32 + 8 * sb,
                                 mw + j * nb32 + 8 * sb, dw + j * nsb + sb, dmw + j * nsb + sb);
            else if (fmt == ORACLE_Q5_K)
                decode_q5k_block(blk, qw + j * K + 256 * sb, scw + j * nb32 + 8 * sb,
                                 mw + j * nb32 + 8 * sb, dw + j * nsb + sb, dmw + j * nsb + sb);
            else
                decode_q6k_block(blk, qw + j * K + 256 * sb, (int8_t *)scw + j * (K / 16) + 16 * sb,
                                 dw + j * nsb + sb);
        }
    }
    /* 3. per-block int32 dots, fp64 combine in ascending b */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < nrows; i++)
        for (int64_t j = 0; j < ncols; j++) {
            const int8_t *xq = qx + i * K;
            const uint8_t *wq = qw + j * K;
            double acc = 0.0;
            for (int64_t b = 0; b < nb32; b++) {
                double d = dw[j * nsb + b / 8];
                double dxb = (double)dx[i * nb32 + b];
                if (fmt == ORACLE_Q8_0) {
                    const int8_t *w8 = (const int8_t *)wq;
                    int32_t I = 0;
                    for (int t = 0; t < 32; t++) I += (int32_t)w8[32 * b + t] * (int32_t)xq[32 * b + t];
                    acc += dxb * dw[j * nb32 + b] * (double)I;
                } else if (fmt != ORACLE_Q6_K) {  /* Q4_K, Q5_K */
                    int32_t I = 0;
                    for (int t = 0; t < 32; t++) I += (int32_t)wq[32 * b + t] * (int32_t)xq[32 * b + t];
                    double sc = scw[j * nb32 + b], m = mw[j * nb32 + b];
                    double dmin = dmw[j * nsb + b / 8];
                    acc += dxb * (d * sc * (double)I - dmin * m * (double)Sx[i * nb32 + b]);
                } else {
                    int32_t Ia = 0, Ib = 0;
                    for (int t = 0; t < 16; t++) Ia += ((int32_t)wq[32 * b + t] - 32) * (int32_t)xq[32 * b + t];
                    for (int t = 16; t < 32; t++) Ib += ((int32_t)wq[32 * b + t] - 32) * (int32_t)xq[32 * b + t];
                    const int8_t *sc = (const int8_t *)scw + j * (K / 16);
                    acc += dxb * d * ((double)sc[2 * b] * (double)Ia + (double)sc[2 * b + 1] * (double)Ib);
                }
            }
            y[i * ncols + j] = acc;
        }
    free(qx); free(dx); free(Sx); free(qw); free(scw); free(mw); free(dw); free(dmw);
    return 0;
}

/* ============================================================================
 * The other design branch: dequantise the weights to 16-bit floats and run a
 * float GEMM on them.  aprender issue #5475 ("apr serve / apr run: Qwen3.5 on
 * CPU prefills one token at a time ..."), section "Ask", item 1, names it as
 * the alternative to the fused Q4_K x int8 kernel (there: dequantise a tile to
 * F32 and call the GEMM); aprender issue #4220 ("CRUX parity spike ..."),
 * section "Readings", has the serving path hold the prefill weights as a
 * dense fp16 copy.  On the matrix cores a float GEMM takes 16-bit operands,
 * so this branch dequantises to IEEE binary16 (11 significant bits, against
 * bfloat16's 8).  The pages fix no rounding; the reading taken here rounds
 * each step once, to nearest with ties to even:
 *   x16  = f16(x)                         (x as its fp32 value; bf16 widens exactly)
 *   Q4_K: dsc = f16(d*sc[j]), dmn = f16(dmin*m[j]), w16 = f16(dsc*q - dmn)
 *   Q6_K: dsc = f16(d*sc[s]),                       w16 = f16(dsc*(q6 - 32))
 *   y[m][n] = sum_k x16[m][k] * w16[n][k]   (exact products, fp64 sum)
 * where f16(v) is the binary16 value nearest to the exact real v (ties to the
 * even significand, magnitudes from 65520 up to infinity).  Every f16() here is
 * applied to an exactly known value, so there is one rounding per step.
 * ========================================================================== */

/* binary16 bits of the value nearest to D * 2^e (D an exact integer). */
static uint16_t f16_round_scaled(int64_t D, int e) {
    uint16_t sign = 0;
    if (D < 0) { sign = 0x8000; D = -D; }
    if (D == 0) return sign;
    /* normalise: D < 2^62 so that shifting left stays exact */
    while (D >= ((int64_t)1 << 62)) {            /* keep a sticky bit while halving */
        int64_t lost = D & 1;
        D = (D >> 1) | lost;
        e += 1;
    }
    int top = 63 - __builtin_clzll((unsigned long long)D);   /* value in [2^(top+e), 2^(top+e+1)) */
    int ev = top + e;                                         /* exponent of the leading bit */
    int qe = ev - 10 < -24 ? -24 : ev - 10;                   /* exponent of one unit in the last place */
    int64_t r;
    if (qe <= e) {
        r = D << (e - qe);                                    /* exact: no bits below the quantum */
    } else {
        int sh = qe - e;
        if (sh > 62) return sign;                             /* far below half the smallest subnormal */
        int64_t keep = D >> sh, rem = D - (keep << sh), half = (int64_t)1 << (sh - 1);
        r = keep + ((rem > half || (rem == half && (keep & 1))) ? 1 : 0);
    }
    /* r counts quanta of 2^qe; for normals r is in [1024, 2048] */
    if (qe == -24 && r < 1024) return (uint16_t)(sign | r);   /* subnormal */
    if (r == 2048) { r = 1024; qe += 1; }
    if (qe - (-24) > 29) return (uint16_t)(sign | 0x7C00);    /* past the largest finite value */
    int ebits = qe + 25;                                      /* biased exponent: value = r * 2^qe */
    if (ebits >= 31) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (ebits << 10) | (r - 1024));
}

/* binary16 bits of the value nearest to the finite double v. */
uint16_t oracle_f64_to_f16(double v) {
    if (v != v) return 0x7E00;
    if (v == INFINITY) return 0x7C00;
    if (v == -INFINITY) return 0xFC00;
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    int e;
    double fr = frexp(v, &e);                 /* v = fr * 2^e, 0.5 <= |fr| < 1 */
    int64_t D = (int64_t)ldexp(fr, 53);       /* exact: 53 significant bits */
    return f16_round_scaled(D, e - 53);
}

/* A binary16 value as an exact integer significand and exponent: v = sig * 2^ex. */
static void f16_split(uint16_t h, int64_t *sig, int *ex) {
    int s = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
    int64_t m = e == 0 ? f : (f | 0x400);
    *sig = s ? -m : m;
    *ex = e == 0 ? -24 : e - 25;
}

/* x [M x K] (fp32 or bf16) -> binary16 bits. */
void oracle_x_to_f16(const void *x, int x_dtype, int64_t M, int64_t K, uint16_t *x16) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M * K; i++) x16[i] = oracle_f64_to_f16((double)load_x(x, x_dtype, i));
}

/* The binary16 weights w16 [N x K] of the rounding chain above. */
void oracle_dequant_f16(int fmt, const uint8_t *W, int64_t N, int64_t K, uint16_t *w16) {
    int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N * nb; i++) {
        uint8_t q[256];
        uint16_t *o = w16 + i * 256;
        if (fmt == ORACLE_Q4_K) {
            uint8_t sc[8], m[8];
            double d, dmin;
            decode_q4k_block(W + i * 144, q, sc, m, &d, &dmin);
            for (int j = 0; j < 8; j++) {
                int64_t a, b;
                int ea, eb;
                f16_split(oracle_f64_to_f16(d * sc[j]), &a, &ea);     /* d*sc is exact in fp64 */
                f16_split(oracle_f64_to_f16(dmin * m[j]), &b, &eb);
                int e0 = ea < eb ? ea : eb;
                for (int t = 0; t < 32; t++) {
                    /* dsc*q - dmn exactly, as an integer times 2^e0 (< 2^60) */
                    int64_t D = a * q[32 * j + t] * ((int64_t)1 << (ea - e0)) - b * ((int64_t)1 << (eb - e0));
                    o[32 * j + t] = f16_round_scaled(D, e0);
                }
            }
        } else {
            int8_t sc[16];
            double d;
            decode_q6k_block(W + i * 210, q, sc, &d);
            for (int s = 0; s < 16; s++) {
                int64_t a;
                int ea;
                f16_split(oracle_f64_to_f16(d * sc[s]), &a, &ea);
                for (int t = 0; t < 16; t++)
                    o[16 * s + t] = f16_round_scaled(a * ((int64_t)q[16 * s + t] - 32), ea);
            }
        }
    }
}

/* y [nrows x ncols] = x16 . w16^T in fp64 over the selected rows / columns
 * (all when rows / cols is NULL), plus yabs = sum_k |x16*w16| (the scale of the
 * fp32 summation error the GPU is allowed).  Returns 0, or -1 on allocation
 * failure. */
int oracle_gemm_deq_f16(int fmt, const uint8_t *W, const void *x, int x_dtype, int64_t M,
                        int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
                        const int64_t *cols, int64_t ncols, double *y, double *yabs) {
    if (!rows) nrows = M;
    if (!cols) ncols = N;
    int64_t bbytes = fmt == ORACLE_Q4_K ? 144 : 210, nsb = K / 256;
    double *xd = malloc(sizeof(double) * (size_t)(nrows * K));
    double *wd = malloc(sizeof(double) * (size_t)(ncols * K));
    uint16_t *tmp = malloc(sizeof(uint16_t) * (size_t)K);
    if (!xd || !wd || !tmp) { free(xd); free(wd); free(tmp); return -1; }
    free(tmp);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; i++) {
        int64_t r = rows ? rows[i] : i;
        for (int64_t k = 0; k < K; k++)
            xd[i * K + k] = oracle_half_to_double(oracle_f64_to_f16((double)load_x(x, x_dtype, r * K + k)));
    }
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < ncols; j++) {
        int64_t n = cols ? cols[j] : j;
        uint16_t w16[256];
        for (int64_t sb = 0; sb < nsb; sb++) {
            oracle_dequant_f16(fmt, W + (n * nsb + sb) * bbytes, 1, 256, w16);
            for (int v = 0; v < 256; v++) wd[j * K + 256 * sb + v] = oracle_half_to_double(w16[v]);
        }
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < nrows; i++)
        for (int64_t j = 0; j < ncols; j++) {
            double acc = 0.0, aabs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = xd[i * K + k] * wd[j * K + k];   /* exact: 11 x 11 significant bits */
                acc += p;
                aabs += fabs(p);
            }
            y[i * ncols + j] = acc;
            if (yabs) yabs[i * ncols + j] = aabs;
        }
    free(xd); free(wd);
    return 0;
}

/* ============================================================================
 * Per-256 activation scales (the Q8_K-style activation block the CPU issue
 * names, aprender issue #5475, section "Ask", item 1: "Q4_K x Q8_K"): one fp32
 * scale per 256-value super-block instead of per 32 values.  The steps are the
 * per-32 quantiser's over 256 values (amax, d = amax/127, id = 1/d, q =
 * rint(x*id) clamped to [-127, 127], q = 0 where x = 0), and the int32 code sum
 * is kept per 32-value sub-block (the weight mins are per sub-block).  The
 * combine is the per-32 formula with every sub-block of a super-block sharing
 * its scale:
 *   Q4_K: y = sum_sb dx[sb] * sum_j ( d*sc[j]*I[j] - dmin*m[j]*S[j] )
 * ========================================================================== */

/* x [M x K] -> q int8 [M x K], d fp32 [M x K/256], S int32 [M x K/32]. */
void oracle_quantize_act256(const void *x, int x_dtype, int64_t M, int64_t K, int8_t *q,
                            float *d256, int32_t *S32) {
    int64_t nsb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; r++) {
        float xf[256];
        for (int64_t sb = 0; sb < nsb; sb++) {
            for (int t = 0; t < 256; t++) xf[t] = load_x(x, x_dtype, r * K + 256 * sb + t);
            float amax = 0.0f;
            for (int t = 0; t < 256; t++) {
                float a = fabsf(xf[t]);
                if (a > amax) amax = a;
            }
            int8_t *qo = q + r * K + 256 * sb;
            int32_t *So = S32 + r * (K / 32) + 8 * sb;
            if (amax == 0.0f) {
                memset(qo, 0, 256);
                d256[r * nsb + sb] = 0.0f;
                for (int j = 0; j < 8; j++) So[j] = 0;
                continue;
            }
            float d = amax / 127.0f;
            float id = 1.0f / d;
            for (int j = 0; j < 8; j++) {
                int32_t S = 0;
                for (int t = 32 * j; t < 32 * j + 32; t++) {
                    int qi = 0;
                    if (xf[t] != 0.0f) {
                        float v = xf[t] * id;
                        float rr = rintf(v);
                        if (rr > 127.0f) rr = 127.0f;
                        if (rr < -127.0f) rr = -127.0f;
                        qi = (int)rr;
                    }
                    qo[t] = (int8_t)qi;
                    S += qi;
                }
                So[j] = S;
            }
            d256[r * nsb + sb] = d;
        }
    }
}

/* Q4_K GEMM with per-256 activation scales over the selected rows / columns
 * (all when rows / cols is NULL): exact int32 sub-block dots, fp64 combine in
 * ascending super-block and sub-block order.  Returns 0, or -1 on allocation
 * failure. */
int oracle_gemm_a256(const uint8_t *W, const void *x, int x_dtype, int64_t M, int64_t N, int64_t K,
                     const int64_t *rows, int64_t nrows, const int64_t *cols, int64_t ncols,
                     double *y) {
    if (!rows) nrows = M;
    if (!cols) ncols = N;
    int64_t nsb = K / 256, nb32 = K / 32;
    int8_t *qx = malloc((size_t)(nrows * K));
    float *dx = malloc(sizeof(float) * (size_t)(nrows * nsb));
    int32_t *Sx = malloc(sizeof(int32_t) * (size_t)(nrows * nb32));
    uint8_t *qw = malloc((size_t)(ncols * K));
    uint8_t *scw = malloc((size_t)(ncols * nb32)), *mw = malloc((size_t)(ncols * nb32));
    double *dw = malloc(sizeof(double) * (size_t)(ncols * nsb)), *dmw = malloc(sizeof(double) * (size_t)(ncols * nsb));
    float *xrow = malloc(sizeof(float) * (size_t)K);
    if (!qx || !dx || !Sx || !qw || !scw || !mw || !dw || !dmw || !xrow) {
        free(qx); free(dx); free(Sx); free(qw); free(scw); free(mw); free(dw); free(dmw); free(xrow);
        return -1;
    }
    free(xrow);
    for (int64_t i = 0; i < nrows; i++) {
        int64_t r = rows ? rows[i] : i;
        if (x_dtype == ORACLE_F32)
            oracle_quantize_act256((const float *)x + r * K, ORACLE_F32, 1, K, qx + i * K,
                                   dx + i * nsb, Sx + i * nb32);
        else
            oracle_quantize_act256((const uint16_t *)x + r * K, ORACLE_BF16, 1, K, qx + i * K,
                                   dx + i * nsb, Sx + i * nb32);
    }
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < ncols; j++) {
        int64_t n = cols ? cols[j] : j;
        for (int64_t sb = 0; sb < nsb; sb++)
            decode_q4k_block(W + (n * nsb + sb) * 144, qw + j * K + 256 * sb, scw + j * nb32 + 8 * sb,
                             mw + j * nb32 + 8 * sb, dw + j * nsb + sb, dmw + j * nsb + sb);
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < nrows; i++)
        for (int64_t j = 0; j < ncols; j++) {
            double acc = 0.0;
            for (int64_t sb = 0; sb < nsb; sb++) {
                double part = 0.0;
                for (int64_t b = 8 * sb; b < 8 * sb + 8; b++) {
                    int32_t I = 0;
                    for (int t = 0; t < 32; t++)
                        I += (int32_t)qw[j * K + 32 * b + t] * (int32_t)qx[i * K + 32 * b + t];
                    part += dw[j * nsb + sb] * (double)scw[j * nb32 + b] * (double)I -
                            dmw[j * nsb + sb] * (double)mw[j * nb32 + b] * (double)Sx[i * nb32 + b];
                }
                acc += (double)dx[i * nsb + sb] * part;
            }
            y[i * ncols + j] = acc;
        }
    free(qx); free(dx); free(Sx); free(qw); free(scw); free(mw); free(dw); free(dmw);
    return 0;
}

/* ============================================================================
 * Fusions on either side of the GEMM.  aprender issue #4220 ("CRUX parity
 * spike: apr serve vs ollama"), table of the techniques llama.cpp uses that
 * apr lacks: technique 2 counts a layer's per-token launches, among them its
 * norms and its swiglu as launches of their own; technique 6 is llama.cpp's
 * norm fused with the multiply by its weight.  sparkinfer PR #464, section
 * "Summary": the projection path's written-then-re-read scratch is the cost
 * its fused kernel removes.  The pages print neither formula; the readings
 * taken are the standard ones of the Qwen-family layers they discuss:
 *
 *   RMSNorm of a row x (length K) with the fp32 norm weight g and epsilon eps:
 *     ss  = sum_k x_k^2           binary64 (each x_k^2 is exact: x has at most
 *                                 24 significant bits)
 *     v   = ss / K + eps          binary64, correctly rounded steps
 *     r   = f32(1 / sqrt(v))      binary64 square root and division, rounded
 *                                 once to binary32
 *     xn_k = f32(f32(x_k * r) * g_k)
 *   and xn goes through the per-32 activation quantiser above.
 *
 *   SwiGLU on the gate and up projections of one FFN, stacked as the weight
 *   rows [gate (F rows); up (F rows)] of one matrix:
 *     h[m][f] = silu(y[m][f]) * y[m][F + f],   silu(z) = z / (1 + e^-z),
 *   evaluated here in binary64 from the oracle's fp64 GEMM output.
 * ========================================================================== */

/* Per row: r32 as above, and the interval [r32_lo, r32_hi] holding the r32 of
 * ANY summation order of ss.  Every order's binary64 sum of the K nonnegative
 * squares lies within (K-1)*2^-53/(1-(K-1)*2^-53) of the exact sum, so within
 * the band ss*(1 -+ delta), delta = 2*(K+1)*2^-53, around this one; r is a
 * monotone function of ss and so is every correctly rounded step, hence the
 * band's ends bound every order's r32. */
static float rms_r32(double ss, int64_t K, float eps) {
    double v = ss / (double)K + (double)eps;
    return (float)(1.0 / sqrt(v));
}

void oracle_rms_scale(const void *x, int x_dtype, int64_t M, int64_t K, float eps, float *r32,
                      float *r32_lo, float *r32_hi) {
    double delta = 2.0 * (double)(K + 1) * ldexp(1.0, -53);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; i++) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double xv = (double)load_x(x, x_dtype, i * K + k);
            ss += xv * xv;
        }
        r32[i] = rms_r32(ss, K, eps);
        float a = rms_r32(ss * (1.0 - delta), K, eps), b = rms_r32(ss * (1.0 + delta), K, eps);
        r32_lo[i] = a < b ? a : b;
        r32_hi[i] = a < b ? b : a;
    }
}

/* xn[i][k] = f32(f32(x[i][k] * r32[i]) * g[k]) */
void oracle_rmsnorm(const void *x, int x_dtype, const float *g, const float *r32, int64_t M,
                    int64_t K, float *xn) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; i++)
        for (int64_t k = 0; k < K; k++) {
            float t = load_x(x, x_dtype, i * K + k) * r32[i];
            xn[i * K + k] = t * g[k];
        }
}

/* h[i] = silu(gate[i]) * up[i] in binary64, silu(z) = z / (1 + exp(-z)). */
void oracle_swiglu(const double *gate, const double *up, int64_t n, double *h) {
    for (int64_t i = 0; i < n; i++) {
        double z = gate[i];
        double silu = z / (1.0 + exp(-z));
        h[i] = silu * up[i];
    }
}
