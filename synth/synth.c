/*
 * synth.c -- seeded synthetic inputs for the Q4_K / Q5_K / Q6_K x int8 prefill GEMM.
 *
 * This module only MAKES inputs.  It holds none of the GEMM's arithmetic
 * (no block decoding, no activation quantisation, no contraction).  Both the
 * CPU oracle and the GPU library consume the buffers it writes; neither links
 * this file.
 *
 * Random numbers: splitmix64 used as a counter-based generator.  The i-th
 * output of splitmix64 seeded with s is mix(s + (i+1)*0x9E3779B97F4A7C15),
 * where mix is the published splitmix64 finaliser (Steele, Lea, Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).  Element i
 * of a tensor always draws from counter i (two counters per normal draw), so
 * any slice can be regenerated on its own.
 *
 * Weight packing (float -> GGUF Q4_K / Q6_K blocks) is input generation: it
 * turns N(0, 0.02^2) draws into legal super-blocks, as the workloads on the
 * sparkinfer PR #464 page (fused Q4K/Q6K->int8 dequant, "Summary") and the
 * Qwen3.5 pages start from GGUF Q4_K_M files.  The rule is this module's own
 * simple min/max fit; any legal block is an equally valid GEMM input.
 *
 * Byte layouts written here (little-endian, binary16 scales):
 *   Q4_K, 144 B / 256 values: d, dmin (fp16) | 12 B packed 6-bit scales and
 *     mins | 128 B of 4-bit quants, value v in byte 32*(v/64) + v%32, low
 *     nibble when v%64 < 32, else high nibble.
 *   Q6_K, 210 B / 256 values: ql[128] low 4 bits | qh[64] high 2 bits |
 *     16 int8 scales (one per 16 values) | d (fp16).
 *   Q5_K, 176 B / 256 values: the Q4_K header | qh[32], bit v/32 of byte v%32
 *     the fifth bit of value v | 128 B of low 4 bits placed as Q4_K's.
 *   Q8_0, 34 B / 32 values: d (fp16) | 32 int8 codes.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* i-th splitmix64 output for seed s (i counts from 0). */
uint64_t synth_u64(uint64_t seed, uint64_t i) { return sm64_mix(seed + (i + 1) * GOLDEN); }

/* Uniform in the open interval (0, 1): 53 random bits, centred in their cell. */
static inline double unif(uint64_t seed, uint64_t i) {
    return ((double)(synth_u64(seed, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Standard normal for element i: Box-Muller on counters 2i and 2i+1. */
static inline double normal(uint64_t seed, uint64_t i) {
    double u1 = unif(seed, 2 * i), u2 = unif(seed, 2 * i + 1);
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

void synth_uniform_f64(uint64_t seed, int64_t n, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = unif(seed, (uint64_t)i);
}

/* out[i] = mean + std * N(0,1), element i on counters 2i, 2i+1. */
void synth_normal_f32(uint64_t seed, int64_t n, double mean, double std, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (float)(mean + std * normal(seed, (uint64_t)i));
}

/* Multiply element i by `factor` when uniform(mask_seed, i) < prob. */
void synth_outliers_f32(uint64_t mask_seed, int64_t n, double prob, double factor, float *x) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        if (unif(mask_seed, (uint64_t)i) < prob) x[i] = (float)((double)x[i] * factor);
}

/* Student-t with 4 degrees of freedom: Z / sqrt(chi2_4 / 4), chi2_4 the sum of
 * four squared normals.  Z uses seed, the chi-square normals seed+1..seed+4. */
void synth_student_t4_f32(uint64_t seed, int64_t n, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        double z = normal(seed, (uint64_t)i), c = 0.0;
        for (int j = 1; j <= 4; j++) {
            double g = normal(seed + (uint64_t)j, (uint64_t)i);
            c += g * g;
        }
        out[i] = (float)(z / sqrt(c / 4.0));
    }
}

/* RMS-normalise every row of x [rows x cols] in place (unit gain):
 * x / sqrt(mean(x^2) + eps), in double, rounded once to float. */
void synth_rmsnorm_rows_f32(float *x, int64_t rows, int64_t cols, double eps) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float *p = x + r * cols;
        double ss = 0.0;
        for (int64_t c = 0; c < cols; c++) ss += (double)p[c] * (double)p[c];
        double inv = 1.0 / sqrt(ss / (double)cols + eps);
        for (int64_t c = 0; c < cols; c++) p[c] = (float)((double)p[c] * inv);
    }
}

/* float -> bfloat16 bits, round to nearest even (finite inputs). */
void synth_f32_to_bf16(const float *in, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        uint32_t u;
        memcpy(&u, &in[i], 4);
        uint32_t r = 0x7FFFu + ((u >> 16) & 1u);
        out[i] = (uint16_t)((u + r) >> 16);
    }
}

/* ---------- binary16 helpers for the packer ---------- */

/* double -> binary16 bits, round to nearest even; finite, non-negative inputs
 * below 65520 (the packer only produces such scales). */
static uint16_t to_half(double v) {
    if (v <= 0.0) return 0;
    int e;
    double m = frexp(v, &e); /* v = m * 2^e, m in [0.5, 1) */
    /* binary16 normal: v = (1 + f/1024) * 2^(E-15), E in 1..30 */
    int E = e - 1 + 15;
    if (E >= 1) {
        double f = (2.0 * m - 1.0) * 1024.0; /* in [0, 1024) */
        double r = nearbyint(f);             /* ties-to-even under the default mode */
        int fi = (int)r;
        if (fi == 1024) { fi = 0; E += 1; }
        if (E >= 31) return 0x7BFF; /* clamp to max finite (not reached by the packer) */
        return (uint16_t)((E << 10) | fi);
    }
    /* subnormal: v = f * 2^-24 */
    double f = nearbyint(ldexp(v, 24));
    int fi = (int)f;
    if (fi >= 1024) return (uint16_t)(1 << 10); /* rounds up to min normal */
    return (uint16_t)fi;
}

static double from_half(uint16_t h) {
    int E = (h >> 10) & 31, f = h & 1023;
    double v = (E == 0) ? ldexp((double)f, -24) : ldexp(1024.0 + (double)f, E - 25);
    return (h & 0x8000) ? -v : v;
}

static inline int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

/* ---------- packers ---------- */

/* Pack w [N x K] (K % 256 == 0) into Q4_K (q5 = 0) or Q5_K (q5 = 1)
 * super-blocks, row n = K/256 blocks.  Both share the header; Q5_K codes take
 * 32 levels, their fifth bit going to qh (bit v/32 of byte v%32). */
static void pack_k(const float *w, int64_t N, int64_t K, uint8_t *out, int q5) {
    const int bytes = q5 ? 176 : 144, qmax = q5 ? 31 : 15;
    int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < N * nb; blk++) {
        const float *x = w + blk * 256; /* rows are contiguous, so block blk is w[256*blk..] */
        uint8_t *o = out + blk * bytes;
        double scale[8], mn[8];
        double smax = 0.0, mmax = 0.0;
        for (int j = 0; j < 8; j++) {
            double lo = 0.0, hi = -INFINITY;
            for (int t = 0; t < 32; t++) {
                double v = x[32 * j + t];
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            scale[j] = (hi - lo) / qmax;
            mn[j] = -lo;
            if (scale[j] > smax) smax = scale[j];
            if (mn[j] > mmax) mmax = mn[j];
        }
        uint16_t hd = to_half(smax / 63.0), hm = to_half(mmax / 63.0);
        double d = from_half(hd), dmin = from_half(hm);
        int sc[8], m[8];
        for (int j = 0; j < 8; j++) {
            sc[j] = d > 0.0 ? clampi((int)nearbyint(scale[j] / d), 0, 63) : 0;
            m[j] = dmin > 0.0 ? clampi((int)nearbyint(mn[j] / dmin), 0, 63) : 0;
        }
        memset(o, 0, (size_t)bytes);
        o[0] = (uint8_t)(hd & 0xFF); o[1] = (uint8_t)(hd >> 8);
        o[2] = (uint8_t)(hm & 0xFF); o[3] = (uint8_t)(hm >> 8);
        uint8_t *s = o + 4;
        for (int j = 0; j < 4; j++) {
            s[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
            s[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
            s[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
        }
        uint8_t *qh = o + 16, *qs = o + (q5 ? 48 : 16);
        for (int v = 0; v < 256; v++) {
            int j = v / 32;
            double step = d * sc[j];
            int q = step > 0.0 ? clampi((int)nearbyint(((double)x[v] + dmin * m[j]) / step), 0, qmax) : 0;
            int byte = 32 * (v / 64) + (v % 32);
            if ((v % 64) < 32) qs[byte] |= (uint8_t)(q & 15);
            else qs[byte] |= (uint8_t)((q & 15) << 4);
            if (q5) qh[v % 32] |= (uint8_t)(((q >> 4) & 1) << (v / 32));
        }
    }
}

void synth_pack_q4k(const float *w, int64_t N, int64_t K, uint8_t *out) { pack_k(w, N, K, out, 0); }
void synth_pack_q5k(const float *w, int64_t N, int64_t K, uint8_t *out) { pack_k(w, N, K, out, 1); }

/* Pack w [N x K] into Q6_K super-blocks. */
void synth_pack_q6k(const float *w, int64_t N, int64_t K, uint8_t *out) {
    int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < N * nb; blk++) {
        const float *x = w + blk * 256;
        uint8_t *o = out + blk * 210;
        double scale[16], smax = 0.0;
        for (int s = 0; s < 16; s++) {
            double a = 0.0;
            for (int t = 0; t < 16; t++) {
                double v = fabs((double)x[16 * s + t]);
                if (v > a) a = v;
            }
            scale[s] = a / 31.0;
            if (scale[s] > smax) smax = scale[s];
        }
        uint16_t hd = to_half(smax / 127.0);
        double d = from_half(hd);
        int sc[16];
        for (int s = 0; s < 16; s++) sc[s] = d > 0.0 ? clampi((int)nearbyint(scale[s] / d), -128, 127) : 0;
        memset(o, 0, 210);
        uint8_t *ql = o, *qh = o + 128;
        for (int v = 0; v < 256; v++) {
            int s = v / 16;
            double step = d * sc[s];
            int q = step != 0.0 ? clampi((int)nearbyint((double)x[v] / step), -32, 31) + 32 : 32;
            int h = v / 128, r = v % 128, c = r / 32, l = r % 32;
            int lb = 64 * h + 32 * (c % 2) + l;
            if (c < 2) ql[lb] |= (uint8_t)(q & 15);
            else ql[lb] |= (uint8_t)((q & 15) << 4);
            qh[32 * h + l] |= (uint8_t)(((q >> 4) & 3) << (2 * c));
        }
        for (int s = 0; s < 16; s++) o[192 + s] = (uint8_t)(int8_t)sc[s];
        o[208] = (uint8_t)(hd & 0xFF); o[209] = (uint8_t)(hd >> 8);
    }
}

/* Pack w [N x K] (K % 32 == 0) into Q8_0 blocks: per 32 values d = f16(amax/127),
 * q = clamp(rint(w / d), -127, 127). */
void synth_pack_q80(const float *w, int64_t N, int64_t K, uint8_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < N * (K / 32); blk++) {
        const float *x = w + blk * 32;
        uint8_t *o = out + blk * 34;
        double amax = 0.0;
        for (int t = 0; t < 32; t++) if (fabs((double)x[t]) > amax) amax = fabs((double)x[t]);
        uint16_t hd = to_half(amax / 127.0);
        double d = from_half(hd);
        o[0] = (uint8_t)(hd & 0xFF); o[1] = (uint8_t)(hd >> 8);
        for (int t = 0; t < 32; t++)
            o[2 + t] = (uint8_t)(int8_t)(d > 0.0 ? clampi((int)nearbyint((double)x[t] / d), -127, 127) : 0);
    }
}

/* Random legal blocks: every byte random except the binary16 scale fields,
 * which get a random sign, a random mantissa and an exponent field drawn from
 * [emin, emax] (0 = subnormal) so that d and dmin are always finite.  fmt 0 =
 * Q4_K, 1 = Q6_K, 2 = Q5_K, 3 = Q8_0 (a block = 256 values: eight 34-byte Q8_0
 * blocks).  Block b uses counters 256*b .. 256*b+255. */
void synth_random_blocks(uint64_t seed, int fmt, int64_t nblocks, int emin, int emax,
                         int allow_negative, uint8_t *out) {
    int bytes = fmt == 0 ? 144 : fmt == 2 ? 176 : fmt == 3 ? 272 : 210;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblocks; b++) {
        uint8_t *o = out + b * bytes;
        for (int i = 0; i < bytes; i++) o[i] = (uint8_t)(synth_u64(seed, (uint64_t)(256 * b + i)) >> 56);
        int nscale = fmt == 1 ? 1 : fmt == 3 ? 8 : 2;
        for (int k = 0; k < nscale; k++) {
            uint64_t r = synth_u64(seed, (uint64_t)(256 * b + 240 + k));
            int E = emin + (int)((r >> 32) % (uint64_t)(emax - emin + 1));
            uint16_t h = (uint16_t)((E << 10) | (int)(r & 1023));
            if (allow_negative && ((r >> 20) & 1)) h |= 0x8000;
            int off = fmt == 1 ? 208 : fmt == 3 ? 34 * k : 2 * k;
            o[off] = (uint8_t)(h & 0xFF);
            o[off + 1] = (uint8_t)(h >> 8);
        }
    }
}
