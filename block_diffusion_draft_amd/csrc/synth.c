/*
 * Seeded synthetic inputs and the host-side Q4_K packer.
 *
 * This file generates data only.  It is not part of the draft step: the GPU
 * path never quantises, and the reference checker decodes Q4_K on its own.
 *
 *   - Random numbers come from a counter-based generator: value #i of a stream
 *     is a pure function of (seed, stream, i), so any slice of any tensor can be
 *     regenerated independently and in parallel.  The 64-bit mixer is Vigna's
 *     SplitMix64 finaliser; normals use the Box-Muller transform on a pair of
 *     53-bit uniforms.
 *   - The Q4_K packer writes 144-byte super-blocks of 256 weights: fp16 d and
 *     dmin, twelve bytes of 6-bit sub-block scales and mins, 128 bytes of 4-bit
 *     quants (low nibbles = first 32 weights of each 64-weight chunk, high
 *     nibbles = the next 32).  Per sub-block it fits (scale, min) with the min
 *     clamped at or below zero, refines them by least squares on the chosen
 *     codes, then quantises scales and mins to 6 bits against fp16 super-block
 *     factors.
 *   - The Q8_0 and FP8 (E4M3, one scale per row) packers quantise the same normals
 *     (see their sections below).
 *
 * Built with gcc -O3 -fopenmp into libdflash_synth.so and called through ctypes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t mix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
    return mix64(seed ^ mix64(stream ^ 0xD1B54A32D192ED03ull));
}

/* normals 2p and 2p+1 of a stream */
static inline void normal_pair(uint64_t key, uint64_t p, double *z0, double *z1) {
    uint64_t a = mix64(key + 2 * p), b = mix64(key + 2 * p + 1);
    double u1 = ((double)(a >> 11) + 0.5) * 0x1.0p-53;   /* (0, 1) */
    double u2 = (double)(b >> 11) * 0x1.0p-53;           /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925 * u2;
    *z0 = r * cos(th);
    *z1 = r * sin(th);
}

static inline double normal_at(uint64_t key, uint64_t i) {
    double z0, z1;
    normal_pair(key, i >> 1, &z0, &z1);
    return (i & 1) ? z1 : z0;
}

static inline uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* float -> IEEE half, round to nearest even, subnormals included */
static uint16_t f32_to_f16(float f) {
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (a < 0x1p-14) return sign | (uint16_t)nearbyint(a * 0x1p24);
    int e;
    double m = frexp(a, &e);          /* a = m 2^e, m in [0.5, 1) */
    double q = nearbyint(m * 2048.0); /* 11 significant bits */
    if (q == 2048.0) { q = 1024.0; e += 1; }
    int E = e - 1 + 15;
    if (E >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(E << 10) | (uint16_t)((int)q - 1024);
}

static double f16_to_f64(uint16_t h) {
    int E = (h >> 10) & 31, M = h & 1023;
    double v = E == 0 ? M * 0x1p-24 : ldexp(1024.0 + M, E - 25);
    return (h & 0x8000) ? -v : v;
}

void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                      float std, float *out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = (float)(std * normal_at(key, offset + (uint64_t)i));
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                       float std, uint16_t *out) {
    uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = f32_to_bf16((float)(std * normal_at(key, offset + (uint64_t)i)));
}

/* uniform integers in [lo, hi) */
void synth_randint(uint64_t seed, uint64_t stream, int64_t n, int32_t lo, int32_t hi,
                   int32_t *out) {
    uint64_t key = stream_key(seed, stream);
    double span = (double)hi - (double)lo;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        double u = (double)(mix64(key + (uint64_t)i) >> 11) * 0x1.0p-53;
        int64_t v = lo + (int64_t)floor(u * span);
        if (v >= hi) v = hi - 1;
        out[i] = (int32_t)v;
    }
}

/* ---------------------------------------------------------------- Q4_K */

static void fit_subblock(const float *x, double *scale, double *minv) {
    double lo = 0.0, hi = -INFINITY;
    for (int i = 0; i < 32; i++) {
        if (x[i] < lo) lo = x[i];
        if (x[i] > hi) hi = x[i];
    }
    if (hi < lo) hi = lo;
    double s = (hi - lo) / 15.0, mn = -lo;   /* w ~ s q - mn, mn >= 0 */
    for (int it = 0; it < 3 && s > 0; it++) {
        double sq = 0, sq2 = 0, sx = 0, sqx = 0;
        for (int i = 0; i < 32; i++) {
            double q = nearbyint((x[i] + mn) / s);
            if (q < 0) q = 0;
            if (q > 15) q = 15;
            sq += q; sq2 += q * q; sx += x[i]; sqx += q * x[i];
        }
        double den = 32.0 * sq2 - sq * sq;
        if (den <= 0) break;
        double ns = (32.0 * sqx - sq * sx) / den;
        double off = (sx - ns * sq) / 32.0;           /* x ~ ns q + off */
        if (off > 0) {                                /* min must stay <= 0 */
            off = 0;
            ns = sq2 > 0 ? sqx / sq2 : 0;
        }
        if (!(ns > 0)) break;
        s = ns;
        mn = -off;
    }
    *scale = s > 0 ? s : 0;
    *minv = mn > 0 ? mn : 0;
}

static void pack_superblock(const float *x, uint8_t *blk) {
    double sc_f[8], mn_f[8], smax = 0, mmax = 0;
    for (int j = 0; j < 8; j++) {
        fit_subblock(x + 32 * j, &sc_f[j], &mn_f[j]);
        if (sc_f[j] > smax) smax = sc_f[j];
        if (mn_f[j] > mmax) mmax = mn_f[j];
    }
    uint16_t dh = f32_to_f16((float)(smax / 63.0));
    uint16_t mh = f32_to_f16((float)(mmax / 63.0));
    double d = f16_to_f64(dh), dmin = f16_to_f64(mh);
    int sc[8], m[8];
    for (int j = 0; j < 8; j++) {
        double a = d > 0 ? nearbyint(sc_f[j] / d) : 0;
        double b = dmin > 0 ? nearbyint(mn_f[j] / dmin) : 0;
        sc[j] = a < 0 ? 0 : (a > 63 ? 63 : (int)a);
        m[j] = b < 0 ? 0 : (b > 63 ? 63 : (int)b);
    }
    memcpy(blk + 0, &dh, 2);
    memcpy(blk + 2, &mh, 2);
    uint8_t *s = blk + 4;
    for (int j = 0; j < 4; j++) {
        s[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        s[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
        s[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
    }
    uint8_t q[256];
    for (int i = 0; i < 256; i++) {
        int j = i / 32;
        double step = d * sc[j];
        double v = step > 0 ? nearbyint((x[i] + dmin * m[j]) / step) : 0;
        q[i] = (uint8_t)(v < 0 ? 0 : (v > 15 ? 15 : v));
    }
    uint8_t *qs = blk + 16;
    for (int c = 0; c < 4; c++)
        for (int i = 0; i < 32; i++)
            qs[32 * c + i] = (uint8_t)(q[64 * c + i] | (q[64 * c + 32 + i] << 4));
}

/* w [rows][cols] float32, cols % 256 == 0 -> out [rows][cols/256][144] */
void synth_q4k_pack(const float *w, int64_t rows, int64_t cols, uint8_t *out) {
    int64_t nb = cols / 256;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++)
            pack_superblock(w + r * cols + b * 256, out + (r * nb + b) * 144);
}

/* Q4_K blocks of a [rows, cols] matrix whose weights are std * N(0,1) of the
 * stream, element (r, c) = normal #(r*cols + c).  Nothing float-sized is stored. */
void synth_q4k_normal(uint64_t seed, uint64_t stream, int64_t rows, int64_t cols, float std,
                      uint8_t *out) {
    uint64_t key = stream_key(seed, stream);
    int64_t nb = cols / 256;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float x[256];
        for (int64_t b = 0; b < nb; b++) {
            uint64_t base = (uint64_t)(r * cols + b * 256);
            for (int i = 0; i < 256; i += 2) {
                double z0, z1;
                normal_pair(key, (base + (uint64_t)i) >> 1, &z0, &z1);
                x[i] = (float)(std * z0);
                x[i + 1] = (float)(std * z1);
            }
            pack_superblock(x, out + (r * nb + b) * 144);
        }
    }
}

/* ---------------------------------------------------------------- Q8_0
 * 34-byte blocks of 32 weights along a row: fp16 scale d (little endian), then 32
 * signed bytes q; w = d q.  Host-side quantizer (a data generator, not part of the
 * draft path): d = max |x| / 127 rounded to fp16, q = x / d rounded to nearest
 * (halves away from zero) and clamped to [-127, 127]; an all-zero block stores d = 0. */
static void pack_q8_0_block(const float *x, uint8_t *blk) {
    double amax = 0.0;
    for (int i = 0; i < 32; i++) amax = fmax(amax, fabs((double)x[i]));
    uint16_t dh = f32_to_f16((float)(amax / 127.0));
    double d = f16_to_f64(dh);
    blk[0] = (uint8_t)(dh & 0xFF);
    blk[1] = (uint8_t)(dh >> 8);
    for (int i = 0; i < 32; i++) {
        double q = d > 0.0 ? round((double)x[i] / d) : 0.0;
        if (q > 127.0) q = 127.0;
        if (q < -127.0) q = -127.0;
        blk[2 + i] = (uint8_t)(int8_t)q;
    }
}

/* w [rows][cols] float32, cols % 32 == 0 -> out [rows][cols/32][34] */
void synth_q8_0_pack(const float *w, int64_t rows, int64_t cols, uint8_t *out) {
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++)
            pack_q8_0_block(w + r * cols + b * 32, out + (r * nb + b) * 34);
}

/* Q8_0 blocks of a [rows, cols] matrix of std * N(0,1) weights of the stream, element
 * (r, c) = normal #(r*cols + c) (the same values synth_q4k_normal quantizes). */
void synth_q8_0_normal(uint64_t seed, uint64_t stream, int64_t rows, int64_t cols, float std,
                       uint8_t *out) {
    uint64_t key = stream_key(seed, stream);
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float x[32];
        for (int64_t b = 0; b < nb; b++) {
            uint64_t base = (uint64_t)(r * cols + b * 32);
            for (int i = 0; i < 32; i += 2) {
                double z0, z1;
                normal_pair(key, (base + (uint64_t)i) >> 1, &z0, &z1);
                x[i] = (float)(std * z0);
                x[i + 1] = (float)(std * z1);
            }
            pack_q8_0_block(x, out + (r * nb + b) * 34);
        }
    }
}

/* ---------------------------------------------------------------- FP8 (E4M3)
 * One code per weight (sign, 4 exponent bits of bias 7, 3 mantissa bits; largest
 * finite 448) and one float32 scale per row: w = s code.  Host-side quantizer (a data
 * generator, not part of the draft path): s = max |x| / 448 of the row (1 for an
 * all-zero row), code = x / s rounded to the nearest E4M3 value, ties to the even
 * mantissa.  Output: the rows' codes, then the rows' scales (little endian). */
static uint8_t f64_to_e4m3(double v) {
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    if (a < 0x1p-6) return sign | (uint8_t)nearbyint(a * 0x1p9);   /* 8 -> code 0x08 */
    int e;
    double m = frexp(a, &e);          /* a = m 2^e, m in [0.5, 1) */
    double q = nearbyint(m * 16.0);   /* 4 significant bits */
    if (q == 16.0) { q = 8.0; e += 1; }
    int E = e - 1 + 7;
    int code = (E << 3) | ((int)q - 8);
    if (code > 0x7E) code = 0x7E;
    return sign | (uint8_t)code;
}

static void pack_fp8_row(const float *x, int64_t cols, uint8_t *codes, float *scale) {
    double amax = 0.0;
    for (int64_t i = 0; i < cols; i++) amax = fmax(amax, fabs((double)x[i]));
    float s = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
    *scale = s;
    for (int64_t i = 0; i < cols; i++) codes[i] = f64_to_e4m3((double)x[i] / (double)s);
}

/* w [rows][cols] float32 -> out: rows * cols codes, then rows float32 scales */
void synth_fp8_pack(const float *w, int64_t rows, int64_t cols, uint8_t *out) {
    float *sc = (float *)(out + rows * cols);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float s;
        pack_fp8_row(w + r * cols, cols, out + r * cols, &s);
        memcpy(sc + r, &s, 4);
    }
}

/* FP8 bytes of a [rows, cols] matrix of std * N(0,1) weights of the stream, element
 * (r, c) = normal #(r*cols + c) (the same values the Q4_K and Q8_0 packers quantise). */
void synth_fp8_normal(uint64_t seed, uint64_t stream, int64_t rows, int64_t cols, float std,
                      uint8_t *out) {
    uint64_t key = stream_key(seed, stream);
    float *sc = (float *)(out + rows * cols);
#pragma omp parallel
    {
        float *x = (float *)malloc((size_t)cols * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; r++) {
            uint64_t base = (uint64_t)(r * cols);
            for (int64_t i = 0; i < cols; i += 2) {
                double z0, z1;
                normal_pair(key, (base + (uint64_t)i) >> 1, &z0, &z1);
                x[i] = (float)(std * z0);
                x[i + 1] = (float)(std * z1);
            }
            float s;
            pack_fp8_row(x, cols, out + r * cols, &s);
            memcpy(sc + r, &s, 4);
        }
        free(x);
    }
}
