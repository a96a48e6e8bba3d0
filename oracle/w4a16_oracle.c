/*
 * w4a16_oracle.c -- plain, slow CPU definition of the W4A16 weight format and matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only the tests,
 * the smoke check and the benchmark's CPU-baseline leg load it.  It shares no code, header,
 * table or constant with the HIP library and includes nothing from it.
 *
 * Sources (the pages' own words are restated, never quoted):
 *  [P1] vidyal.ai, "Low-Precision Kernels: INT4, INT8 and FP8 Matmuls, Measured",
 *       section "Step 2: a W4A16 kernel in Triton" -- group of 128 along K, scale =
 *       (max - min)/15, code = round((w - min)/scale) in 0..15, eight codes per 32-bit word
 *       along K (row 8r+j of the unpacked tile is nibble j of packed row r), a K/8 x N packed
 *       matrix plus K/128 x N bf16 scales and minimums, dequant q*s + min in fp32 rounded to
 *       bf16; the FP64 product with the same 4-bit weights as accuracy reference.
 *  [P2] thuongvuho.com, "Why My 4-Bit CUDA Kernel Wasn't Faster", sections "Why fewer bytes
 *       should have helped" and "Loading the same bytes differently" -- Q4 blocks of 32
 *       weights: 16 code bytes plus one fp16 scale; decode = (code - bias) * scale; the low
 *       nibble of code byte j multiplies x[2j], the high nibble x[2j+1].
 *  [P3] anrans.github.io, "Quantization and GEMV", sections "The quantization formulas" and
 *       "W4A16: dequantizing in registers" -- first element in the low 4 bits of a word,
 *       extraction (word >> 4i) & 0xF, a zero range gives scale 1, FP64 reference sums; and the
 *       integer-zero-point format: s = (max - min)/15, z = round(-min/s),
 *       q = clamp(round(w/s) + z, 0, 15), w_hat = (q - z) * s, words [N][K/8] (a row's words
 *       along K), scales and zero points [N][K/128]; and, from its first exercise, W8A16:
 *       per row s = max|w| / 127, q = clamp(round(w/s), -127, 127) stored as int8 [N][K],
 *       the row's scale applied once after the row's sum.
 *  [P1'] vidyal.ai, "Low-Precision Kernels", sections "INT8 on a GeForce chip" and "The cost of
 *       quantizing activations" -- W4A8: the activations quantized to 8-bit integers per row on
 *       every call (absolute value, maximum per row, divide, round, convert), integer products
 *       summed in 32 bits, and the activation and weight scales applied to those sums in the
 *       epilogue.
 *
 * Readings where the pages leave a step open (each is listed in the design notes):
 *  - codes are computed from the STORED (rounded) scale and minimum, so encode and decode
 *    agree; the clamp to 0..15 guards the rounding of both ends;
 *  - "round" is round-half-to-even (rintf); division is IEEE fp32 division, correctly rounded;
 *  - a group whose max equals its min gets scale 1.0 (as [P3] does); a zero min/max is +0;
 *  - dequant uses one fused multiply-add in fp32, then bf16 round-to-nearest-even;
 *  - Q4: bias 8 and scale max|w|/7 rounded to fp16 (a zero block gets scale 1.0);
 *  - Q4 storage is two arrays: codes [N][K/32][16] bytes and scales [N][K/32] fp16;
 *  - the matmul reference is the fp64 sum, in k order, of x times the exactly dequantized
 *    weight q*s + min (or (q - 8)*s), which fp64 holds without rounding at these magnitudes;
 *  - zero-point format: scale and zero point are stored as fp16 (the page keeps the zero point
 *    "as fp16" as one of its options); codes use the stored scale and zero point; "round" is the
 *    page's std::round, half away from zero (roundf), for both z and the codes; z is clamped to
 *    [-2048, 2048], the integers fp16 holds exactly (only a group whose range is below 1/2048 of
 *    its distance from zero reaches the clamp); the code is round(w/s) + z as the formula
 *    writes it (the page's example rounds w/s + z, which differs only at exact ties).
 *  - W4A8 activations: symmetric per row, a = max|x| / 127 in fp32 (IEEE division), an all-zero
 *    row gets a = 1, xq = clamp(rint(x / a), -127, 127) with ties to even; the weights are the
 *    G128 format unchanged.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math -lm
 * Every function returns 0 on success and a nonzero code on a bad argument or a
 * non-finite input; nothing is allocated.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NONFINITE 2

/* ------------------------------------------------------------------------------------------
 * Number formats, written out from the IEEE-754 definitions.
 * bfloat16: sign, the 8-bit float32 exponent, 7 fraction bits (the top half of a float32).
 * binary16: sign, 5-bit exponent (bias 15), 10 fraction bits, subnormals below 2^-14.
 * Rounding is to nearest, ties to even: scale by a power of two so that the last kept bit
 * has weight 1, round to the nearest integer with nearbyint (ties to even in the default
 * rounding mode), scale back.  All of this is exact in double.
 * ---------------------------------------------------------------------------------------- */

static int floor_log2(double a) /* a > 0, finite */
{
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    return e - 1;
}

uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(f)) return (uint16_t)(sign | 0x7F80u);
    if (f == 0.0f) return sign;
    const double a = fabs((double)f);
    int e = floor_log2(a);
    if (e < -126) e = -126;                 /* subnormal range: fixed quantum 2^-133 */
    const double quantum = ldexp(1.0, e - 7); /* 8 significant bits */
    const double r = nearbyint(a / quantum) * quantum;
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u); /* overflow to infinity */
    const float rf = (float)r;               /* exact: at most 8 significant bits */
    uint32_t v;
    memcpy(&v, &rf, 4);
    return (uint16_t)(sign | (v >> 16));
}

float oracle_bf16_to_f32(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t oracle_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
    if (f == 0.0f) return sign;
    const double a = fabs((double)f);
    int e = floor_log2(a);
    if (e < -14) e = -14;                      /* subnormal range: fixed quantum 2^-24 */
    const double quantum = ldexp(1.0, e - 10); /* 11 significant bits */
    const double r = nearbyint(a / quantum) * quantum;
    if (r >= 65536.0) return (uint16_t)(sign | 0x7C00u); /* past 65504: infinity */
    if (r == 0.0) return sign;
    const int re = floor_log2(r);
    if (re < -14) /* subnormal: value = frac * 2^-24 */
        return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    const uint16_t frac = (uint16_t)((ldexp(r, -re) - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)((re + 15) << 10) | frac);
}

double oracle_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 31;
    const int frac = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)frac, -24);
    else if (e == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp(1.0 + frac / 1024.0, e - 15);
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------------------------
 * Nibble packing [P1 Step 2; P3 "W4A16: dequantizing in registers"]: element j of a run of
 * eight sits in bits 4j..4j+3 of the 32-bit word, the first element lowest.
 * ---------------------------------------------------------------------------------------- */

uint32_t oracle_pack_word(const uint8_t q[8])
{
    uint32_t w = 0;
    for (int j = 0; j < 8; ++j) w |= (uint32_t)(q[j] & 0xF) << (4 * j);
    return w;
}

void oracle_unpack_word(uint32_t w, uint8_t q[8])
{
    for (int j = 0; j < 8; ++j) q[j] = (uint8_t)((w >> (4 * j)) & 0xFu);
}

/* ------------------------------------------------------------------------------------------
 * Format G128 [P1 Step 2]: asymmetric, groups of 128 consecutive k, bf16 scale and minimum.
 *   W      fp32 [N][K] row-major (N outputs, K inputs), K % 128 == 0
 *   codes  uint32 [K/8][N]   word (r, n) holds k = 8r..8r+7 of column n, k = 8r lowest
 *   scales bf16 bits [K/128][N], mins bf16 bits [K/128][N]
 * For every (n, g):
 *   lo, hi = min, max of W[n][128g .. 128g+127]              (a zero is taken as +0)
 *   s = (hi - lo) / 15 in fp32;  s_b = bf16(s), or 1.0 if that is zero;  m_b = bf16(lo)
 *   q = clamp(rint((w - m_b) / s_b), 0, 15)                  (fp32 subtract and divide)
 * ---------------------------------------------------------------------------------------- */

int oracle_quantize_g128(const float* W, int64_t N, int64_t K, uint32_t* codes, uint16_t* scales,
                         uint16_t* mins)
{
    if (!W || !codes || !scales || !mins || N <= 0 || K <= 0 || K % 128) return ORACLE_BAD_ARG;
    const int64_t G = K / 128;
    for (int64_t i = 0; i < (K / 8) * N; ++i) codes[i] = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float* w = W + n * K + g * 128;
            float lo = w[0], hi = w[0];
            for (int j = 0; j < 128; ++j) {
                if (!isfinite(w[j])) return ORACLE_NONFINITE;
                if (w[j] < lo) lo = w[j];
                if (w[j] > hi) hi = w[j];
            }
            if (lo == 0.0f) lo = 0.0f; /* -0 becomes +0 */
            if (hi == 0.0f) hi = 0.0f;
            const float s = (hi - lo) / 15.0f;
            uint16_t s_b = oracle_f32_to_bf16(s);
            if (oracle_bf16_to_f32(s_b) == 0.0f) s_b = 0x3F80; /* 1.0 */
            const uint16_t m_b = oracle_f32_to_bf16(lo);
            if (!isfinite(oracle_bf16_to_f32(s_b)) || !isfinite(oracle_bf16_to_f32(m_b)))
                return ORACLE_NONFINITE;
            scales[g * N + n] = s_b;
            mins[g * N + n] = m_b;
            const float sf = oracle_bf16_to_f32(s_b), mf = oracle_bf16_to_f32(m_b);
            for (int j = 0; j < 128; ++j) {
                const float t = rintf((w[j] - mf) / sf);
                const int q = t < 0.0f ? 0 : (t > 15.0f ? 15 : (int)t);
                const int64_t k = g * 128 + j;
                codes[(k / 8) * N + n] |= (uint32_t)q << (4 * (k % 8));
            }
        }
    }
    return ORACLE_OK;
}

static int g128_code(const uint32_t* codes, int64_t N, int64_t n, int64_t k)
{
    uint8_t q[8];
    oracle_unpack_word(codes[(k / 8) * N + n], q);
    return q[k % 8];
}

/* Dequantized weight, three ways:
 *   kind 0: fp32 fmaf(q, s_b, m_b)                            -> float  [N][K]
 *   kind 1: bf16 round-to-nearest-even of kind 0              -> uint16 [N][K]
 *   kind 2: fp64 q*s_b + m_b, exact at these magnitudes       -> double [N][K]   */
int oracle_dequant_g128(const uint32_t* codes, const uint16_t* scales, const uint16_t* mins,
                        int64_t N, int64_t K, int kind, void* out)
{
    if (!codes || !scales || !mins || !out || N <= 0 || K <= 0 || K % 128 || kind < 0 || kind > 2)
        return ORACLE_BAD_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const int q = g128_code(codes, N, n, k);
            const uint16_t s_b = scales[(k / 128) * N + n], m_b = mins[(k / 128) * N + n];
            const float s = oracle_bf16_to_f32(s_b), m = oracle_bf16_to_f32(m_b);
            if (kind == 0)
                ((float*)out)[n * K + k] = fmaf((float)q, s, m);
            else if (kind == 1)
                ((uint16_t*)out)[n * K + k] = oracle_f32_to_bf16(fmaf((float)q, s, m));
            else
                ((double*)out)[n * K + k] = (double)q * (double)s + (double)m;
        }
    return ORACLE_OK;
}

static double g128_weight_exact(const uint32_t* codes, const uint16_t* scales, const uint16_t* mins,
                                int64_t N, int64_t n, int64_t k)
{
    const int q = g128_code(codes, N, n, k);
    return (double)q * (double)oracle_bf16_to_f32(scales[(k / 128) * N + n]) +
           (double)oracle_bf16_to_f32(mins[(k / 128) * N + n]);
}

/* ------------------------------------------------------------------------------------------
 * Format Q4B32 [P2]: symmetric blocks of 32 along k with an fp16 scale and a bias of 8.
 *   codes  uint8 [N][K/32][16]: byte j of block b holds the code of k = 32b+2j in its low
 *          nibble and of k = 32b+2j+1 in its high nibble
 *   scales fp16 bits [N][K/32]
 * For every (n, b):  a = max |w|;  s = a / 7 in fp32;  s_h = fp16(s), or 1.0 if zero;
 *   q = clamp(rint(w / s_h) + 8, 0, 15);  decode (q - 8) * s_h (exact in fp32).
 * ---------------------------------------------------------------------------------------- */

int oracle_quantize_q4b32(const float* W, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales)
{
    if (!W || !codes || !scales || N <= 0 || K <= 0 || K % 32) return ORACLE_BAD_ARG;
    const int64_t B = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < B; ++b) {
            const float* w = W + n * K + b * 32;
            float a = 0.0f;
            for (int j = 0; j < 32; ++j) {
                if (!isfinite(w[j])) return ORACLE_NONFINITE;
                if (fabsf(w[j]) > a) a = fabsf(w[j]);
            }
            const float s = a / 7.0f;
            uint16_t s_h = oracle_f32_to_f16(s);
            if (oracle_f16_to_f64(s_h) == 0.0) s_h = 0x3C00; /* 1.0 */
            if (!isfinite(oracle_f16_to_f64(s_h))) return ORACLE_NONFINITE;
            scales[n * B + b] = s_h;
            const float sf = (float)oracle_f16_to_f64(s_h);
            uint8_t* blk = codes + (n * B + b) * 16;
            for (int j = 0; j < 16; ++j) blk[j] = 0;
            for (int j = 0; j < 32; ++j) {
                const float t = rintf(w[j] / sf) + 8.0f;
                const int q = t < 0.0f ? 0 : (t > 15.0f ? 15 : (int)t);
                blk[j / 2] |= (uint8_t)(q << (4 * (j % 2)));
            }
        }
    return ORACLE_OK;
}

static int q4b32_code(const uint8_t* codes, int64_t K, int64_t n, int64_t k)
{
    const uint8_t byte = codes[n * (K / 2) + k / 2]; /* 16 bytes per 32 k, row after row */
    return (k % 2) ? (byte >> 4) : (byte & 0xF);
}

/* kind 0: fp32 (q-8)*s_h (exact); kind 1: bf16 of that; kind 2: fp64; kind 3: fp16 of it. */
int oracle_dequant_q4b32(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K,
                         int kind, void* out)
{
    if (!codes || !scales || !out || N <= 0 || K <= 0 || K % 32 || kind < 0 || kind > 3)
        return ORACLE_BAD_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const int q = q4b32_code(codes, K, n, k);
            const float s = (float)oracle_f16_to_f64(scales[n * (K / 32) + k / 32]);
            const float v = (float)(q - 8) * s;
            if (kind == 0)
                ((float*)out)[n * K + k] = v;
            else if (kind == 1)
                ((uint16_t*)out)[n * K + k] = oracle_f32_to_bf16(v);
            else if (kind == 2)
                ((double*)out)[n * K + k] = (double)(q - 8) * oracle_f16_to_f64(scales[n * (K / 32) + k / 32]);
            else
                ((uint16_t*)out)[n * K + k] = oracle_f32_to_f16(v);
        }
    return ORACLE_OK;
}

static double q4b32_weight_exact(const uint8_t* codes, const uint16_t* scales, int64_t K, int64_t n,
                                 int64_t k)
{
    return (double)(q4b32_code(codes, K, n, k) - 8) * oracle_f16_to_f64(scales[n * (K / 32) + k / 32]);
}

/* ------------------------------------------------------------------------------------------
 * Format G128-ZP [P3 "The quantization formulas", "W4A16: dequantizing in registers"]:
 * asymmetric groups of 128 along k with an fp16 scale and an fp16 integer zero point.
 *   codes  uint32 [N][K/8]    word (n, r) holds k = 8r..8r+7 of row n, k = 8r lowest
 *   scales fp16 bits [N][K/128], zeros fp16 bits [N][K/128] (integer values)
 * For every (n, g):
 *   lo, hi = min, max of W[n][128g .. 128g+127]              (a zero is taken as +0)
 *   s = (hi - lo) / 15 in fp32;  s_h = fp16(s), or 1.0 if that is zero
 *   z = clamp(roundf(-lo / s_h), -2048, 2048)  stored as fp16 (exact)
 *   q = clamp(roundf(w / s_h) + z, 0, 15)                    (fp32 divide, half away from zero)
 *   w_hat = (q - z) * s_h, exact in fp32: |q - z| < 2^12 and s_h has 11 significant bits.
 * ---------------------------------------------------------------------------------------- */

int oracle_quantize_g128zp(const float* W, int64_t N, int64_t K, uint32_t* codes, uint16_t* scales,
                           uint16_t* zeros)
{
    if (!W || !codes || !scales || !zeros || N <= 0 || K <= 0 || K % 128) return ORACLE_BAD_ARG;
    const int64_t G = K / 128;
    for (int64_t i = 0; i < N * (K / 8); ++i) codes[i] = 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < G; ++g) {
            const float* w = W + n * K + g * 128;
            float lo = w[0], hi = w[0];
            for (int j = 0; j < 128; ++j) {
                if (!isfinite(w[j])) return ORACLE_NONFINITE;
                if (w[j] < lo) lo = w[j];
                if (w[j] > hi) hi = w[j];
            }
            if (lo == 0.0f) lo = 0.0f;
            if (hi == 0.0f) hi = 0.0f;
            const float s_zp = (hi - lo) / 15.0f;
            uint16_t s_h = oracle_f32_to_f16(s_zp);
            if (s_h == 0 || s_h == 0x8000) s_h = 0x3C00; /* a zero scale becomes 1.0 */
            if (!isfinite(oracle_f16_to_f64(s_h))) return ORACLE_NONFINITE;
            const float sf = (float)oracle_f16_to_f64(s_h);
            float z = roundf(-lo / sf);
            if (z < -2048.0f) z = -2048.0f;
            if (z > 2048.0f) z = 2048.0f;
            if (z == 0.0f) z = 0.0f; /* -0 becomes +0 */
            const uint16_t z_h = oracle_f32_to_f16(z);
            scales[n * G + g] = s_h;
            zeros[n * G + g] = z_h;
            const float zf = (float)oracle_f16_to_f64(z_h);
            for (int j = 0; j < 128; ++j) {
                const float tz = roundf(w[j] / sf) + zf;
                const int q = tz < 0.0f ? 0 : (tz > 15.0f ? 15 : (int)tz);
                const int64_t k = g * 128 + j;
                codes[n * (K / 8) + k / 8] |= (uint32_t)q << (4 * (k % 8));
            }
        }
    return ORACLE_OK;
}

static int g128zp_code(const uint32_t* codes, int64_t K, int64_t n, int64_t k)
{
    uint8_t q[8];
    oracle_unpack_word(codes[n * (K / 8) + k / 8], q);
    return q[k & 7];
}

static double g128zp_weight_exact(const uint32_t* codes, const uint16_t* scales, const uint16_t* zeros,
                                  int64_t K, int64_t n, int64_t k)
{
    const int64_t gi = n * (K / 128) + k / 128;
    return ((double)g128zp_code(codes, K, n, k) - oracle_f16_to_f64(zeros[gi])) * oracle_f16_to_f64(scales[gi]);
}

/* kind 0: fp32 (q - z) * s (exact); kind 1: bf16 of it; kind 2: fp64; kind 3: fp16 of it. */
int oracle_dequant_g128zp(const uint32_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t N,
                          int64_t K, int kind, void* out)
{
    if (!codes || !scales || !zeros || !out || N <= 0 || K <= 0 || K % 128 || kind < 0 || kind > 3)
        return ORACLE_BAD_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const int64_t gi = n * (K / 128) + k / 128;
            const float s = (float)oracle_f16_to_f64(scales[gi]), z = (float)oracle_f16_to_f64(zeros[gi]);
            const float v = ((float)g128zp_code(codes, K, n, k) - z) * s;
            if (kind == 0)
                ((float*)out)[n * K + k] = v;
            else if (kind == 1)
                ((uint16_t*)out)[n * K + k] = oracle_f32_to_bf16(v);
            else if (kind == 2)
                ((double*)out)[n * K + k] = g128zp_weight_exact(codes, scales, zeros, K, n, k);
            else
                ((uint16_t*)out)[n * K + k] = oracle_f32_to_f16(v);
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------
 * Format W8 [P3 "Exercises", 1]: symmetric per-channel int8.
 *   codes  int8 [N][K] row-major;  scales fp32 [N], one per row (output channel)
 * For every row n:  a = max |w|;  s = a / 127 in fp32 (1.0 for an all-zero row);
 *   q = clamp(roundf(w / s), -127, 127)   (fp32 divide, half away from zero: std::round)
 *   w_hat = q * s  (exact in fp64; the fp32 product is rounded)
 * ---------------------------------------------------------------------------------------- */

int oracle_quantize_w8row(const float* W, int64_t N, int64_t K, int8_t* codes, float* scales)
{
    if (!W || !codes || !scales || N <= 0 || K <= 0) return ORACLE_BAD_ARG;
    for (int64_t n = 0; n < N; ++n) {
        const float* w = W + n * K;
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            if (!isfinite(w[k])) return ORACLE_NONFINITE;
            if (fabsf(w[k]) > a) a = fabsf(w[k]);
        }
        float s8 = a / 127.0f;
        if (s8 == 0.0f) s8 = 1.0f;
        scales[n] = s8;
        for (int64_t k = 0; k < K; ++k) {
            const float r8 = roundf(w[k] / s8);
            codes[n * K + k] = (int8_t)(r8 < -127.0f ? -127 : (r8 > 127.0f ? 127 : (int)r8));
        }
    }
    return ORACLE_OK;
}

/* kind 0: fp32 q * s (one rounding); kind 1: bf16 of that fp32 value; kind 2: fp64 (exact);
 * kind 3: fp16 of the fp32 value.  (As for the group-128 format, the reference dequant forms
 * the fp32 weight first and rounds it to 16 bits.) */
int oracle_dequant_w8row(const int8_t* codes, const float* scales, int64_t N, int64_t K, int kind, void* out)
{
    if (!codes || !scales || !out || N <= 0 || K <= 0 || kind < 0 || kind > 3) return ORACLE_BAD_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const double v = (double)codes[n * K + k] * (double)scales[n];
            const float v32 = (float)codes[n * K + k] * scales[n];
            if (kind == 0)
                ((float*)out)[n * K + k] = v32;
            else if (kind == 1)
                ((uint16_t*)out)[n * K + k] = oracle_f32_to_bf16(v32);
            else if (kind == 2)
                ((double*)out)[n * K + k] = v;
            else
                ((uint16_t*)out)[n * K + k] = oracle_f32_to_f16(v32);
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------
 * Matmul y = x . W_hat^T in fp64 [P1 Step 2 accuracy reference; P3 FP64 reference sums]:
 *   y[m][n] = sum over k, in k order, of x[m][k] * w_hat_exact[n][k]
 * x is [M][K] of 16-bit activations: x_kind 0 = bf16 bits, 1 = fp16 bits.
 * The _at variants evaluate only the listed (row, col) outputs, for spot checks at full size.
 * ---------------------------------------------------------------------------------------- */

static double act_value(const uint16_t* x, int x_kind, int64_t i)
{
    return x_kind == 0 ? (double)oracle_bf16_to_f32(x[i]) : oracle_f16_to_f64(x[i]);
}

static double g128_dot(const uint16_t* x, int x_kind, const uint32_t* codes, const uint16_t* scales,
                       const uint16_t* mins, int64_t N, int64_t K, int64_t m, int64_t n)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += act_value(x, x_kind, m * K + k) * g128_weight_exact(codes, scales, mins, N, n, k);
    return acc;
}

static double q4b32_dot(const uint16_t* x, int x_kind, const uint8_t* codes, const uint16_t* scales,
                        int64_t K, int64_t m, int64_t n)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += act_value(x, x_kind, m * K + k) * q4b32_weight_exact(codes, scales, K, n, k);
    return acc;
}

static double g128zp_dot(const uint16_t* x, int x_kind, const uint32_t* codes, const uint16_t* scales,
                         const uint16_t* zeros, int64_t K, int64_t m, int64_t n)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += act_value(x, x_kind, m * K + k) * g128zp_weight_exact(codes, scales, zeros, K, n, k);
    return acc;
}

int oracle_matmul_g128_f64(const uint16_t* x, int x_kind, int64_t M, const uint32_t* codes,
                           const uint16_t* scales, const uint16_t* mins, int64_t N, int64_t K,
                           double* y)
{
    if (!x || !codes || !scales || !mins || !y || M <= 0 || N <= 0 || K <= 0 || K % 128 ||
        (x_kind != 0 && x_kind != 1))
        return ORACLE_BAD_ARG;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) y[m * N + n] = g128_dot(x, x_kind, codes, scales, mins, N, K, m, n);
    return ORACLE_OK;
}

int oracle_matmul_g128_f64_at(const uint16_t* x, int x_kind, int64_t M, const uint32_t* codes,
                              const uint16_t* scales, const uint16_t* mins, int64_t N, int64_t K,
                              const int64_t* rows, const int64_t* cols, int64_t count, double* y)
{
    if (!x || !codes || !scales || !mins || !rows || !cols || !y || M <= 0 || N <= 0 || K <= 0 ||
        K % 128 || count < 0 || (x_kind != 0 && x_kind != 1))
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < count; ++i) {
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return ORACLE_BAD_ARG;
        y[i] = g128_dot(x, x_kind, codes, scales, mins, N, K, rows[i], cols[i]);
    }
    return ORACLE_OK;
}

int oracle_matmul_q4b32_f64(const uint16_t* x, int x_kind, int64_t M, const uint8_t* codes,
                            const uint16_t* scales, int64_t N, int64_t K, double* y)
{
    if (!x || !codes || !scales || !y || M <= 0 || N <= 0 || K <= 0 || K % 32 ||
        (x_kind != 0 && x_kind != 1))
        return ORACLE_BAD_ARG;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) y[m * N + n] = q4b32_dot(x, x_kind, codes, scales, K, m, n);
    return ORACLE_OK;
}

int oracle_matmul_q4b32_f64_at(const uint16_t* x, int x_kind, int64_t M, const uint8_t* codes,
                               const uint16_t* scales, int64_t N, int64_t K, const int64_t* rows,
                               const int64_t* cols, int64_t count, double* y)
{
    if (!x || !codes || !scales || !rows || !cols || !y || M <= 0 || N <= 0 || K <= 0 || K % 32 ||
        count < 0 || (x_kind != 0 && x_kind != 1))
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < count; ++i) {
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return ORACLE_BAD_ARG;
        y[i] = q4b32_dot(x, x_kind, codes, scales, K, rows[i], cols[i]);
    }
    return ORACLE_OK;
}

int oracle_matmul_g128zp_f64(const uint16_t* x, int x_kind, int64_t M, const uint32_t* codes,
                             const uint16_t* scales, const uint16_t* zeros, int64_t N, int64_t K, double* y)
{
    if (!x || !codes || !scales || !zeros || !y || M <= 0 || N <= 0 || K <= 0 || K % 128 ||
        (x_kind != 0 && x_kind != 1))
        return ORACLE_BAD_ARG;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) y[m * N + n] = g128zp_dot(x, x_kind, codes, scales, zeros, K, m, n);
    return ORACLE_OK;
}

int oracle_matmul_g128zp_f64_at(const uint16_t* x, int x_kind, int64_t M, const uint32_t* codes,
                                const uint16_t* scales, const uint16_t* zeros, int64_t N, int64_t K,
                                const int64_t* rows, const int64_t* cols, int64_t count, double* y)
{
    if (!x || !codes || !scales || !zeros || !rows || !cols || !y || M <= 0 || N <= 0 || K <= 0 ||
        K % 128 || count < 0 || (x_kind != 0 && x_kind != 1))
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < count; ++i) {
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return ORACLE_BAD_ARG;
        y[i] = g128zp_dot(x, x_kind, codes, scales, zeros, K, rows[i], cols[i]);
    }
    return ORACLE_OK;
}

int oracle_matmul_w8row_f64(const uint16_t* x, int x_kind, int64_t M, const int8_t* codes, const float* scales,
                            int64_t N, int64_t K, double* y)
{
    if (!x || !codes || !scales || !y || M <= 0 || N <= 0 || K <= 0 || (x_kind != 0 && x_kind != 1))
        return ORACLE_BAD_ARG;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += act_value(x, x_kind, m * K + k) * ((double)codes[n * K + k] * (double)scales[n]);
            y[m * N + n] = acc;
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------
 * W4A8 with the G128 weights [P1']: per-row int8 activations, integer sums per group.
 *   x      bf16 bits [M][K], K % 128 == 0
 *   a_m    = max_k |x[m][k]| / 127 in fp32; 1.0 for an all-zero row       -> ascale fp32 [M]
 *   xq     = clamp(rint(x / a_m), -127, 127)  (fp32 divide, ties to even)  -> int8 [M][K]
 *   X[g][m] = sum of xq[m][k] over group g (an exact integer)              -> xsum fp32 [K/128][M]
 * y[m][n] = sum over k of (a_m * xq[m][k]) * (q * s_b + m_b) in fp64 and k order: the plain
 * product of the dequantized activations and weights (a kernel computes the same number as
 * a_m * sum_g (s_b * sum_k xq * q + m_b * X[g][m])).
 * ---------------------------------------------------------------------------------------- */

int oracle_quantize_act_i8(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* ascale, float* xsum)
{
    if (!x || !xq || !ascale || !xsum || M <= 0 || K <= 0 || K % 128) return ORACLE_BAD_ARG;
    const int64_t G = K / 128;
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float v = oracle_bf16_to_f32(row[k]);
            if (!isfinite(v)) return ORACLE_NONFINITE;
            if (fabsf(v) > amax) amax = fabsf(v);
        }
        float a8 = amax / 127.0f;
        if (a8 == 0.0f) a8 = 1.0f; /* an all-zero row */
        ascale[m] = a8;
        for (int64_t g = 0; g < G; ++g) {
            int64_t sum = 0;
            for (int64_t k = 128 * g; k < 128 * g + 128; ++k) {
                const float t8 = rintf(oracle_bf16_to_f32(row[k]) / a8);
                const int q8 = t8 < -127.0f ? -127 : (t8 > 127.0f ? 127 : (int)t8);
                xq[m * K + k] = (int8_t)q8;
                sum += q8;
            }
            xsum[g * M + m] = (float)sum; /* |sum| <= 127 * 128: exact */
        }
    }
    return ORACLE_OK;
}

static double w4a8_dot(const int8_t* xq, const float* ascale, const uint32_t* codes, const uint16_t* scales,
                       const uint16_t* mins, int64_t N, int64_t K, int64_t m, int64_t n)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += ((double)ascale[m] * (double)xq[m * K + k]) * g128_weight_exact(codes, scales, mins, N, n, k);
    return acc;
}

int oracle_matmul_w4a8_f64(const int8_t* xq, const float* ascale, int64_t M, const uint32_t* codes,
                           const uint16_t* scales, const uint16_t* mins, int64_t N, int64_t K, double* y)
{
    if (!xq || !ascale || !codes || !scales || !mins || !y || M <= 0 || N <= 0 || K <= 0 || K % 128)
        return ORACLE_BAD_ARG;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) y[m * N + n] = w4a8_dot(xq, ascale, codes, scales, mins, N, K, m, n);
    return ORACLE_OK;
}

int oracle_matmul_w4a8_f64_at(const int8_t* xq, const float* ascale, int64_t M, const uint32_t* codes,
                              const uint16_t* scales, const uint16_t* mins, int64_t N, int64_t K,
                              const int64_t* rows, const int64_t* cols, int64_t count, double* y)
{
    if (!xq || !ascale || !codes || !scales || !mins || !rows || !cols || !y || M <= 0 || N <= 0 || K <= 0 ||
        K % 128 || count < 0)
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < count; ++i) {
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return ORACLE_BAD_ARG;
        y[i] = w4a8_dot(xq, ascale, codes, scales, mins, N, K, rows[i], cols[i]);
    }
    return ORACLE_OK;
}

/* The same fp64 product against the ORIGINAL fp32 weights W [N][K]: the quantization error of
 * the format is measured against this, apart from any kernel's implementation error. */
int oracle_matmul_f32w_f64(const uint16_t* x, int x_kind, int64_t M, const float* W, int64_t N,
                           int64_t K, double* y)
{
    if (!x || !W || !y || M <= 0 || N <= 0 || K <= 0 || (x_kind != 0 && x_kind != 1))
        return ORACLE_BAD_ARG;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += act_value(x, x_kind, m * K + k) * (double)W[n * K + k];
            y[m * N + n] = acc;
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------
 * The format-generic calls, dispatching on fmt: 0 = G128, 1 = Q4 block-32, 2 = zero-point,
 * 3 = W8 per row (the library's numbering of its formats).  `mins` holds the minimums (G128) or
 * the zero points (zero-point format) and must be NULL for Q4 and W8, whose scales are fp16 and
 * fp32 respectively.  Each call forwards to the format's own function above, with its layouts,
 * its kinds and its argument checks.
 * ---------------------------------------------------------------------------------------- */
int oracle_quantize_pack(int fmt, const float* W, int64_t N, int64_t K, void* codes, void* scales, void* mins)
{
    switch (fmt) {
    case 0: return oracle_quantize_g128(W, N, K, codes, scales, mins);
    case 1: return mins ? ORACLE_BAD_ARG : oracle_quantize_q4b32(W, N, K, codes, scales);
    case 2: return oracle_quantize_g128zp(W, N, K, codes, scales, mins);
    case 3: return mins ? ORACLE_BAD_ARG : oracle_quantize_w8row(W, N, K, codes, scales);
    default: return ORACLE_BAD_ARG;
    }
}

int oracle_dequant(int fmt, const void* codes, const void* scales, const void* mins, int64_t N, int64_t K,
                   int kind, void* out)
{
    switch (fmt) {
    case 0: return oracle_dequant_g128(codes, scales, mins, N, K, kind, out);
    case 1: return mins ? ORACLE_BAD_ARG : oracle_dequant_q4b32(codes, scales, N, K, kind, out);
    case 2: return oracle_dequant_g128zp(codes, scales, mins, N, K, kind, out);
    case 3: return mins ? ORACLE_BAD_ARG : oracle_dequant_w8row(codes, scales, N, K, kind, out);
    default: return ORACLE_BAD_ARG;
    }
}

int oracle_matmul_f64(int fmt, const uint16_t* x, int x_kind, int64_t M, const void* codes, const void* scales,
                      const void* mins, int64_t N, int64_t K, double* y)
{
    switch (fmt) {
    case 0: return oracle_matmul_g128_f64(x, x_kind, M, codes, scales, mins, N, K, y);
    case 1: return mins ? ORACLE_BAD_ARG : oracle_matmul_q4b32_f64(x, x_kind, M, codes, scales, N, K, y);
    case 2: return oracle_matmul_g128zp_f64(x, x_kind, M, codes, scales, mins, N, K, y);
    case 3: return mins ? ORACLE_BAD_ARG : oracle_matmul_w8row_f64(x, x_kind, M, codes, scales, N, K, y);
    default: return ORACLE_BAD_ARG;
    }
}
