/*
 * pn_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow, obviously-correct CPU oracle for the decode-step GEMV y = W.x over
 * block-quantized weights (PN types pn3t / pn4t, and NVFP4 W4A16). It is written from the
 * format pages' definitions, step by step, and shares no code, header, table or constant
 * generator with the GPU library. Only the test suite, the smoke entry and the bench's
 * CPU-baseline leg load it. The GPU library never calls it.
 *
 * Sources (cited by page title and section):
 *   [PN]    "PN weight format" (tensorless docs, PNX-FORMAT-v0): sections "Types",
 *           "Block layout", "Value", "Reference quantizer", "Validation".
 *   [QP]    "Quantisation and profiles" (TandemLLM docs): sections "NVFP4", "The clip search".
 *   [TF]    NInfer "tensor formats" maintainer page: the BF16 word (section 3.1), the NVFP4
 *           representation with its E2M1 / E4M3FN words (section 3.3), the row-scaled E4M3FN
 *           format FP8_E4M3FN_ROW_BF16S (section 3.4), and the integral rounding examples of the
 *           canonical encoder (section 7).
 *   [QP]    also "The FP8 head": one scale per row, a search over 1.0, 0.95, 0.90 of the row's
 *           largest weight.
 *
 * Floating point: everything that is not stated as fp32 by the pages is done in double.
 * Build with -ffp-contract=off so that no multiply-add is fused behind our back.
 *
 * Pins (what fixes each function other than itself; the tests under tests/ check them):
 *   codecs      exhaustive closed forms of the pages; numpy's binary16 rounding as a library pin.
 *   PN layout   the bit table and the shift formula are written separately (pack / unpack) and
 *               must round-trip; a decoder that shifts by element index must fail the fixtures.
 *   PN decode   the printed ranges -4d..+3d / -8d..+7d and the -0.0 rule, over all 65,536 d words.
 *   validation  the closed rule over all d words and every single-bit flip of the payload.
 *   GEMV        exact rational brute force on small rows; one-hot and block-indicator x.
 *   quantizers  invariants and brute-force re-scans only: parity unpinned against the engines'
 *               own quantizers (no printed vectors exist on the pages).
 *   Hadamard    against an independent library construction of the Sylvester matrix (scipy),
 *               the textbook H_2 / H_4, involution (H_B / sqrt(B) is symmetric and orthogonal),
 *               norm preservation; the rotated GEMV against a dense product of those.
 *   row E4M3    decode by the section 3.4 product over all 256 code words at power-of-two and
 *               other scales; each validity clause of section 3.4 on its own; the bf16 rounding
 *               against the integer round-half-even of binary32 words.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OR_PN3T 124
#define OR_PN4T 125

/* ------------------------------------------------------------------------------------------ */
/* binary16 / bfloat16 / E4M3FN / E2M1 words                                                   */
/* ------------------------------------------------------------------------------------------ */

/* IEEE binary16 word -> exact double value. Subnormals are m * 2^-24; no flush to zero. */
double or_f16_to_double(uint16_t h)
{
    int neg = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return neg ? -v : v;
}

/* double -> binary16 with one round-to-nearest-even step, subnormals kept, overflow to inf.
 * This is the "rounded to fp16" of [PN] "Reference quantizer", read as a single rounding
 * from the double value. */
uint16_t or_double_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7E00);
    if (isinf(v))
        return (uint16_t)(sign | 0x7C00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: the quantum is 2^-24; a * 2^24 is exact in double */
        double r = rint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)r); /* r == 1024 is the smallest normal, 0x0400 */
    }
    int e2;
    frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;         /* a in [2^E, 2^(E+1)) */
    double r = rint(ldexp(a, 10 - E)); /* significand * 1024, in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)r - 1024));
}

/* [TF] section 3.1: a bfloat16 word is the high half of a binary32 word. */
float or_bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Double -> bfloat16 word, one rounding to nearest with ties to even (8 significant bits,
 * binary32's exponent range, subnormals down to 2^-133), +-inf past the largest finite value. */
uint16_t or_double_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80);
    int e2;
    frexp(a, &e2);
    int E = e2 - 1; /* a in [2^E, 2^(E+1)) */
    if (E < -126) {
        double r = rint(ldexp(a, 133)); /* subnormal quantum 2^-133; r = 128 is the smallest normal */
        return (uint16_t)(sign | (uint16_t)r);
    }
    double r = rint(ldexp(a, 7 - E)); /* in [128, 256] */
    if (r == 256.0) {
        r = 128.0;
        E += 1;
    }
    if (E > 127)
        return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)(r - 128.0));
}

/* [TF] section 3.3: E4M3FN. sign bit 7, exponent bits 6:3 (bias 7), fraction bits 2:0.
 * e = 0: m * 2^-9; 1 <= e <= 14, and e = 15 with m < 7: (1 + m/8) * 2^(e-7); e = 15, m = 7: NaN. */
double or_e4m3_to_double(uint8_t c)
{
    int neg = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return neg ? -v : v;
}

/* [TF] section 3.3: E2M1. sign bit 3, exponent bits 2:1, mantissa bit 0.
 * Positive words 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6 ([QP] "NVFP4" lists the same grid). */
double or_e2m1_to_double(uint8_t c)
{
    int neg = (c >> 3) & 1;
    int e = (c >> 1) & 3;
    int m = c & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return neg ? -v : v;
}

/* Non-negative double -> E4M3FN word, nearest with ties to the even fraction, saturating at the
 * largest finite value 448 (word 0x7E); never produces the NaN word. Used by the NVFP4 quantizer. */
uint8_t or_double_to_e4m3_sat(double v)
{
    if (!(v > 0))
        return 0; /* +0 (callers pass v >= 0) */
    if (v >= 448.0)
        return 0x7E;
    if (v < ldexp(1.0, -6)) {
        double r = rint(ldexp(v, 9)); /* subnormal quantum 2^-9 */
        return (uint8_t)r;            /* r == 8 is the smallest normal, word 0x08 */
    }
    int e2;
    frexp(v, &e2);
    int E = e2 - 1; /* v in [2^E, 2^(E+1)), E in [-6, 8] */
    double r = rint(ldexp(v, 3 - E)); /* in [8, 16] */
    if (r == 16.0) {
        r = 8.0;
        E += 1;
    }
    int code = ((E + 7) << 3) | ((int)r - 8);
    if (code > 0x7E)
        code = 0x7E;
    return (uint8_t)code;
}

/* Signed double -> E2M1 word: nearest grid value {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the word
 * with an even mantissa bit, saturating at 6. Negative inputs keep the sign bit, even when the
 * magnitude rounds to zero (word 0x8). */
uint8_t or_double_to_e2m1_sat(double v)
{
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs(v);
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    int best = 7;
    if (a < 6.0) {
        for (int c = 0; c < 7; c++) {
            double lo = grid[c], hi = grid[c + 1];
            if (a <= hi) {
                double dlo = a - lo, dhi = hi - a;
                if (dlo < dhi)
                    best = c;
                else if (dhi < dlo)
                    best = c + 1;
                else
                    best = (c % 2 == 0) ? c : c + 1; /* tie: even mantissa bit */
                break;
            }
        }
    }
    return (uint8_t)(sign | best);
}

/* ------------------------------------------------------------------------------------------ */
/* PN format                                                                                   */
/* ------------------------------------------------------------------------------------------ */

/* [PN] "Types": pn3t holds 80 weights of 3 bits, 10 codes per u32 word, zero point 4;
 * pn4t holds 64 weights of 4 bits, 8 codes per word, zero point 8. Both are 34 bytes. */
int or_pn_params(int type, int *bits, int *per_block, int *per_word, int *z)
{
    if (type == OR_PN3T) {
        *bits = 3; *per_block = 80; *per_word = 10; *z = 4;
        return 0;
    }
    if (type == OR_PN4T) {
        *bits = 4; *per_block = 64; *per_word = 8; *z = 8;
        return 0;
    }
    return -1;
}

static uint32_t rd_le32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

static void wr_le32(uint8_t *p, uint32_t v)
{
    p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); p[2] = (uint8_t)(v >> 16); p[3] = (uint8_t)(v >> 24);
}

/* Unpack one 34-byte block with the shift formula of [PN] "Block layout":
 * element e is in word e / per_word, local index t = e mod per_word,
 * code = (word >> (BITS * (t >> 1) + 16 * (t & 1))) & (2^BITS - 1).
 * Bytes are assembled one at a time, so no alignment is assumed. */
void or_pn_unpack_block(int type, const uint8_t *blk, uint16_t *d, uint8_t *codes)
{
    int bits, G, cpw, z;
    or_pn_params(type, &bits, &G, &cpw, &z);
    *d = (uint16_t)(blk[0] | (blk[1] << 8));
    for (int e = 0; e < G; e++) {
        int i = e / cpw, t = e % cpw;
        uint32_t word = rd_le32(blk + 2 + 4 * i);
        int shift = bits * (t >> 1) + 16 * (t & 1);
        codes[e] = (uint8_t)((word >> shift) & ((1u << bits) - 1));
    }
}

/* Pack one block from the bit table of [PN] "Block layout": even t = 2j sits at bits
 * BITS*j .. of the low 16-bit half, odd t = 2j+1 at the same bits of the high half; for pn3t bits
 * 15 and 31 stay 0. Codes are masked to BITS bits. */
void or_pn_pack_block(int type, uint16_t d, const uint8_t *codes, uint8_t *blk)
{
    int bits, G, cpw, z;
    or_pn_params(type, &bits, &G, &cpw, &z);
    blk[0] = (uint8_t)(d & 0xFF);
    blk[1] = (uint8_t)(d >> 8);
    uint32_t mask = (1u << bits) - 1;
    for (int i = 0; i < 8; i++) {
        uint32_t lo = 0, hi = 0;
        for (int j = 0; j < cpw / 2; j++) {
            lo |= ((uint32_t)codes[i * cpw + 2 * j] & mask) << (bits * j);
            hi |= ((uint32_t)codes[i * cpw + 2 * j + 1] & mask) << (bits * j);
        }
        wr_le32(blk + 2 + 4 * i, lo | (hi << 16));
    }
}

/* Bytes per row of K weights; 0 if K is not a whole number of blocks. */
int64_t or_pn_row_bytes(int type, int64_t K)
{
    int bits, G, cpw, z;
    if (or_pn_params(type, &bits, &G, &cpw, &z) || K <= 0 || K % G)
        return 0;
    return (K / G) * 34;
}

/* [PN] "Value": w = d * (n - z), computed in fp32. Both factors are exact in fp32 and so is the
 * product; IEEE signs apply, so code z with a negative d gives -0.0. */
void or_pn_dequantize_row(int type, const uint8_t *row, int64_t K, float *out)
{
    int bits, G, cpw, z;
    or_pn_params(type, &bits, &G, &cpw, &z);
    uint8_t codes[80];
    for (int64_t b = 0; b < K / G; b++) {
        uint16_t d16;
        or_pn_unpack_block(type, row + 34 * b, &d16, codes);
        float d = (float)or_f16_to_double(d16);
        for (int e = 0; e < G; e++)
            out[b * G + e] = d * (float)(codes[e] - z);
    }
}

void or_pn_dequantize_rows(int type, const uint8_t *W, int64_t nrows, int64_t K, float *out)
{
    int64_t rb = or_pn_row_bytes(type, K);
    for (int64_t r = 0; r < nrows; r++)
        or_pn_dequantize_row(type, W + r * rb, K, out + r * K);
}

/* [PN] "Validation": a row is invalid when some block's d is an fp16 NaN or infinity, or, for
 * pn3t, when bit 15 or bit 31 of some word is set. Returns 1 for a valid row, 0 otherwise. */
int or_pn_validate_row(int type, const uint8_t *row, int64_t K)
{
    int bits, G, cpw, z;
    or_pn_params(type, &bits, &G, &cpw, &z);
    for (int64_t b = 0; b < K / G; b++) {
        const uint8_t *blk = row + 34 * b;
        uint16_t d16 = (uint16_t)(blk[0] | (blk[1] << 8));
        if (!isfinite(or_f16_to_double(d16)))
            return 0;
        if (type == OR_PN3T)
            for (int i = 0; i < 8; i++)
                if (rd_le32(blk + 2 + 4 * i) & 0x80008000u)
                    return 0;
    }
    return 1;
}

void or_pn_validate_rows(int type, const uint8_t *W, int64_t nrows, int64_t K, int32_t *verdict)
{
    int64_t rb = or_pn_row_bytes(type, K);
    for (int64_t r = 0; r < nrows; r++)
        verdict[r] = or_pn_validate_row(type, W + r * rb, K);
}

/* The code step of [PN] "Reference quantizer": n = clamp(rint(w / s) + z, 0, 2z - 1), with the
 * quotient and the clamp in double. rint rounds half-way cases to even (the C default mode), which
 * matches the canonical encoder's printed examples in [TF] section 7 (+-0.5 -> 0, +-1.5 -> +-2,
 * +-2.5 -> +-2). */
int or_pn_code(double w, double s, int z)
{
    double q = rint(w / s) + z;
    if (q < 0)
        q = 0;
    if (q > 2 * z - 1)
        q = 2 * z - 1;
    return (int)q;
}

/* Status bits of the reference quantizer. */
#define OR_Q_NONFINITE 1 /* a group held a NaN or infinity: written as the canonical zero group */
#define OR_Q_OVERFLOW 2  /* every candidate scale overflowed fp16: canonical zero group */

/* [PN] "Reference quantizer", for one group of G fp32 weights:
 *  1. amax, max and min in double; amax == 0 gives the canonical zero group (d = +0, codes z).
 *  2. sigma = +1 if |min| > max, else -1.
 *  3. for m = 0.50, 0.52, ..., 1.20 (36 values, m_i = (50 + 2i) / 100):
 *       s = fp16(sigma * m * amax / z), skipped when it is zero (or not finite);
 *       n_k = clamp(rint(w_k / s) + z, 0, 2z - 1);
 *       err = sum_k (w_k - s (n_k - z))^2 in double.
 *  4. keep the smallest err; a tie goes to the larger m (ascending scan with <=).
 * When every candidate is zero (a tiny group) the group is written as the canonical zero group. */
static int quantize_group(int type, const float *w, uint8_t *blk)
{
    int bits, G, cpw, z;
    or_pn_params(type, &bits, &G, &cpw, &z);
    uint8_t codes[80], trial[80];
    double amax = 0.0, mx = -INFINITY, mn = INFINITY;
    int status = 0;
    for (int k = 0; k < G; k++) {
        double v = (double)w[k];
        if (!isfinite(v))
            status |= OR_Q_NONFINITE;
        if (fabs(v) > amax) amax = fabs(v);
        if (v > mx) mx = v;
        if (v < mn) mn = v;
    }
    uint16_t dbest = 0;
    for (int k = 0; k < G; k++)
        codes[k] = (uint8_t)z;
    if (status || amax == 0.0) {
        or_pn_pack_block(type, 0, codes, blk);
        return status;
    }
    double sigma = (fabs(mn) > mx) ? 1.0 : -1.0;
    double best = INFINITY;
    int found = 0, overflowed = 0;
    for (int i = 0; i < 36; i++) {
        double m = (50 + 2 * i) / 100.0;
        uint16_t s16 = or_double_to_f16(sigma * m * amax / z);
        double s = or_f16_to_double(s16);
        if (s == 0.0)
            continue;
        if (!isfinite(s)) {
            overflowed = 1;
            continue;
        }
        double err = 0.0;
        for (int k = 0; k < G; k++) {
            trial[k] = (uint8_t)or_pn_code((double)w[k], s, z);
            double e = (double)w[k] - s * (double)((int)trial[k] - z);
            err += e * e;
        }
        if (err <= best) {
            best = err;
            dbest = s16;
            memcpy(codes, trial, (size_t)G);
            found = 1;
        }
    }
    if (!found) {
        for (int k = 0; k < G; k++)
            codes[k] = (uint8_t)z;
        or_pn_pack_block(type, 0, codes, blk);
        return overflowed ? OR_Q_OVERFLOW : 0;
    }
    or_pn_pack_block(type, dbest, codes, blk);
    return 0;
}

/* Quantize rows [0, nrows) of w (row-major, K per row). status[r] ORs the group statuses. */
int or_pn_quantize_rows(int type, const float *w, int64_t nrows, int64_t K, uint8_t *W, int32_t *status)
{
    int bits, G, cpw, z;
    if (or_pn_params(type, &bits, &G, &cpw, &z) || K % G)
        return -1;
    int64_t rb = or_pn_row_bytes(type, K);
    for (int64_t r = 0; r < nrows; r++) {
        int st = 0;
        for (int64_t b = 0; b < K / G; b++)
            st |= quantize_group(type, w + r * K + b * G, W + r * rb + 34 * b);
        if (status)
            status[r] = st;
    }
    return 0;
}

/* Decode-step GEMV, y[m, n] = sum_k w[n, k] x[m, k], accumulated in double in k order, with
 * bound[m, n] = sum_k |w[n, k] x[m, k]|. w is the fp32 decode of [PN] "Value"; every product
 * w * x is exact in double. */
void or_pn_gemv(int type, const uint8_t *W, int64_t N, int64_t K, const float *x, int64_t M,
                double *y, double *bound)
{
    int64_t rb = or_pn_row_bytes(type, K);
    int bits, G, cpw, z;
    or_pn_params(type, &bits, &G, &cpw, &z);
    uint8_t codes[80];
    double acc[M], abs_acc[M];
    for (int64_t n = 0; n < N; n++) {
        for (int64_t m = 0; m < M; m++)
            acc[m] = abs_acc[m] = 0.0;
        for (int64_t b = 0; b < K / G; b++) {
            uint16_t d16;
            or_pn_unpack_block(type, W + n * rb + 34 * b, &d16, codes);
            float d = (float)or_f16_to_double(d16);
            for (int e = 0; e < G; e++) {
                double wv = (double)(d * (float)(codes[e] - z));
                for (int64_t m = 0; m < M; m++) {
                    double p = wv * (double)x[m * K + b * G + e];
                    acc[m] += p;
                    abs_acc[m] += fabs(p);
                }
            }
        }
        for (int64_t m = 0; m < M; m++) {
            y[m * N + n] = acc[m];
            bound[m * N + n] = abs_acc[m];
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Hadamard-rotated activations ([PN] "Files that use PN": the model applies a Hadamard rotation */
/* to the activations that reach the PN weights; the engine performs it). The page gives neither */
/* the order of the transform nor its normalisation. Reading: K is cut into consecutive slices   */
/* of B elements (B a power of two dividing K), and each slice is multiplied by the orthonormal  */
/* Sylvester-ordered Walsh-Hadamard matrix H_B / sqrt(B), with H_B[i][j] = (-1)^popcount(i & j) */
/* (the closed form of the Sylvester doubling H_2n = [[H, H], [H, -H]]).                         */
/* ------------------------------------------------------------------------------------------ */

static int popcount64(uint64_t v)
{
    int c = 0;
    while (v) {
        c += (int)(v & 1);
        v >>= 1;
    }
    return c;
}

/* out[m, k] = (1/sqrt(B)) sum_{j < B} H_B[i][j] x[m, base + j] for k = base + i, the matrix product
 * written out (B^2 terms per slice), in double. mass[m, k] = (1/sqrt(B)) sum_j |x[m, base + j]|:
 * the sum of the magnitudes that meet in out[m, k] (used by the tests to bound rounding). Either
 * output may be NULL. */
void or_hadamard_rows(const double *x, int64_t M, int64_t K, int64_t B, double *out, double *mass)
{
    const double inv = 1.0 / sqrt((double)B);
    for (int64_t m = 0; m < M; m++) {
        for (int64_t base = 0; base < K; base += B) {
            const double *xs = x + m * K + base;
            double amass = 0.0;
            for (int64_t j = 0; j < B; j++)
                amass += fabs(xs[j]);
            for (int64_t i = 0; i < B; i++) {
                double acc = 0.0;
                for (int64_t j = 0; j < B; j++)
                    acc += (popcount64((uint64_t)(i & j)) & 1) ? -xs[j] : xs[j];
                if (out)
                    out[m * K + base + i] = acc * inv;
                if (mass)
                    mass[m * K + base + i] = amass * inv;
            }
        }
    }
}

/* The GEMV of "PN weight format" with activations given in double (the rotated x above):
 * y[m, n] = sum_k w[n, k] x[m, k] in double, bound[m, n] = sum_k |w[n, k] x[m, k]|, and, when
 * xmass is given, mbound[m, n] = sum_k |w[n, k]| xmass[m, k]. */
void or_pn_gemv_dx(int type, const uint8_t *W, int64_t N, int64_t K, const double *x,
                   const double *xmass, int64_t M, double *y, double *bound, double *mbound)
{
    int64_t rb = or_pn_row_bytes(type, K);
    int bits, G, cpw, z;
    or_pn_params(type, &bits, &G, &cpw, &z);
    uint8_t codes[80];
    double acc[M], abs_acc[M], m_acc[M];
    for (int64_t n = 0; n < N; n++) {
        for (int64_t m = 0; m < M; m++)
            acc[m] = abs_acc[m] = m_acc[m] = 0.0;
        for (int64_t b = 0; b < K / G; b++) {
            uint16_t d16;
            or_pn_unpack_block(type, W + n * rb + 34 * b, &d16, codes);
            float d = (float)or_f16_to_double(d16);
            for (int e = 0; e < G; e++) {
                double w_nk = (double)(d * (float)(codes[e] - z));
                for (int64_t m = 0; m < M; m++) {
                    double p = w_nk * x[m * K + b * G + e];
                    acc[m] += p;
                    abs_acc[m] += fabs(p);
                    if (xmass)
                        m_acc[m] += fabs(w_nk) * xmass[m * K + b * G + e];
                }
            }
        }
        for (int64_t m = 0; m < M; m++) {
            y[m * N + n] = acc[m];
            bound[m * N + n] = abs_acc[m];
            if (mbound)
                mbound[m * N + n] = m_acc[m];
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* NVFP4 (W4A16)                                                                              */
/* Layout (the pages leave it open; this is the reading used throughout): codes [N, K/2] bytes, */
/* element k in byte k/2 with even k in the low nibble; scales [N, K/16] E4M3FN words, row-major. */
/* ------------------------------------------------------------------------------------------ */

/* [QP] "NVFP4": w = e2m1(code) * weight_scale[n, k / 16] * weight_scale_2, in fp32:
 * the first product is exact in fp32, the second rounds once. */
void or_nvfp4_dequantize_rows(const uint8_t *codes, const uint8_t *scales, float g, int64_t N,
                              int64_t K, float *out)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            uint8_t byte = codes[n * (K / 2) + k / 2];
            uint8_t c = (k & 1) ? (byte >> 4) : (byte & 0xF);
            float e = (float)or_e2m1_to_double(c);
            float s = (float)or_e4m3_to_double(scales[n * (K / 16) + k / 16]);
            float p = e * s;
            out[n * K + k] = p * g;
        }
}

/* [TF] section 3.3 validity: stored scale words must be sign-zero and finite (+0 allowed;
 * negative values, -0 and the NaN words are invalid); the global field must be finite and > 0.
 * Returns 1 for a valid row. */
void or_nvfp4_validate_rows(const uint8_t *scales, float g, int64_t N, int64_t K, int32_t *verdict)
{
    int gok = isfinite(g) && g > 0.0f;
    for (int64_t n = 0; n < N; n++) {
        int ok = gok;
        for (int64_t j = 0; j < K / 16; j++) {
            uint8_t s = scales[n * (K / 16) + j];
            if ((s & 0x80) || (s & 0x7F) == 0x7F)
                ok = 0;
        }
        verdict[n] = ok;
    }
}

/* Global multiplier: fp32(amax_tensor / (6 * 448)), or 1 for an all-zero tensor. Returns NaN when
 * the tensor holds a non-finite value. */
float or_nvfp4_global_scale(const float *w, int64_t count)
{
    double amax = 0.0;
    for (int64_t i = 0; i < count; i++) {
        double v = fabs((double)w[i]);
        if (!isfinite(v))
            return NAN;
        if (v > amax)
            amax = v;
    }
    if (amax == 0.0)
        return 1.0f;
    return (float)(amax / (6.0 * 448.0));
}

/* [QP] "The clip search", with uniform channel weights (act_ms = 1): for each group of 16, try the
 * multipliers 1.00, 0.95, 0.90, 0.85, 0.80 on the group's scale, round every weight to the nearest
 * E2M1 word, and keep the multiplier whose decoded weights have the smallest squared error. For
 * multiplier c the scale word is e4m3(c * amax_group / (6 g)), saturated at 448; each code is the
 * E2M1 rounding of w / (S g), or +0 when S is 0. A tie keeps the earlier (larger) multiplier. */
void or_nvfp4_quantize_rows(const float *w, int64_t N, int64_t K, float g, uint8_t *codes,
                            uint8_t *scales)
{
    static const double mult[5] = {1.00, 0.95, 0.90, 0.85, 0.80};
    for (int64_t n = 0; n < N; n++)
        for (int64_t j = 0; j < K / 16; j++) {
            const float *wg = w + n * K + j * 16;
            double amax = 0.0;
            for (int k = 0; k < 16; k++)
                if (fabs((double)wg[k]) > amax)
                    amax = fabs((double)wg[k]);
            double best = INFINITY;
            uint8_t best_s = 0, best_c[16], trial[16];
            memset(best_c, 0, sizeof best_c);
            for (int i = 0; i < 5; i++) {
                uint8_t sw = or_double_to_e4m3_sat(mult[i] * amax / (6.0 * (double)g));
                double S = or_e4m3_to_double(sw);
                double err = 0.0;
                for (int k = 0; k < 16; k++) {
                    trial[k] = (S == 0.0) ? 0 : or_double_to_e2m1_sat((double)wg[k] / (S * (double)g));
                    float p = (float)or_e2m1_to_double(trial[k]) * (float)S;
                    float dq = p * g;
                    double e = (double)wg[k] - (double)dq;
                    err += e * e;
                }
                if (err < best) {
                    best = err;
                    best_s = sw;
                    memcpy(best_c, trial, 16);
                }
            }
            scales[n * (K / 16) + j] = best_s;
            for (int k = 0; k < 16; k += 2)
                codes[n * (K / 2) + (j * 16 + k) / 2] = (uint8_t)(best_c[k] | (best_c[k + 1] << 4));
        }
}

/* W4A16 GEMV: y[m, n] = sum_k w[n, k] x[m, k] in double, w the fp32 decode above and x the exact
 * fp32 expansion of the bf16 activations; bound = sum |w x|. */
void or_nvfp4_gemv(const uint8_t *codes, const uint8_t *scales, float g, int64_t N, int64_t K,
                   const uint16_t *x, int64_t M, double *y, double *bound)
{
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0, abs_acc = 0.0;
            for (int64_t k = 0; k < K; k++) {
                uint8_t byte = codes[n * (K / 2) + k / 2];
                uint8_t c = (k & 1) ? (byte >> 4) : (byte & 0xF);
                float e = (float)or_e2m1_to_double(c);
                float s = (float)or_e4m3_to_double(scales[n * (K / 16) + k / 16]);
                float p = e * s;
                double wv = (double)(p * g);
                double pr = wv * (double)or_bf16_to_float(x[m * K + k]);
                acc += pr;
                abs_acc += fabs(pr);
            }
            y[m * N + n] = acc;
            bound[m * N + n] = abs_acc;
        }
}

/* ------------------------------------------------------------------------------------------ */
/* Row-scaled E4M3FN ([TF] section 3.4, FP8_E4M3FN_ROW_BF16S; [QP] "The FP8 head"): codes        */
/* [N, K] E4M3FN words, row-major; one bfloat16 multiplier word per row.                         */
/* ------------------------------------------------------------------------------------------ */

/* [TF] section 3.4: w = binary32(e4m3(c) * bf16(s)), the scale a multiplier. */
void or_fp8row_dequantize_rows(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                               float *out)
{
    for (int64_t n = 0; n < N; n++) {
        float s32 = or_bf16_to_float(scales[n]);
        for (int64_t k = 0; k < K; k++) {
            float c32 = (float)or_e4m3_to_double(codes[n * K + k]);
            out[n * K + k] = c32 * s32;
        }
    }
}

/* [TF] section 3.4 validity, per row: the scale word has sign bit 0 and is finite (positive zero
 * and positive subnormals included); no code is a NaN word (0x7F, 0xFF); a positive-zero scale
 * requires every code to be a signed zero (0x00 or 0x80). Returns 1 for a valid row. */
void or_fp8row_validate_rows(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                             int32_t *verdict)
{
    for (int64_t n = 0; n < N; n++) {
        uint16_t s = scales[n];
        int ok = !(s & 0x8000) && (s & 0x7F80) != 0x7F80;
        for (int64_t k = 0; k < K; k++) {
            uint8_t c = codes[n * K + k];
            if ((c & 0x7F) == 0x7F)
                ok = 0;
            if (s == 0 && (c & 0x7F) != 0)
                ok = 0;
        }
        verdict[n] = ok;
    }
}

/* [QP] "The FP8 head", with the scale stored as the [TF] section 3.4 bfloat16 multiplier: for each
 * row and each multiplier c in 1.0, 0.95, 0.90, the scale word is bf16(c * amax / 448) (skipped when
 * it is zero or not finite); each code is the E4M3FN word nearest to w / s, ties to the even
 * fraction, saturating at 448, sign kept (also when the magnitude rounds to zero); the error is the
 * squared difference between w and the fp32 decode, summed in double over k in increasing order
 * (the plain sum; the pages do not say more); the smallest error wins, a tie keeping the earlier
 * multiplier. An all-zero row, or one whose candidates are
 * all skipped, is scale +0 with codes 0x00. status[n] = 1 when the row holds a NaN or infinity
 * (the row is then written as the zero row). */
void or_fp8row_quantize_rows(const float *w, int64_t N, int64_t K, uint8_t *codes,
                             uint16_t *scales, int32_t *status)
{
    static const double mult[3] = {1.0, 0.95, 0.90};
    for (int64_t n = 0; n < N; n++) {
        const float *wr = w + n * K;
        uint8_t *cr = codes + n * K;
        double amax = 0.0;
        int bad = 0;
        for (int64_t k = 0; k < K; k++) {
            double a = fabs((double)wr[k]);
            if (!isfinite(a))
                bad = 1;
            else if (a > amax)
                amax = a;
        }
        status[n] = bad;
        scales[n] = 0;
        memset(cr, 0, (size_t)K);
        if (bad || amax == 0.0)
            continue;
        double best = INFINITY;
        for (int i = 0; i < 3; i++) {
            uint16_t sw = or_double_to_bf16(mult[i] * amax / 448.0);
            double sd = (double)or_bf16_to_float(sw);
            if (sd == 0.0 || !isfinite(sd))
                continue;
            float s32 = (float)sd;
            double err = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double q = (double)wr[k] / sd;
                uint8_t c = (uint8_t)((signbit(q) ? 0x80 : 0) | or_double_to_e4m3_sat(fabs(q)));
                float dq = (float)or_e4m3_to_double(c) * s32;
                double e = (double)wr[k] - (double)dq;
                err += e * e;
            }
            if (err < best) {
                best = err;
                scales[n] = sw;
                for (int64_t k = 0; k < K; k++) {
                    double q = (double)wr[k] / sd;
                    cr[k] = (uint8_t)((signbit(q) ? 0x80 : 0) | or_double_to_e4m3_sat(fabs(q)));
                }
            }
        }
    }
}

/* GEMV: y[m, n] = sum_k w[n, k] x[m, k] in double with w the fp32 decode above, x fp32;
 * bound = sum |w x|. */
void or_fp8row_gemv(const uint8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                    const float *x, int64_t M, double *y, double *bound)
{
    for (int64_t n = 0; n < N; n++) {
        float s32 = or_bf16_to_float(scales[n]);
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0, abs_acc = 0.0;
            for (int64_t k = 0; k < K; k++) {
                float wv = (float)or_e4m3_to_double(codes[n * K + k]) * s32;
                double pr = (double)wv * (double)x[m * K + k];
                acc += pr;
                abs_acc += fabs(pr);
            }
            y[m * N + n] = acc;
            bound[m * N + n] = abs_acc;
        }
    }
}

void or_double_to_bf16_n(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = or_double_to_bf16(v[i]);
}

/* Vector helpers for the tests (element-wise wrappers of the scalar codecs). */
void or_f16_to_double_n(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = or_f16_to_double(h[i]);
}

void or_double_to_f16_n(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = or_double_to_f16(v[i]);
}

void or_double_to_e4m3_sat_n(const double *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = or_double_to_e4m3_sat(v[i]);
}

void or_double_to_e2m1_sat_n(const double *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = or_double_to_e2m1_sat(v[i]);
}
