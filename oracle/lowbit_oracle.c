/*
 * lowbit_oracle.c -- plain, slow, obviously correct CPU oracle for
 * weight-only low-bit RTN quantization, packing, dequantization and the fp64
 * reference matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * calls it, and the two share no source, header, table or helper.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (x86-64: float arithmetic is IEEE binary32 in SSE registers, so every
 * float operation below is one correctly rounded IEEE operation).
 *
 * What the method computes, and where it comes from:
 *  - "MinMax" quantization is plain round-to-nearest (RTN) with no calibration
 *    data (BladeLLM model quantization, "Quantization algorithms", MinMax).
 *  - The grid is the uniform asymmetric min-max grid of each row (OPTQ
 *    reproducibility card, "Experiment Setup" row), or of each block of
 *    consecutive input channels sharing one set of parameters (BladeLLM model
 *    quantization, "block_wise_quant": S in R^{Ci/64 x Co}).
 *  - For b bits, M = 2^b - 1:  scale = (max - min) / M,  zero = round(-min/scale),
 *    q = clamp(round(w/scale) + zero, 0, M), with round-half-to-even.
 *  - Several codes share one byte or one 32-bit word: two 4-bit codes per
 *    byte, four 2-bit codes per byte, sixteen 2-bit codes per 32-bit word
 *    ([Feature Request] 4bit and 2bit and 1bit quantization support,
 *    comments).
 *  - At run time the low-bit weights are turned back into real values and
 *    multiplied against fp16 activations (same feature request, elephantpanda's
 *    comment on storing 4-bit weights and converting them with GPU cores);
 *    the weight a code stands for is code times scale, plus the offset the
 *    zero point or block minimum carries (GGUF file format, quantization-type
 *    table: w = q * block_scale + block_minimum).
 *
 * Readings taken where the pages leave a step open (each listed in the design
 * notes of the repository):
 *  R1 scale arithmetic: lo, hi are the fp16 weights widened to fp32 (exact);
 *     d = hi - lo and s32 = d / M are single IEEE fp32 operations; the scale
 *     is stored as s16 = fp16_rne(s32) and the STORED value is the scale used
 *     for the zero point, the codes and the dequantization.
 *  R2 a zero stored scale (hi == lo, or d/M below half the smallest fp16
 *     subnormal) is replaced by 1.0.
 *  R3 zero = (int32) rint(-lo / s) with the division in fp32; kept as a
 *     signed, unclamped int32.
 *  R4 q = clamp((int) rint(w / s) + zero, 0, M) with w / s one fp32 division.
 *  R5 packing: per row, code k occupies bits [b*k, b*k + b) of a little-endian
 *     bitstream of 32-bit words; 3-bit codes straddle word boundaries; every
 *     row starts on a word boundary.
 *  R6 dequantized weight: deq = (q - zero) * s, the exact real value (in
 *     double it is exact: fewer than 44 significant bits); it is not rounded
 *     to fp16 or to any other format.
 *  R7 reference product: y[b][n] = sum_k x[b][k] * deq[n][k] in fp64.
 */
#include "lowbit_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* IEEE 754 binary16 <-> binary64, written from the format's definition:  */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is */
/* the subnormal range (value = frac * 2^-24), exponent 31 is inf / NaN.  */
/* ---------------------------------------------------------------------- */

double orc_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even (the default
 * IEEE rounding-direction attribute).  The scaling by powers of two below is
 * exact, and nearbyint() rounds to an integer in the current rounding mode,
 * which is round-to-nearest-even by default. */
uint16_t orc_f64_to_f16(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7e00;
    if (isinf(a)) return sign | 0x7c00;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: the representable values are multiples of 2^-24 */
        double m = nearbyint(ldexp(a, 24));
        /* m == 1024 is the smallest normal number, whose encoding is 0x0400 */
        return sign | (uint16_t)m;
    }
    int E;
    frexp(a, &E);                 /* a = f * 2^E, f in [0.5, 1) */
    int e = E - 1;                /* a = (2f) * 2^e, 2f in [1, 2) */
    double m = nearbyint(ldexp(a, 10 - e));   /* 11-bit significand */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    if (e > 15) return sign | 0x7c00;         /* overflow rounds to infinity */
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

/* Widths: 2, 3 and 4 bits (the feature request's packed widths), and 8
 * bits (reading R15: BladeLLM's weight-only mode supports 8 and 4 bits,
 * "Quantization modes"; GGUF lists 8-bit round-to-nearest block types next to
 * the 4-bit ones).  Every formula below is written for any b; at 8 bits the
 * bitstream of R5 puts code k in byte k of the row. */
static int valid_bits(int bits) { return bits == 2 || bits == 3 || bits == 4 || bits == 8; }

/* group_size 0 means one group per row */
static int64_t groups_of(int64_t K, int64_t group_size) {
    return group_size == 0 ? 1 : K / group_size;
}

/* ---------------------------------------------------------------------- */
/* Quantization: group min/max, scale, zero point, codes (readings R1-R4). */
/* The core accepts any group size that divides K; the shape rules of the  */
/* GPU library are stricter and are enforced there, not here.              */
/* ---------------------------------------------------------------------- */
int orc_quantize_rtn(const uint16_t* w, int64_t N, int64_t K, int bits, int64_t group_size,
                     uint8_t* codes, uint16_t* scales, int32_t* zeros) {
    if (!w || !codes || !scales || !zeros || N < 0 || K <= 0 || !valid_bits(bits)) return -1;
    if (group_size < 0 || (group_size > 0 && K % group_size != 0)) return -1;
    const int64_t g = group_size == 0 ? K : group_size;
    const int64_t G = groups_of(K, group_size);
    const int M = (1 << bits) - 1;

    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < G; ++j) {
            const uint16_t* wg = w + n * K + j * g;
            /* step 1: the group's minimum and maximum (fp16 -> fp32 is exact) */
            float lo = (float)orc_f16_to_f64(wg[0]);
            float hi = lo;
            for (int64_t k = 1; k < g; ++k) {
                float v = (float)orc_f16_to_f64(wg[k]);
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            /* step 2: scale = (max - min) / M in fp32, stored as fp16 (R1, R2) */
            float d = hi - lo;
            float s32 = d / (float)M;
            uint16_t s16 = orc_f64_to_f16((double)s32);
            if ((s16 & 0x7fff) == 0) s16 = 0x3c00;
            float s = (float)orc_f16_to_f64(s16);
            /* step 3: zero point = round(-min / scale), half to even (R3) */
            float zf = nearbyintf(-lo / s);
            int32_t z = (int32_t)zf;
            scales[n * G + j] = s16;
            zeros[n * G + j] = z;
            /* step 4: codes = clamp(round(w / scale) + zero, 0, M) (R4) */
            for (int64_t k = 0; k < g; ++k) {
                float v = (float)orc_f16_to_f64(wg[k]);
                float t = nearbyintf(v / s);
                int64_t q = (int64_t)t + (int64_t)z;
                if (q < 0) q = 0;
                if (q > M) q = M;
                codes[n * K + j * g + k] = (uint8_t)q;
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Signed symmetric variant (reading R14).  BladeLLM's weight-only modes    */
/* are "signed symmetric" by default (BladeLLM model quantization,          */
/* "Quantization modes"), and the GGUF Q4_0 / Q8_0 types reconstruct a      */
/* weight as code times block scale (GGUF, quantization type table).  The   */
/* grid is centred on zero: with qmax = 2^(b-1) - 1,                        */
/*   s = fp16(fl32(max |w| / qmax)), a zero scale replaced by 1.0,          */
/*   q = clamp(rint(w / s), -qmax, qmax)  (half to even),                   */
/* stored as the code q + 2^(b-1) with the zero point 2^(b-1), so that the   */
/* dequantized weight (code - zero) * s is q * s and the packed form and    */
/* the products are those of the asymmetric mode.                           */
/* ---------------------------------------------------------------------- */
int orc_quantize_rtn_sym(const uint16_t* w, int64_t N, int64_t K, int bits, int64_t group_size,
                         uint8_t* codes, uint16_t* scales, int32_t* zeros) {
    if (!w || !codes || !scales || !zeros || N < 0 || K <= 0 || !valid_bits(bits)) return -1;
    if (group_size < 0 || (group_size > 0 && K % group_size != 0)) return -1;
    const int64_t gs = group_size == 0 ? K : group_size;
    const int64_t ng = groups_of(K, group_size);
    const int qmax = (1 << (bits - 1)) - 1;
    const int32_t z = 1 << (bits - 1);

    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < ng; ++j) {
            const uint16_t* wr = w + n * K + j * gs;
            /* step 1: the group's largest magnitude (fp16 -> fp32 is exact) */
            float amax = 0.0f;
            for (int64_t k = 0; k < gs; ++k) {
                float a = fabsf((float)orc_f16_to_f64(wr[k]));
                if (a > amax) amax = a;
            }
            /* step 2: scale = max|w| / qmax in fp32, stored as fp16; 0 -> 1.0 */
            float sq = amax / (float)qmax;
            uint16_t sh = orc_f64_to_f16((double)sq);
            if ((sh & 0x7fff) == 0) sh = 0x3c00;
            float sc = (float)orc_f16_to_f64(sh);
            scales[n * ng + j] = sh;
            zeros[n * ng + j] = z;
            /* step 3: q = clamp(rint(w / s), -qmax, qmax), code = q + zero */
            for (int64_t k = 0; k < gs; ++k) {
                float v = (float)orc_f16_to_f64(wr[k]);
                float r = nearbyintf(v / sc);
                int64_t q = (int64_t)r;
                if (q < -qmax) q = -qmax;
                if (q > qmax) q = qmax;
                codes[n * K + j * gs + k] = (uint8_t)(q + z);
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Packing (reading R5): code k of a row sits at bit b*k of the row's      */
/* little-endian bitstream.                                                */
/* ---------------------------------------------------------------------- */
int orc_pack(const uint8_t* codes, int64_t N, int64_t K, int bits, uint32_t* packed) {
    if (!codes || !packed || N < 0 || K <= 0 || !valid_bits(bits)) return -1;
    if ((K * bits) % 32 != 0) return -1;
    const int64_t words = K * bits / 32;
    for (int64_t n = 0; n < N; ++n) {
        uint32_t* row = packed + n * words;
        memset(row, 0, (size_t)words * sizeof(uint32_t));
        for (int64_t k = 0; k < K; ++k) {
            uint32_t q = codes[n * K + k];
            int64_t bit = (int64_t)bits * k;
            int64_t wi = bit / 32;
            int off = (int)(bit % 32);
            row[wi] |= q << off;
            if (off + bits > 32) row[wi + 1] |= q >> (32 - off);
        }
    }
    return 0;
}

int orc_unpack(const uint32_t* packed, int64_t N, int64_t K, int bits, uint8_t* codes) {
    if (!codes || !packed || N < 0 || K <= 0 || !valid_bits(bits)) return -1;
    if ((K * bits) % 32 != 0) return -1;
    const int64_t words = K * bits / 32;
    const uint32_t mask = (1u << bits) - 1u;
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t* row = packed + n * words;
        for (int64_t k = 0; k < K; ++k) {
            int64_t bit = (int64_t)bits * k;
            int64_t wi = bit / 32;
            int off = (int)(bit % 32);
            uint32_t q = row[wi] >> off;
            if (off + bits > 32) q |= row[wi + 1] << (32 - off);
            codes[n * K + k] = (uint8_t)(q & mask);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Compact group metadata (reading R16): one 32-bit word per group, the     */
/* fp16 scale in bits 0-15 and the zero point as a two's-complement 16-bit  */
/* integer in bits 16-31, in place of a 2-byte scale plus a 4-byte zero.    */
/* Per-group parameters are what the block formats store next to the codes */
/* (GGUF file format, quantization-type table: a block scale, and for the   */
/* "_1" types a block minimum); this word keeps the integer zero point of    */
/* the min-max grid instead of a float minimum, so the dequantized weights  */
/* do not change.  A zero point outside [-32768, 32767] cannot be stored:   */
/* it is saturated and counted.                                              */
/* ---------------------------------------------------------------------- */
int64_t orc_pack_meta(const uint16_t* scales, const int32_t* zeros, int64_t count,
                      uint32_t* meta) {
    if (!scales || !zeros || !meta || count < 0) return -1;
    int64_t saturated = 0;
    for (int64_t i = 0; i < count; ++i) {
        int32_t z = zeros[i];
        if (z > 32767) { z = 32767; ++saturated; }
        if (z < -32768) { z = -32768; ++saturated; }
        uint32_t zfield = (uint32_t)(uint16_t)(int16_t)z;
        meta[i] = (uint32_t)scales[i] | (zfield << 16);
    }
    return saturated;
}

int orc_unpack_meta(const uint32_t* meta, int64_t count, uint16_t* scales, int32_t* zeros) {
    if (!meta || !scales || !zeros || count < 0) return -1;
    for (int64_t i = 0; i < count; ++i) {
        scales[i] = (uint16_t)(meta[i] & 0xffffu);
        zeros[i] = (int32_t)(int16_t)(uint16_t)(meta[i] >> 16);
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Error-feedback quantization (GPTQ / OPTQ), readings R17-R20.            */
/* BladeLLM model quantization, "Quantization algorithms", GPTQ: the       */
/* parameters of a channel are quantized one after another, and the       */
/* inverse of the Hessian built from the layer's input activations is used */
/* to adjust the parameters not yet quantized, compensating the error.     */
/* OPTQ reproducibility card, "Experiment Setup" row: layer Hessians are   */
/* accumulated from calibration inputs; per-row asymmetric min-max grid.   */
/* ---------------------------------------------------------------------- */

/* H = (2/n) X^T X for calibration inputs x[n][K] (fp16), in fp64, plus      */
/* damp * mean(diag H) on the diagonal (R17).                               */
int orc_hessian(const uint16_t* x, int64_t n, int64_t K, double damp, double* H) {
    if (!x || !H || n <= 0 || K <= 0 || damp < 0) return -1;
    double* row = (double*)malloc((size_t)K * sizeof(double));
    if (!row) return -1;
    /* acc[i][j] = sum over t (in order) of x[t][i] * x[t][j] */
    for (int64_t i = 0; i < K * K; ++i) H[i] = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        for (int64_t i = 0; i < K; ++i) row[i] = orc_f16_to_f64(x[t * K + i]);
        for (int64_t i = 0; i < K; ++i)
            for (int64_t j = 0; j < K; ++j) H[i * K + j] += row[i] * row[j];
    }
    free(row);
    for (int64_t i = 0; i < K * K; ++i) H[i] = 2.0 * H[i] / (double)n;
    double tr = 0.0;
    for (int64_t i = 0; i < K; ++i) tr += H[i * K + i];
    const double add = damp * tr / (double)K;
    for (int64_t i = 0; i < K; ++i) H[i * K + i] += add;
    return 0;
}

/* Inverse of a symmetric positive definite matrix by Gauss-Jordan          */
/* elimination on [A | I] (no pivoting: the pivots of an SPD matrix are      */
/* positive).  Before step c, columns < c of the left half are unit columns  */
/* and row c of the right half is zero beyond column c, so the row updates   */
/* skip those known zeros.  Returns -1 on a non-positive pivot.             */
static int spd_inverse(const double* A, int64_t K, double* inv, double* work) {
    for (int64_t i = 0; i < K; ++i)
        for (int64_t j = 0; j < K; ++j) {
            work[i * K + j] = A[i * K + j];
            inv[i * K + j] = (i == j) ? 1.0 : 0.0;
        }
    for (int64_t c = 0; c < K; ++c) {
        const double p = work[c * K + c];
        if (!(p > 0.0)) return -1;
        for (int64_t j = c; j < K; ++j) work[c * K + j] /= p;
        for (int64_t j = 0; j <= c; ++j) inv[c * K + j] /= p;
        for (int64_t r = 0; r < K; ++r) {
            if (r == c) continue;
            const double f = work[r * K + c];
            if (f == 0.0) continue;
            for (int64_t j = c; j < K; ++j) work[r * K + j] -= f * work[c * K + j];
            for (int64_t j = 0; j <= c; ++j) inv[r * K + j] -= f * inv[c * K + j];
        }
    }
    return 0;
}

/* GPTQ codes for w[N][K] given the Hessian H[K][K] (R18-R20):               */
/*  - the grid (scales, zeros) is the RTN grid of the ORIGINAL weights, per  */
/*    row or per group, exactly as orc_quantize_rtn (min-max) or            */
/*    orc_quantize_rtn_sym (signed symmetric, codes from 1);                */
/*  - columns are taken in their natural order i = 0 .. K-1;                */
/*  - at column i, with Hinv the inverse Hessian of the columns not yet      */
/*    quantized: q = clamp(rint(w_i / s) + z, 0, M) on the current fp64     */
/*    weight, deq = (q - z) * s exactly, err = (w_i - deq) / Hinv[i][i],      */
/*    w_j -= err * Hinv[i][j] for every later column j, then column i is     */
/*    removed from Hinv: Hinv[j][k] -= Hinv[j][i] * Hinv[i][k] / Hinv[i][i]. */
/* Rows are independent, so any subset of rows may be passed.              */
static int gptq_codes(const uint16_t* w, int64_t N, int64_t K, const double* H, int bits,
                      int64_t group_size, int sym, uint8_t* codes, uint16_t* scales,
                      int32_t* zeros, double* work /* 3*K*K + N*K doubles */) {
    if (!w || !H || !codes || !scales || !zeros || !work || N < 0 || K <= 0) return -1;
    const int grid = sym ? orc_quantize_rtn_sym(w, N, K, bits, group_size, codes, scales, zeros)
                         : orc_quantize_rtn(w, N, K, bits, group_size, codes, scales, zeros);
    if (grid != 0) return -1;
    const int64_t minq = sym ? 1 : 0;
    const int64_t g = group_size == 0 ? K : group_size;
    const int64_t G = groups_of(K, group_size);
    const int64_t maxq = (1 << bits) - 1;
    double* hinv = work;
    double* tmp = work + K * K;
    double* cur = work + 3 * K * K;
    if (spd_inverse(H, K, hinv, tmp) != 0) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) cur[n * K + k] = orc_f16_to_f64(w[n * K + k]);
    for (int64_t i = 0; i < K; ++i) {
        const double hii = hinv[i * K + i];
        if (!(hii > 0.0)) return -1;
        for (int64_t n = 0; n < N; ++n) {
            const double s = orc_f16_to_f64(scales[n * G + i / g]);
            const int64_t z = zeros[n * G + i / g];
            const double v = cur[n * K + i];
            int64_t q = (int64_t)nearbyint(v / s) + z;
            if (q < minq) q = minq;
            if (q > maxq) q = maxq;
            codes[n * K + i] = (uint8_t)q;
            const double deq = (double)(q - z) * s;
            const double err = (v - deq) / hii;
            for (int64_t j = i + 1; j < K; ++j) cur[n * K + j] -= err * hinv[i * K + j];
        }
        for (int64_t j = i + 1; j < K; ++j) {
            const double f = hinv[j * K + i] / hii;
            if (f == 0.0) continue;
            for (int64_t k = i + 1; k < K; ++k) hinv[j * K + k] -= f * hinv[i * K + k];
        }
    }
    return 0;
}

int orc_quantize_gptq(const uint16_t* w, int64_t N, int64_t K, const double* H, int bits,
                      int64_t group_size, uint8_t* codes, uint16_t* scales, int32_t* zeros,
                      double* work) {
    return gptq_codes(w, N, K, H, bits, group_size, 0, codes, scales, zeros, work);
}

int orc_quantize_gptq_sym(const uint16_t* w, int64_t N, int64_t K, const double* H, int bits,
                          int64_t group_size, uint8_t* codes, uint16_t* scales, int32_t* zeros,
                          double* work) {
    return gptq_codes(w, N, K, H, bits, group_size, 1, codes, scales, zeros, work);
}

/* ---------------------------------------------------------------------- */
/* Dequantization (reading R6): deq = (q - zero) * scale, exact in fp64.    */
/* ---------------------------------------------------------------------- */
int orc_dequant(const uint8_t* codes, const uint16_t* scales, const int32_t* zeros,
                int64_t N, int64_t K, int bits, int64_t group_size, double* deq) {
    if (!codes || !scales || !zeros || !deq || N < 0 || K <= 0 || !valid_bits(bits)) return -1;
    if (group_size < 0 || (group_size > 0 && K % group_size != 0)) return -1;
    const int64_t g = group_size == 0 ? K : group_size;
    const int64_t G = groups_of(K, group_size);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t j = k / g;
            double s = orc_f16_to_f64(scales[n * G + j]);
            double qz = (double)((int64_t)codes[n * K + k] - (int64_t)zeros[n * G + j]);
            deq[n * K + k] = qz * s;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Reference product (reading R7): y = x * deq^T accumulated in fp64.      */
/* ---------------------------------------------------------------------- */
int orc_matmul_f64(const uint16_t* x, const double* deq, int64_t B, int64_t N, int64_t K,
                   double* y) {
    if (!x || !deq || !y || B < 0 || N < 0 || K <= 0) return -1;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += orc_f16_to_f64(x[b * K + k]) * deq[n * K + k];
            y[b * N + n] = acc;
        }
    }
    return 0;
}
