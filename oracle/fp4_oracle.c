/*
 * fp4_oracle.c - plain, slow CPU oracle for block-scaled FP4 (E2M1) quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library shares
 * no code, header, table or helper with it.
 *
 * Every routine is written from the definitions on the pages it cites:
 *   [FMT]  "NVFP4 / MXFP4 format" article, charlestar.github.io (2026-10-15),
 *          sections 1-8;
 *   [MATH] "FP4 / NVFP4 math summary", devpress.csdn.net (AMD community),
 *          sections 1-11;
 *   [GLOS] Ultralytics glossary "FP4", section "Come funziona FP4";
 *   [PREC] "FP4, FP8 and INT8/INT4: ranges, block scaling and inference
 *          precision", tom-jerr.github.io, sections 2-5.
 * Where those pages leave a step open the reading taken is stated beside it.
 *
 * Arithmetic: IEEE binary32 where the method fixes fp32 (the element divide,
 * the reconstruction, the scale-search loss), otherwise binary64 used only
 * where it is provably exact, or exact comparisons.  Build with
 * -ffp-contract=off and without fast-math so that every C operation is one
 * correctly rounded IEEE operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_FLAG_NONFINITE 1
#define OR_FLAG_SCALE_UNDERFLOW 2

#define OR_DT_F32 0
#define OR_DT_BF16 1

/* ------------------------------------------------------------------------ */
/* Element load: bf16 widens to fp32 exactly (its bits are the top half).   */
/* ------------------------------------------------------------------------ */
static float load_elem(const void *x, int dt, int64_t i) {
    float f;
    if (dt == OR_DT_BF16) {
        uint32_t b = (uint32_t)((const uint16_t *)x)[i] << 16;
        memcpy(&f, &b, 4);
    } else {
        f = ((const float *)x)[i];
    }
    return f;
}

static uint32_t f32_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* ------------------------------------------------------------------------ */
/* E2M1 ([FMT] section 1, table of the eight magnitude codes; [MATH] s.1)   */
/* ------------------------------------------------------------------------ */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Value of a 4-bit code: bit 3 is the sign, bits 0-2 index the magnitude
 * table; code 8 is negative zero ([FMT] section 1). */
double or_e2m1_value(int code) {
    double m = E2M1_MAG[code & 7];
    return (code & 8) ? -m : m;
}

/* RoundE2M1 of a finite fp32 value ([FMT] section 1, "the even of a
 * midpoint is the low bit of the code"): the code whose magnitude is nearest
 * to min(|q|, 6); at an exact midpoint the code with an even low bit wins;
 * the sign bit of q becomes bit 3, so -0.0 and negative values that round
 * to zero give code 8.  Distances are taken in binary64: for |q| >= 0.25 the
 * subtraction is exact (at most 28 significant bits); below 0.25 code 0 is
 * strictly nearest whatever the rounding of the other distances.
 * Returns -1 for a non-finite input (the page rejects it). */
int or_e2m1_round(float q) {
    if (!isfinite(q)) return -1;
    int sign = signbit(q) ? 8 : 0;
    double m = fabs((double)q);
    if (m > 6.0) m = 6.0;
    int best = 0;
    double bestd = fabs(E2M1_MAG[0] - m);
    for (int c = 1; c < 8; ++c) {
        double d = fabs(E2M1_MAG[c] - m);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return sign | best;
}

/* RoundE2M1 applied to each of n fp32 values (code 255 marks a non-finite
 * input). */
void or_e2m1_round_array(const float *q, int64_t n, uint8_t *codes) {
    for (int64_t i = 0; i < n; ++i) {
        int c = or_e2m1_round(q[i]);
        codes[i] = (uint8_t)(c < 0 ? 255 : c);
    }
}

/* Nibble packing ([FMT] section 1): byte j holds code 2j in its low nibble
 * and code 2j+1 in its high nibble.  n must be even. */
void or_pack(const uint8_t *codes, int64_t n, uint8_t *out) {
    for (int64_t j = 0; j < n / 2; ++j)
        out[j] = (uint8_t)((codes[2 * j] & 15) | ((codes[2 * j + 1] & 15) << 4));
}

void or_unpack(const uint8_t *bytes, int64_t nbytes, uint8_t *codes) {
    for (int64_t j = 0; j < nbytes; ++j) {
        codes[2 * j] = bytes[j] & 15;
        codes[2 * j + 1] = bytes[j] >> 4;
    }
}

/* ------------------------------------------------------------------------ */
/* E4M3FN ([FMT] section 2 and section 3: bias 7, max 448, smallest         */
/* subnormal 2^-9, code 0x7F is NaN; the FN variant, not FNUZ)              */
/* ------------------------------------------------------------------------ */
double or_e4m3_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, f = code & 7;
    double v;
    if ((code & 0x7F) == 0x7F) return NAN;
    if (e == 0)
        v = f * ldexp(1.0, -9);
    else
        v = ldexp(1.0 + f / 8.0, e - 7);
    return s ? -v : v;
}

/* Nearest non-negative finite E4M3 code to the exact real num/den, ties to
 * the even code, saturating at 448 (code 126) ([FMT] section 4, the scale
 * encoder: nearest value, even code on a tie, finite saturation).
 * The quotient is never formed: code c is nearer than code b < c exactly
 * when num > den * (v_b + v_c) / 2.  Each midpoint has at most 19
 * significant bits and den = 6 * s_g at most 26, so the product is exact in
 * binary64, as is num (an fp32 value, or the product of two fp32 values).
 * Requires num >= 0, den > 0, both finite. */
static double E4M3_POS[127];
static int e4m3_table_ready = 0;

static void e4m3_table(void) {
    if (e4m3_table_ready) return;
    for (int c = 0; c < 127; ++c) E4M3_POS[c] = or_e4m3_value(c);
    e4m3_table_ready = 1;
}

int or_e4m3_nearest(double num, double den) {
    e4m3_table();
    int best = 0;
    for (int c = 1; c <= 126; ++c) {
        double mid = (E4M3_POS[best] + E4M3_POS[c]) * 0.5;
        double p = mid * den;
        if (num > p || (num == p && (c & 1) == 0)) best = c;
    }
    return best;
}

/* ------------------------------------------------------------------------ */
/* bf16 output rounding: nearest bf16 to a finite fp32 value, ties to the   */
/* even significand (the usual IEEE rule; bf16 shares fp32's exponent       */
/* range, so only the low 16 bits are dropped).  NaN stays a quiet NaN.     */
/* ------------------------------------------------------------------------ */
uint16_t or_f32_to_bf16(float f) {
    uint32_t b = f32_bits(f);
    if (isnan(f)) return (uint16_t)((b >> 16) | 0x40);
    uint32_t lo = b & 0xFFFF, hi = b >> 16;
    if (lo > 0x8000 || (lo == 0x8000 && (hi & 1))) hi += 1;
    return (uint16_t)hi;
}

static void store_out(void *y, int dt, int64_t i, float v) {
    if (dt == OR_DT_BF16)
        ((uint16_t *)y)[i] = or_f32_to_bf16(v);
    else
        ((float *)y)[i] = v;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 ([FMT] section 2: 32-element blocks, E8M0 scale 2^(c-127);          */
/* [FMT] section 5: the OCP recommended conversion)                         */
/* ------------------------------------------------------------------------ */

/* Shared exponent of one MX block by the OCP floor rule ([FMT] section 5):
 * 2^floor(log2 amax) divided by 4, the largest power of two of E2M1, so
 * e = floor(log2 amax) - 2.  floor(log2) is read exactly from frexp, never
 * from a rounded log2.  Readings: a zero block takes e = 0 (scale 1.0, the
 * page's zero convention for scales); e is clamped below at -127, the
 * smallest E8M0 exponent (it binds only for amax < 2^-125). */
int or_mx_exponent(double amax) {
    if (amax == 0.0) return 0;
    int ex;
    (void)frexp(amax, &ex); /* amax = m * 2^ex, m in [0.5, 1) */
    int e = (ex - 1) - 2;
    if (e < -127) e = -127;
    return e;
}

/* Quantize n elements (n a multiple of 32) in 32-element blocks.
 * packed: n/2 bytes, scales: n/32 E8M0 bytes.  Element step: q = x / 2^e
 * as one correctly rounded fp32 division (the method's "divide by the
 * scale"), then RoundE2M1.  Returns OR_FLAG_NONFINITE if any input is
 * not finite (outputs are then unspecified). */
int or_mx_quantize(const void *x, int dt, int64_t n, uint8_t *packed, uint8_t *scales) {
    int flags = 0;
    uint8_t codes[32];
    for (int64_t b = 0; b < n / 32; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            float v = load_elem(x, dt, b * 32 + i);
            if (!isfinite(v)) flags |= OR_FLAG_NONFINITE;
            else if (fabs((double)v) > amax) amax = fabs((double)v);
        }
        int e = or_mx_exponent(amax);
        float s = ldexpf(1.0f, e); /* exact: 2^-127 is an fp32 subnormal */
        scales[b] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; ++i) {
            float v = load_elem(x, dt, b * 32 + i);
            float q = v / s;
            int c = or_e2m1_round(q);
            codes[i] = (uint8_t)(c < 0 ? 0 : c);
        }
        or_pack(codes, 32, packed + b * 16);
    }
    return flags;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 encoder variants ([FMT] section 5: the format fixes the scale set, */
/* not the rule that picks a scale; the OCP floor rule above is one such    */
/* rule).  Element rounding is the same RoundE2M1 in every variant.         */
/* ------------------------------------------------------------------------ */

/* Ceil rule, as the section describes ModelOpt's packed path: the scale is
 * 2^ceil(log2(amax / 6)), i.e. the smallest power of two 2^e with
 * 6 * 2^e >= amax, so the block maximum lands in (3, 6] and never
 * saturates.  Found by exact comparisons (6 * 2^e is exact in binary64).
 * Readings: the lower exponent limit the section mentions is the E8M0
 * minimum -127; a zero block takes e = 0, as under the floor rule. */
int or_mx_exponent_ceil(double amax) {
    if (amax == 0.0) return 0;
    int e = or_mx_exponent(amax); /* floor rule: 4 * 2^e <= amax < 8 * 2^e */
    while (6.0 * ldexp(1.0, e) < amax) ++e;
    while (e > -127 && 6.0 * ldexp(1.0, e - 1) >= amax) --e;
    if (e < -127) e = -127;
    return e;
}

/* Squared error of one 32-element block quantized with scale 2^e, in fp32
 * as the NVFP4 search evaluates its 16-element loss: q = RN32(x / 2^e),
 * x_hat = E2M1(q) * 2^e (exact), err = RN32(x - x_hat), t = RN32(err^2),
 * summed as a balanced pairwise tree in index order. */
float or_block_loss32_pow2(const float *xb, int e) {
    float t[32];
    float s = ldexpf(1.0f, e);
    for (int i = 0; i < 32; ++i) {
        float q = xb[i] / s;
        int c = or_e2m1_round(q);
        float xh = (float)(or_e2m1_value(c) * (double)s);
        float err = xb[i] - xh;
        t[i] = err * err;
    }
    for (int w = 16; w >= 1; w /= 2)
        for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    return t[0];
}

/* MXFP4 quantize with a chosen exponent rule:
 *   rule 0: the OCP floor rule (or_mx_exponent);
 *   rule 1: the ceil rule (or_mx_exponent_ceil);
 *   rule 2: a squared-error search over the E8M0 exponents e0 - 1, e0,
 *           e0 + 1 around the floor rule's e0 (the section's "other
 *           algorithms"; the search objective is the same block MSE the
 *           NVFP4 search minimises).  Readings: e0 is the incumbent and a
 *           neighbour replaces it only with a strictly smaller loss; e0 - 1
 *           is tried before e0 + 1, so of two neighbours with equal loss the
 *           lower exponent wins; exponents below -127 are not candidates; a
 *           zero block keeps e = 0.
 * Outputs as or_mx_quantize. */
int or_mx_quantize_rule(const void *x, int dt, int64_t n, int rule, uint8_t *packed,
                        uint8_t *scales) {
    int flags = 0;
    float xb[32];
    uint8_t codes[32];
    for (int64_t b = 0; b < n / 32; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            xb[i] = load_elem(x, dt, b * 32 + i);
            if (!isfinite(xb[i])) flags |= OR_FLAG_NONFINITE;
            else if (fabs((double)xb[i]) > amax) amax = fabs((double)xb[i]);
        }
        int e = rule == 1 ? or_mx_exponent_ceil(amax) : or_mx_exponent(amax);
        if (rule == 2 && amax != 0.0 && !(flags & OR_FLAG_NONFINITE)) {
            const int e0 = e;
            float best = or_block_loss32_pow2(xb, e0);
            const int alt[2] = {e0 - 1, e0 + 1};
            for (int k = 0; k < 2; ++k) {
                if (alt[k] < -127 || alt[k] > 127) continue;
                float L = or_block_loss32_pow2(xb, alt[k]);
                if (L < best) {
                    best = L;
                    e = alt[k];
                }
            }
        }
        float s = ldexpf(1.0f, e);
        scales[b] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; ++i) {
            int c = or_e2m1_round(xb[i] / s);
            codes[i] = (uint8_t)(c < 0 ? 0 : c);
        }
        or_pack(codes, 32, packed + b * 16);
    }
    return flags;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 ([FMT] section 3: a = A/(6*448), b* = A_g/(6a), b = E4M3(b*),       */
/* p = E2M1(x/(a b)); the block scale is encoded before it quantizes;       */
/* [MATH] section 3 and section 10: alpha_b = s_b * g)                      */
/* ------------------------------------------------------------------------ */

/* Tensor scale ([FMT] section 3, zero/tiny contract): A = max|x|; an all-zero
 * tensor takes a = 1; otherwise a = A / 2688 computed in binary64 and rounded
 * once to fp32, which equals the correctly rounded fp32 quotient.  An a that
 * rounds to zero is an error. */
int or_nv_global_scale(const void *x, int dt, int64_t n, float *s_g) {
    int flags = 0;
    double A = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        float v = load_elem(x, dt, i);
        if (!isfinite(v)) flags |= OR_FLAG_NONFINITE;
        else if (fabs((double)v) > A) A = fabs((double)v);
    }
    if (A == 0.0) {
        *s_g = 1.0f;
        return flags;
    }
    float a = (float)(A / (6.0 * 448.0));
    *s_g = a;
    if (a == 0.0f) flags |= OR_FLAG_SCALE_UNDERFLOW;
    return flags;
}

/* E4M3 block-scale code for block amax A_g under tensor scale s_g: the
 * exact real A_g / (6 s_g) rounded to E4M3 ([FMT] section 3).  The page does
 * not state a precision for this quotient; the exact real is taken. A zero
 * block takes scale 1.0 (code 0x38).  *underflow is set when a nonzero block
 * rounds to code 0. */
static int nv_block_code(double amax, float s_g, int *underflow) {
    if (amax == 0.0) return 0x38;
    int c = or_e4m3_nearest(amax, 6.0 * (double)s_g);
    if (c == 0) *underflow = 1;
    return c;
}

/* The single fp32 scale used for both directions: alpha = RN32(s_g * s_b)
 * ([MATH] section 3, alpha_b = s_b * g; the method divides by one fp32
 * scale).  The binary64 product is exact (24 + 4 significant bits). */
static float nv_alpha(float s_g, int code) {
    return (float)((double)s_g * or_e4m3_value(code));
}

/* Quantize n elements (n a multiple of 16) in 16-element blocks with a given
 * tensor scale s_g (from or_nv_global_scale over the whole tensor).
 * packed: n/2 bytes, scales: n/16 E4M3 bytes. */
int or_nv_quantize(const void *x, int dt, int64_t n, float s_g, uint8_t *packed,
                   uint8_t *scales) {
    int flags = 0;
    uint8_t codes[16];
    for (int64_t b = 0; b < n / 16; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 16; ++i) {
            float v = load_elem(x, dt, b * 16 + i);
            if (!isfinite(v)) flags |= OR_FLAG_NONFINITE;
            else if (fabs((double)v) > amax) amax = fabs((double)v);
        }
        int under = 0;
        int sc = nv_block_code(amax, s_g, &under);
        float alpha = nv_alpha(s_g, sc);
        if (alpha == 0.0f) under = 1;
        if (under) flags |= OR_FLAG_SCALE_UNDERFLOW;
        scales[b] = (uint8_t)sc;
        for (int i = 0; i < 16; ++i) {
            float v = load_elem(x, dt, b * 16 + i);
            int c = (alpha == 0.0f) ? -1 : or_e2m1_round(v / alpha);
            codes[i] = (uint8_t)(c < 0 ? 0 : c);
        }
        or_pack(codes, 16, packed + b * 8);
    }
    return flags;
}

/* ------------------------------------------------------------------------ */
/* Dequantization ([MATH] section 10: x_hat = q * alpha_b; [FMT] section 2,  */
/* x_hat = s * p with p the decoded E2M1 value)                              */
/* fmt 0 = MXFP4 (block 32, E8M0), fmt 1 = NVFP4 (block 16, E4M3 * s_g).     */
/* MX: value * 2^e is exact in fp32 and bf16.  NV: RN32(value * alpha), then */
/* the output rounding.  A NaN scale code (E8M0 255, E4M3 0x7F/0xFF) gives   */
/* NaN outputs.                                                              */
/* ------------------------------------------------------------------------ */
void or_dequantize(int fmt, const uint8_t *packed, const uint8_t *scales, float s_g,
                   int64_t n, int out_dt, void *y) {
    int block = fmt == 0 ? 32 : 16;
    for (int64_t i = 0; i < n; ++i) {
        int code = (i & 1) ? (packed[i / 2] >> 4) : (packed[i / 2] & 15);
        int sc = scales[i / block];
        double val = or_e2m1_value(code);
        float out;
        if (fmt == 0) {
            if (sc == 255) out = NAN;
            else out = (float)(val * ldexp(1.0, sc - 127));
        } else {
            double sb = or_e4m3_value(sc);
            if (isnan(sb)) out = NAN;
            else {
                float alpha = (float)((double)s_g * sb);
                out = (float)(val * (double)alpha);
            }
        }
        store_out(y, out_dt, i, out);
    }
}

/* ------------------------------------------------------------------------ */
/* MSE-optimal block-scale search ([MATH] section 9: choose the scale that    */
/* minimises sum_i (x_i - s * Round_FP4(x_i / s))^2; [FMT] section 4: the    */
/* encoded scale is what quantizes, and a max-based scale need not be the    */
/* MSE optimum).                                                             */
/*                                                                           */
/* Readings (the pages fix none of these):                                   */
/*  - candidate k of n: c_k = RN32(((n-1-k) c_lo + k c_hi) / (n-1)), i.e.    */
/*    linspace(c_lo, c_hi, n) rounded once to fp32;                          */
/*  - each candidate is encoded first: code_k = E4M3(c_k * A_g / (6 s_g))    */
/*    as an exact real; code 0 is skipped; alpha_k = RN32(s_g * s_b(code_k));*/
/*  - the loss is evaluated in fp32 exactly as the kernel evaluates it:      */
/*    q = RN32(x/alpha), x_hat = RN32(E2M1(q) * alpha), e = RN32(x - x_hat), */
/*    t = RN32(e*e), summed as a balanced pairwise tree in index order       */
/*    ((t0+t1)+(t2+t3))+... ;                                                */
/*  - the winner is the smallest k with the least loss.                      */
/* ------------------------------------------------------------------------ */
float or_block_loss_f32(const float *xb, float alpha) {
    float t[16];
    for (int i = 0; i < 16; ++i) {
        float q = xb[i] / alpha;
        int c = or_e2m1_round(q);
        float xh = (float)(or_e2m1_value(c) * (double)alpha);
        float e = xb[i] - xh;
        t[i] = e * e;
    }
    for (int w = 8; w >= 1; w /= 2)
        for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    return t[0];
}

float or_candidate_c(int k, int ncand, float c_lo, float c_hi) {
    double num = (double)(ncand - 1 - k) * (double)c_lo + (double)k * (double)c_hi;
    return (float)(num / (double)(ncand - 1));
}

/* Search over n elements (multiple of 16) with tensor scale s_g.
 * best_loss (nullable) receives the winning fp32 loss of each block. */
int or_scale_search(const void *x, int dt, int64_t n, float s_g, int ncand, float c_lo,
                    float c_hi, uint8_t *packed, uint8_t *scales, float *best_loss) {
    int flags = 0;
    float xb[16];
    uint8_t codes[16];
    for (int64_t b = 0; b < n / 16; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 16; ++i) {
            xb[i] = load_elem(x, dt, b * 16 + i);
            if (!isfinite(xb[i])) flags |= OR_FLAG_NONFINITE;
            else if (fabs((double)xb[i]) > amax) amax = fabs((double)xb[i]);
        }
        int win = -1;
        float winloss = 0.0f;
        if (amax == 0.0) {
            win = 0x38;
        } else {
            for (int k = 0; k < ncand; ++k) {
                float ck = or_candidate_c(k, ncand, c_lo, c_hi);
                int code = or_e4m3_nearest((double)ck * amax, 6.0 * (double)s_g);
                if (code == 0) continue;
                float alpha = nv_alpha(s_g, code);
                if (alpha == 0.0f) continue;
                float L = or_block_loss_f32(xb, alpha);
                if (win < 0 || L < winloss) {
                    win = code;
                    winloss = L;
                }
            }
        }
        if (win < 0) {
            flags |= OR_FLAG_SCALE_UNDERFLOW;
            win = 0;
        }
        float alpha = nv_alpha(s_g, win);
        scales[b] = (uint8_t)win;
        if (best_loss) best_loss[b] = winloss;
        for (int i = 0; i < 16; ++i) {
            int c = (alpha == 0.0f) ? -1 : or_e2m1_round(xb[i] / alpha);
            codes[i] = (uint8_t)(c < 0 ? 0 : c);
        }
        or_pack(codes, 16, packed + b * 8);
    }
    return flags;
}

/* Brute force over every E4M3 block scale ([FMT] section 4: the worked
 * block [0.4 x 15, 3.6] at a = 1, where the max-based 0.625 loses to 0.875,
 * found by trying every legal E4M3 scale).  Per block with amax > 0, every
 * code 1..126 whose alpha = RN32(s_g * E4M3(code)) is nonzero is a
 * candidate; the loss is or_block_loss_f32; the winner is the smallest code
 * with the least loss.  A zero block takes 0x38.  Outputs as
 * or_scale_search. */
int or_scale_search_all(const void *x, int dt, int64_t n, float s_g, uint8_t *packed,
                        uint8_t *scales, float *best_loss) {
    int flags = 0;
    float xb[16];
    uint8_t codes[16];
    for (int64_t b = 0; b < n / 16; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 16; ++i) {
            xb[i] = load_elem(x, dt, b * 16 + i);
            if (!isfinite(xb[i])) flags |= OR_FLAG_NONFINITE;
            else if (fabs((double)xb[i]) > amax) amax = fabs((double)xb[i]);
        }
        int win = -1;
        float winloss = 0.0f;
        if (amax == 0.0) {
            win = 0x38;
        } else {
            for (int code = 1; code <= 126; ++code) {
                float alpha = nv_alpha(s_g, code);
                if (alpha == 0.0f) continue;
                float L = or_block_loss_f32(xb, alpha);
                if (win < 0 || L < winloss) {
                    win = code;
                    winloss = L;
                }
            }
        }
        if (win < 0) {
            flags |= OR_FLAG_SCALE_UNDERFLOW;
            win = 0;
        }
        float alpha = nv_alpha(s_g, win);
        scales[b] = (uint8_t)win;
        if (best_loss) best_loss[b] = winloss;
        for (int i = 0; i < 16; ++i) {
            int c = (alpha == 0.0f) ? -1 : or_e2m1_round(xb[i] / alpha);
            codes[i] = (uint8_t)(c < 0 ? 0 : c);
        }
        or_pack(codes, 16, packed + b * 8);
    }
    return flags;
}

/* ------------------------------------------------------------------------ */
/* Ideal, unencoded scale (teaching device of [MATH] sections 7-8 and the     */
/* [GLOS] block-size snippet): alpha = RN32(A_g / 6) per block of `block`    */
/* elements, q = RN32(x / alpha), reconstruction RN32(E2M1(q) * alpha).      */
/* A zero block reconstructs to zeros.  Used only to reproduce the pages'    */
/* printed numbers; it is not an encoder of either format.                   */
/* ------------------------------------------------------------------------ */
void or_ideal_roundtrip(const float *x, int64_t n, int block, float *y) {
    for (int64_t b = 0; b < n / block; ++b) {
        double amax = 0.0;
        for (int i = 0; i < block; ++i)
            if (fabs((double)x[b * block + i]) > amax) amax = fabs((double)x[b * block + i]);
        float alpha = (float)amax / 6.0f;
        for (int i = 0; i < block; ++i) {
            float v = x[b * block + i];
            if (alpha == 0.0f) { y[b * block + i] = 0.0f * v; continue; }
            int c = or_e2m1_round(v / alpha);
            y[b * block + i] = (float)(or_e2m1_value(c) * (double)alpha);
        }
    }
}

/* Ideal-scale code of one value at a given scale ([MATH] sections 5 and 8:
 * x / alpha, then the nearest FP4 value). */
int or_ideal_code(float x, float alpha) { return or_e2m1_round(x / alpha); }

/* Storage of complete blocks ([FMT] section 8): T/2 payload bytes, one byte
 * per block and `global_bytes` for a tensor scale. */
int64_t or_storage_bytes(int64_t elements, int block, int64_t global_bytes) {
    return elements / 2 + elements / block + global_bytes;
}

/* ------------------------------------------------------------------------ */
/* Row-padded layout ([FMT] section 8: an R x K matrix whose rows are padded */
/* to whole blocks holds B = R * ceil(K / G) blocks and B (G/2 + 1) bytes,   */
/* plus 4 for the NVFP4 tensor scale; decoding restores the padded layout   */
/* and crops each row to the logical shape kept as metadata).  Readings:    */
/* the padding elements are zeros (code 0), so they change no block amax;   */
/* the NVFP4 tensor scale is that of the logical elements.  Each routine    */
/* builds the zero-padded matrix and runs the complete-block routine on it. */
/* ------------------------------------------------------------------------ */

static float *padded_copy(const void *x, int dt, int64_t rows, int64_t cols, int block,
                          int64_t *pcols) {
    int64_t pc = (cols + block - 1) / block * block;
    float *xp = (float *)calloc((size_t)(rows * pc), sizeof(float));
    if (!xp) return NULL;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) xp[r * pc + c] = load_elem(x, dt, r * cols + c);
    *pcols = pc;
    return xp;
}

int64_t or_padded_storage_bytes(int64_t rows, int64_t cols, int block, int64_t global_bytes) {
    int64_t nb = rows * ((cols + block - 1) / block);
    return nb * (block / 2 + 1) + global_bytes;
}

/* packed: rows * pcols / 2 bytes; scales: rows * pcols / 32.  Returns flags,
 * or -1 if memory ran out. */
int or_mx_quantize_padded(const void *x, int dt, int64_t rows, int64_t cols, uint8_t *packed,
                          uint8_t *scales) {
    int64_t pc;
    float *xp = padded_copy(x, dt, rows, cols, 32, &pc);
    if (!xp) return -1;
    int f = or_mx_quantize(xp, OR_DT_F32, rows * pc, packed, scales);
    free(xp);
    return f;
}

/* s_g is read from the logical elements (or_nv_global_scale), then the
 * padded matrix is quantized with it.  Returns flags, or -1. */
int or_nv_quantize_padded(const void *x, int dt, int64_t rows, int64_t cols, uint8_t *packed,
                          uint8_t *scales, float *s_g) {
    int f = or_nv_global_scale(x, dt, rows * cols, s_g);
    if (f) return f;
    int64_t pc;
    float *xp = padded_copy(x, dt, rows, cols, 16, &pc);
    if (!xp) return -1;
    f |= or_nv_quantize(xp, OR_DT_F32, rows * pc, *s_g, packed, scales);
    free(xp);
    return f;
}

/* Dequantize a padded layout and crop each row to cols values. */
int or_dequantize_padded(int fmt, const uint8_t *packed, const uint8_t *scales, float s_g,
                         int64_t rows, int64_t cols, int out_dt, void *y) {
    int block = fmt == 0 ? 32 : 16;
    int64_t pc = (cols + block - 1) / block * block;
    float *yp = (float *)malloc((size_t)(rows * pc) * sizeof(float));
    if (!yp) return -1;
    or_dequantize(fmt, packed, scales, s_g, rows * pc, OR_DT_F32, yp);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) store_out(y, out_dt, r * cols + c, yp[r * pc + c]);
    free(yp);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Stochastic rounding to E2M1 ([GLOS] section "Inferenza e addestramento   */
/* FP4": NVFP4 pretraining rounds gradients stochastically; the pages give   */
/* no rule, only the name).                                                  */
/* Readings: the quotient q is the deterministic path's (fp32 correctly      */
/* rounded); |q| >= 6 saturates; otherwise with lo <= |q| < hi the two       */
/* neighbouring E2M1 magnitudes, q rounds up with probability (|q| - lo) /    */
/* (hi - lo), decided by 24 random bits r as r * (hi - lo) * 2^-24 < |q| - lo */
/* (exact: both sides are exact in binary64); grid values never move; the    */
/* sign comes from the sign bit, as in RoundE2M1.                            */
/* Random bits: SplitMix64 (Steele, Lea and Flood, "Fast splittable          */
/* pseudorandom number generators", 2014; the finalizer with Stafford's       */
/* "Mix13" constants) on the counter seed + (i/2 + 1) * 0x9E3779B97F4A7C15,  */
/* i the flat element index; element i takes the top 24 bits of the low (i   */
/* even) or high (i odd) 32-bit half.                                        */
/* ------------------------------------------------------------------------ */

static uint64_t splitmix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint32_t or_sr_bits(uint64_t seed, int64_t i) {
    uint64_t z = splitmix64(seed + ((uint64_t)i / 2 + 1) * 0x9E3779B97F4A7C15ull);
    uint32_t half = (i & 1) ? (uint32_t)(z >> 32) : (uint32_t)z;
    return half >> 8;
}

int or_e2m1_round_sr(float q, uint32_t r24) {
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    int s = signbit(q) ? 8 : 0;
    double m = fabs((double)q);
    if (m >= 6.0) return s | 7;
    int k = 0;
    while (k < 7 && mag[k + 1] <= m) ++k; /* mag[k] <= m < mag[k+1] */
    if (m == mag[k]) return s | k;
    double gap = mag[k + 1] - mag[k];
    int up = (double)r24 * gap * 0x1p-24 < m - mag[k];
    return s | (k + up);
}

/* MXFP4 / NVFP4 quantize with stochastic element rounding; scales as the
 * deterministic encoders (OCP floor rule; NVFP4 max-based E4M3 with the
 * given s_g).  Outputs and flags as or_mx_quantize / or_nv_quantize. */
int or_mx_quantize_sr(const void *x, int dt, int64_t n, uint64_t seed, uint8_t *packed,
                      uint8_t *scales) {
    int flags = 0;
    uint8_t codes[32];
    for (int64_t b = 0; b < n / 32; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            float v = load_elem(x, dt, b * 32 + i);
            if (!isfinite(v)) flags |= OR_FLAG_NONFINITE;
            else if (fabs((double)v) > amax) amax = fabs((double)v);
        }
        int e = or_mx_exponent(amax);
        float sc = ldexpf(1.0f, e);
        scales[b] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; ++i) {
            int64_t idx = b * 32 + i;
            float q = load_elem(x, dt, idx) / sc;
            codes[i] = (uint8_t)or_e2m1_round_sr(q, or_sr_bits(seed, idx));
        }
        or_pack(codes, 32, packed + b * 16);
    }
    return flags;
}

int or_nv_quantize_sr(const void *x, int dt, int64_t n, float s_g, uint64_t seed,
                      uint8_t *packed, uint8_t *scales) {
    int flags = 0;
    uint8_t codes[16];
    for (int64_t b = 0; b < n / 16; ++b) {
        double amax = 0.0;
        for (int i = 0; i < 16; ++i) {
            float v = load_elem(x, dt, b * 16 + i);
            if (!isfinite(v)) flags |= OR_FLAG_NONFINITE;
            else if (fabs((double)v) > amax) amax = fabs((double)v);
        }
        int under = 0;
        int code = amax == 0.0 ? 0x38 : nv_block_code(amax, s_g, &under);
        float alpha = nv_alpha(s_g, code);
        if (under || alpha == 0.0f) flags |= OR_FLAG_SCALE_UNDERFLOW;
        scales[b] = (uint8_t)code;
        for (int i = 0; i < 16; ++i) {
            int64_t idx = b * 16 + i;
            float q = alpha == 0.0f ? 0.0f : load_elem(x, dt, idx) / alpha;
            codes[i] = (uint8_t)or_e2m1_round_sr(q, or_sr_bits(seed, idx));
        }
        or_pack(codes, 16, packed + b * 8);
    }
    return flags;
}

