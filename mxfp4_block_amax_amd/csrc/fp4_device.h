// fp4_device.h - gfx950 device helpers for block-scaled FP4 (E2M1) kernels.
//
// Format facts used here ("NVFP4 / MXFP4 format" page, charlestar.github.io,
// sections 1-3): E2M1 codes with bit 3 the sign and magnitudes
// {0, .5, 1, 1.5, 2, 3, 4, 6}, rounded to nearest with ties to the even code
// and saturated at 6; E8M0 scale byte c = 2^(c-127); E4M3FN block scales
// (bias 7, max 448 at code 0x7E, subnormal step 2^-9).
//
// Compile with -ffp-contract=off: every fp32 expression below is meant as the
// separately rounded IEEE operations it spells; fused operations are written
// explicitly with __builtin_fma*.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_recip_table.h"

namespace fp4dev {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr uint32_t FLAG_NONFINITE = 1;
constexpr uint32_t FLAG_SCALE_UNDERFLOW = 2;
constexpr uint32_t FLAG_BARRIER_TIMEOUT = 4;

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

// The scale operand of the gfx950 v_cvt_scalef32_* conversions carries an
// E8M0 exponent in the fp32 exponent field: byte c is passed as c << 23.
__device__ __forceinline__ float e8m0_operand(uint32_t c) { return u2f(c << 23); }
constexpr uint32_t E8M0_ONE = 127u;

// Streaming (non-temporal) 16-byte loads and stores: data touched once.
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
    u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(uint4 *p, uint4 v) {
    u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (u32x4_t *)p);
}

// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format,
// no swizzle): the form untyped buffer loads and stores take.
constexpr int kBufferRsrcWord3 = 0x00020000;

// ---- DPP lane exchange inside quads -------------------------------------
constexpr int QP_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int QP_XOR2 = 0x4E;  // quad_perm [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    // full row and bank masks: every lane is written, so no old value (and
    // bound_ctrl changes nothing for in-quad permutes)
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return u2f(dpp<CTRL>(f2u(v)));
}

// ---- block amax on bit patterns -----------------------------------------
// |x| ordering of finite values equals the unsigned ordering of their
// sign-cleared bit patterns, and NaN/Inf patterns sort above every finite
// one, so an integer max both finds the amax and flags non-finite input.

// Max of the 8 sign-cleared bf16 patterns held in a uint4 (as 16-bit value).
__device__ __forceinline__ uint32_t amax_bf16x8(uint4 w) {
    u16x2_t a = __builtin_bit_cast(u16x2_t, w.x & 0x7FFF7FFFu);
    u16x2_t b = __builtin_bit_cast(u16x2_t, w.y & 0x7FFF7FFFu);
    u16x2_t c = __builtin_bit_cast(u16x2_t, w.z & 0x7FFF7FFFu);
    u16x2_t d = __builtin_bit_cast(u16x2_t, w.w & 0x7FFF7FFFu);
    u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                          __builtin_elementwise_max(c, d));
    return m.x > m.y ? (uint32_t)m.x : (uint32_t)m.y;
}

// Max of 8 sign-cleared fp32 patterns.
__device__ __forceinline__ uint32_t amax_f32x8(uint4 lo, uint4 hi) {
    uint32_t m0 = max(max(lo.x & 0x7FFFFFFFu, lo.y & 0x7FFFFFFFu), lo.z & 0x7FFFFFFFu);
    uint32_t m1 = max(max(lo.w & 0x7FFFFFFFu, hi.x & 0x7FFFFFFFu), hi.y & 0x7FFFFFFFu);
    uint32_t m2 = max(hi.z & 0x7FFFFFFFu, hi.w & 0x7FFFFFFFu);
    return max(max(m0, m1), m2);
}

// ---- E2M1 conversion on the hardware converter ---------------------------
// v_cvt_scalef32_pk_fp4_{bf16,f32}: two values divided by the E8M0 scale
// (an exponent shift), rounded to nearest E2M1 with ties to even, saturated,
// sign kept; the pair lands in byte SEL of the result, first value in the
// low nibble.  Bit-exactness against the RoundE2M1 definition is a parity
// test (all bf16 patterns times every scale exponent).
__device__ __forceinline__ uint32_t cvt_fp4x8_bf16(uint4 w, float scale) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w.x), scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w.y), scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w.z), scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w.w), scale, 3);
    return r;
}

__device__ __forceinline__ uint32_t cvt_fp4x8_f32(const float (&q)[8], float scale) {
    // the four converts write all four bytes: the start value (here the
    // first input's bits, which need no register of their own) is never read
    uint32_t r = __builtin_bit_cast(uint32_t, q[0]);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q[0], q[1], scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q[2], q[3], scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q[4], q[5], scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, q[6], q[7], scale, 3);
    return r;
}

// Unpack a 16-byte chunk into 8 fp32 values (bf16 widens exactly).
__device__ __forceinline__ void widen_bf16x8(uint4 w, float (&x)[8]) {
    x[0] = u2f(w.x << 16); x[1] = u2f(w.x & 0xFFFF0000u);
    x[2] = u2f(w.y << 16); x[3] = u2f(w.y & 0xFFFF0000u);
    x[4] = u2f(w.z << 16); x[5] = u2f(w.z & 0xFFFF0000u);
    x[6] = u2f(w.w << 16); x[7] = u2f(w.w & 0xFFFF0000u);
}
__device__ __forceinline__ void widen_f32x8(uint4 lo, uint4 hi, float (&x)[8]) {
    x[0] = u2f(lo.x); x[1] = u2f(lo.y); x[2] = u2f(lo.z); x[3] = u2f(lo.w);
    x[4] = u2f(hi.x); x[5] = u2f(hi.y); x[6] = u2f(hi.z); x[7] = u2f(hi.w);
}

// ---- MX shared exponent (OCP floor rule, format page section 5) ----------
// From the amax bit pattern (exponent field E, width ebits shift `sh`):
// e = floor(log2 amax) - 2, clamped at -127; byte = e + 127.  For a normal
// amax floor(log2) = E - 127, so byte = max(E - 2, 0); a subnormal amax has
// floor(log2) <= -127, giving byte 0; a zero block takes byte 127.
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits, int exp_shift) {
    if (amax_bits == 0) return E8M0_ONE;
    uint32_t E = amax_bits >> exp_shift;
    return E > 2u ? E - 2u : 0u;
}

// Ceil rule (format page, section 5, the ModelOpt packed path): the smallest
// e with 6 * 2^e >= amax, clamped at -127.  For a normal amax = m 2^(E-127),
// m in [1, 2): e = E - 127 - 2 + [m > 1.5], since 6 * 2^(E-129) = 1.5 * 2^(E-127);
// a subnormal amax gives e <= -128, clamped; a zero block takes byte 127.
__device__ __forceinline__ uint32_t mx_scale_byte_ceil(uint32_t amax_bits, int exp_shift) {
    if (amax_bits == 0) return E8M0_ONE;
    const uint32_t E = amax_bits >> exp_shift;
    if (E == 0) return 0u;
    const uint32_t frac = amax_bits & ((1u << exp_shift) - 1u);
    const int b = (int)E - 2 + (frac > (1u << (exp_shift - 1)) ? 1 : 0);
    return b > 0 ? (uint32_t)b : 0u;
}

// ---- E4M3FN block scales --------------------------------------------------
// Value of a non-negative finite code c in [0, 126].
__device__ __forceinline__ float e4m3_pos_value(uint32_t c) {
    return c >= 8u ? u2f((((c >> 3) + 120u) << 23) | ((c & 7u) << 20))
                   : (float)c * 0x1p-9f;
}

// Significand index k (E4M3(c) = (1 + k/8) 2^e) of a nonzero code c.
__device__ __forceinline__ uint32_t e4m3_frac_index(uint32_t c) {
    // subnormal codes c 2^-9: 1, 2, 4 -> 1; 3, 6 -> 1.5; 5 -> 1.25; 7 -> 1.75
    return c >= 8u ? (c & 7u) : ((0x64204000u >> (4u * c)) & 0xFu);
}

// 6 times the midpoint between codes c and c+1, c in [0, 125]; exact in fp32.
// Subnormal side: (2c+1) * 2^-10; normal side: 2^(E-7) (17 + 2f) / 16.
__device__ __forceinline__ float e4m3_mid6(uint32_t c) {
    if (c < 8u) return (float)(3u * (2u * c + 1u)) * 0x1p-9f;
    float p2 = u2f(((c >> 3) - 10u + 127u) << 23);
    return (float)(3u * (17u + 2u * (c & 7u))) * p2;
}

// ---- per-tensor E4M3 block-scale table ------------------------------------
// Once s_g is known the NVFP4 block scale is a function of the block amax
// alone and takes one of 127 values, so a workgroup tabulates per call:
//   lo[k]  the smallest fp32 amax whose code is >= k (lo[0] = 0, lo[127] =
//          +inf), from the exact threshold 6 * midpoint(k-1, k) * s_g (at most
//          31 significant bits, so exact in binary64); at an exact tie the
//          amax goes to the even code;
//   th[k]  that threshold itself, for amax multiples that are not fp32;
//   q[c]   {alpha_c, alpha'_c, +-1/alpha'_c, sc_c}: alpha_c = RN32(s_g E4M3(c));
//          the divide x / alpha_c is done as (x sc) / alpha'_c with
//          alpha'_c = alpha_c sc, where sc = 2^64 when alpha_c < 2^-90 (else
//          1): scaling both operands by a power of two leaves the quotient
//          unchanged and keeps the reciprocal-correction divide away from
//          underflow.  The reciprocal is 0 when alpha_c = 0 (a scale
//          underflow; outputs are then unspecified).  Its sign bit marks
//          codes whose one-multiply quotient may differ (see below).
//
// One-multiply quotient for bf16 input.  With y = RN32(1/a), q0 = RN32(x y)
// is within 2^-23 (relative) of x/a, and RN32(x/a) within 2^-24, so their
// E2M1 codes can differ only if x/a lies within 2^-22 of a decision point m
// (0.25, 0.75, ..., 5).  A bf16 value (scaled by sc or not) has at most 8
// significant bits; if no such value lies that close to m a, for every m,
// the product alone decides every bf16 element of a block with this scale.
constexpr float kDivScale = 0x1p64f;
constexpr float kDivScaleBelow = 0x1p-90f;

struct NvScaleTable {
    float lo[128];
    float4 q[127];
    float yc[127];  // the reciprocal the one-product quotient uses (when q.z > 0)
    double th[128];
};

// Whether some value with at most 8 significant bits lies within 2^-22 of
// m a for an E2M1 decision point m (a normal, a >= 2^-90).  m a is exact in
// binary64; its distance to the nearest 8-significant-bit value is the
// smaller of the 45 discarded mantissa bits and their complement, counted
// in units of 2^(e-52) for m a in [2^e, 2^(e+1)), and m a 2^-22 < 2^(e-21)
// is 2^31 such units (so the test below flags a superset).
__device__ __forceinline__ bool near_bf16_midpoint(float a) {
    const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    bool near = false;
#pragma unroll
    for (int i = 0; i < 7; ++i) {
        const uint64_t b = (uint64_t)__double_as_longlong(mids[i] * (double)a);
        const uint64_t low = b & ((1ull << 45) - 1ull);
        const uint64_t dist = low < (1ull << 44) ? low : (1ull << 45) - low;
        near = near || dist <= (1ull << 31);
    }
    return near;
}

// Exact threshold between codes k-1 and k (k in 1..126), times 6 s_g.
__device__ __forceinline__ double nv_threshold(int k, float s_g) {
    return (double)e4m3_mid6((uint32_t)k - 1u) * (double)s_g;  // exact
}

// lo[k]: the smallest fp32 amax whose code is >= k.
__device__ __forceinline__ float nv_lo(int k, float s_g) {
    if (k == 0) return 0.0f;
    if (k == 127) return __builtin_inff();
    const double th = nv_threshold(k, s_g);
    const float f = (float)th;
    const double fd = (double)f;
    // f if it is the first fp32 value reaching code k, else its successor
    return (fd > th || (fd == th && (k & 1) == 0)) ? f : u2f(f2u(f) + 1u);
}

// {alpha_c, alpha'_c, +-1/alpha'_c, sc_c} of code c in 0..126.
__device__ __forceinline__ float4 nv_divisor(int c, float s_g) {
    const float a = s_g * e4m3_pos_value((uint32_t)c);
    const float sc = a > 0.0f && a < kDivScaleBelow ? kDivScale : 1.0f;  // code 0: alpha = 0
    const float ad = a * sc;  // exact
    float y = a > 0.0f ? 1.0f / ad : 0.0f;
    if (a > 0.0f && near_bf16_midpoint(ad)) y = -y;
    return make_float4(a, ad, y, sc);
}

// recipM: for a bf16 tensor whose s_g is a normal number, the significand
// index M of its amax (low 7 bits of its bf16 pattern), else -1.  With it,
// a code's one-product quotient uses the corrected reciprocal of
// kRecipCorrection (fp4_recip_table.h: exact for every bf16 input, see the
// direct table below) and is marked only where no reciprocal fits; without
// it, the plain RN32(1/alpha') is used where no 8-significant-bit value
// comes near a decision point (near_bf16_midpoint), and the rest is marked.
__device__ __forceinline__ void nv_table_build(NvScaleTable &T, float s_g, int recipM) {
    for (int k = threadIdx.x; k < 128; k += blockDim.x) {
        T.lo[k] = nv_lo(k, s_g);
        T.th[k] = k == 0 ? -1.0 : (k == 127 ? __builtin_inf() : nv_threshold(k, s_g));
        if (k < 127) {
            float4 q = nv_divisor(k, s_g);
            float yc = __builtin_fabsf(q.z);
            if (recipM >= 0 && q.x > 0.0f && q.w == 1.0f) {
                const uint32_t sel = (kRecipCorrection[recipM & 127] >> (2u * e4m3_frac_index((uint32_t)k))) & 3u;
                q.z = sel < 3u ? yc : -yc;
                if (sel == 1u) yc = u2f(f2u(yc) - 1u);
                if (sel == 2u) yc = u2f(f2u(yc) + 1u);
            }
            T.q[k] = q;
            T.yc[k] = yc;
        }
    }
}

// Truncated E4M3 code of an approximate quotient t >= 0 (saturating);
// branch-free: the subnormal-range form reads t clamped below 2^-6.
__device__ __forceinline__ uint32_t e4m3_trunc_code(float t) {
    const uint32_t sub = (uint32_t)(__builtin_fminf(t, 0x1p-6f) * 512.0f);
    const uint32_t nrm = min((f2u(t) >> 20) - 960u, 126u);  // wraps to 126 below 2^-6
    return t < 0x1p-6f ? sub : nrm;
}

// First guess of a block's E4M3 code in fp32: t = amax * r approximates
// amax / (6 s_g) * 2^-k (relative error ~2^-23, or an absolute error far
// below the subnormal code step), with k = 64 when s_g < 2^-120 so that r
// stays a normal number; the truncated code of t 2^k is read off t's bits
// with the shift folded into the constants.
struct CodeGuess {
    float r;         // RN32(2^-k / (6 s_g))
    float sub_lim;   // 2^(-6-k): below it the code is floor(t 2^(9+k))
    float sub_mul;   // 2^(9+k)
    uint32_t bias;   // 960 - 8k: exponent-and-mantissa bits of t minus this is the code
    float cs;        // 2^-k: the FP8 converter divides by its scale's power of two
};

__device__ __forceinline__ CodeGuess make_code_guess(float s_g) {
    const bool tiny = s_g < 0x1p-120f;
    CodeGuess G;
    G.r = (float)((tiny ? 0x1p-64 : 1.0) / (6.0 * (double)s_g));
    G.sub_lim = tiny ? 0x1p-70f : 0x1p-6f;
    G.sub_mul = tiny ? 0x1p73f : 0x1p9f;
    G.bias = tiny ? 960u - 512u : 960u;
    G.cs = tiny ? 0x1p-64f : 1.0f;
    return G;
}

// E4M3 code of a nonzero finite block amax ag: nearest to the exact
// ag / (6 s_g), ties to the even code, saturating at 448.  The truncated code
// of the approximate quotient is within one code of the answer; the two exact
// thresholds around it settle it.  A zero amax gives code 0.
__device__ __forceinline__ uint32_t code_guess(float ag, const CodeGuess &G) {
    const float t = ag * G.r;
    const uint32_t sub = (uint32_t)(__builtin_fminf(t, G.sub_lim) * G.sub_mul);
    const uint32_t nrm = min((f2u(t) >> 20) - G.bias, 126u);
    return t < G.sub_lim ? sub : nrm;
}

__device__ __forceinline__ uint32_t nv_code(const NvScaleTable &T, float ag, const CodeGuess &G) {
    const uint32_t g = code_guess(ag, G);
    const float l0 = T.lo[g], l1 = T.lo[g + 1];
    return g + (uint32_t)(ag >= l1) - (uint32_t)(ag < l0);
}

// The same for a real z >= 0 exact in binary64 but not necessarily in fp32
// (a candidate multiple c * amax), against the exact binary64 thresholds.
__device__ __forceinline__ uint32_t nv_code_real(const NvScaleTable &T, double z, double inv6sg) {
    const uint32_t g = e4m3_trunc_code((float)(z * inv6sg));
    const double t0 = T.th[g], t1 = T.th[g + 1];
    if (z > t1 || (z == t1 && ((g + 1u) & 1u) == 0)) return g + 1u;
    if (z < t0 || (z == t0 && (g & 1u))) return g - 1u;
    return g;
}

// ---- the NV element divide ------------------------------------------------
// RN32(x / alpha) from y = RN32(1 / alpha): q0 = RN(x y) is within an ulp
// of x/alpha, the residual alpha q0 - x is exact in one fma, and one more
// fma gives the correctly rounded quotient (Markstein's theorem; it needs
// alpha and 1/alpha to be normal, which the caller guarantees).  Writing the
// residual with its sign flipped makes x = -0 come out as -0.
__device__ __forceinline__ float div_rn(float x, float alpha, float y) {
    float q0 = x * y;
    float rn = __builtin_fmaf(alpha, q0, -x);
    return __builtin_fmaf(-rn, y, q0);
}

// ---- direct block-scale table of the one-pass bf16 kernel ------------------
// For a bf16 tensor every block amax is a bf16 magnitude, and under one s_g
// every amax with a nonzero E4M3 code lies in a window of under 20 binades:
// from 6 s_g 2^-10 (the threshold of code 1) to the tensor amax 2688 s_g.
// The table maps each bf16 magnitude of a 20-binade window straight to its
// block's E4M3 code and divisor term, so a block scale is one LDS lookup
// indexed by the amax bits:
//   index 0      a zero block: code 0x38 (scale 1);
//   index 1      a nonzero amax below the window: code 0 (a scale underflow);
//   index 2 + i  the bf16 magnitude whose bits are base + i.
// The divisor term Y_c of code c is a reciprocal of alpha_c = RN32(s_g E4M3(c))
// for which the one product RN32(x Y_c) gives every bf16 x the E2M1 code of
// the correctly rounded quotient RN32(x / alpha_c): RN32(1 / alpha_c) or one
// of its two fp32 neighbours, as kRecipCorrection (fp4_recip_table.h, with the
// rule that chose it) gives for the amax significand M and alpha_c's
// significand 1 + k/8.  Any of the three is within 2^-21.4 of 1 / alpha_c, so
// it decides every x farther than 2^-20 from a decision point m alpha_c (m =
// 0.25, 0.75, ..., 5) as the correctly rounded quotient does; the table's
// choice also decides the bf16 values nearer to one.  Where none fits (exact
// ties x = m alpha_c, with alpha_c of few significant bits), the code takes
// the two-operation quotient fma(x, Y, x D) with Y = RD32(1 / alpha),
// D = RN32(1 / alpha - Y), exact for an alpha of at most 16 significant bits.
// A tensor whose s_g is not a normal number, or with an alpha below 2^-90
// (operands would need scaling), takes the exact compact loop instead.
constexpr int RES_NIDX = 2560;  // window entries: 20 binades of 128 bf16 magnitudes
constexpr uint32_t NV_NEEDS_TWO_OP = 1;  // some code takes fma(x, Y, x D)
constexpr uint32_t NV_NEEDS_EXACT = 2;   // some code needs the exact divide loop

struct NvDirectTable {
    float y[RES_NIDX + 2];       // Y of each entry's code (0 for code 0)
    float yc[128];               // per code: Y_c
    float dc[128];               // per code: D_c (0 where the product alone is exact)
    uint32_t lo[128];            // bf16 bits of the smallest magnitude with code >= c
    uint8_t code[RES_NIDX + 4];  // each entry's E4M3 code
    uint32_t need;               // NV_NEEDS_* of the call
};

// Bits of the largest bf16 magnitude at or below 6 s_g 2^-10, the threshold
// of E4M3 code 1 (smaller amaxes all take code 0).
__device__ __forceinline__ uint32_t nv_window_base(float s_g) {
    const double t = 6.0 * (double)s_g * 0x1p-10;  // exact
    float f = (float)t;
    if ((double)f > t) f = u2f(f2u(f) - 1u);
    return f2u(f) >> 16;
}

// Bits of the smallest bf16 magnitude whose E4M3 code under s_g is at least
// c (1 <= c <= 126): above the exact threshold 6 s_g midpoint(c - 1, c) (at
// most 31 significant bits, so exact in binary64), or on it when c is even.
__device__ __forceinline__ uint32_t nv_lo_bf16(uint32_t c, float s_g) {
    const double th = (double)e4m3_mid6(c - 1u) * (double)s_g;
    const uint32_t f = f2u((float)th);
    uint32_t b = f >> 16;
    b = b > 0u ? b - 1u : 0u;
    for (int k = 0; k < 4 && b < 0x7F80u; ++k) {
        const double v = (double)u2f(b << 16);
        if (v > th || (v == th && (c & 1u) == 0)) break;
        ++b;
    }
    return b;
}

// Builds the table in two steps (per code; per window entry) for the tensor
// scale s_g of a bf16 tensor; rcrow is kRecipCorrection's row for the tensor
// amax's significand index M (its low 7 bits).  Entry i >= 2 is the bf16
// magnitude base + i - 2; only entries 0, 1 and those in [i0, i1) are
// written (a workgroup fills those its blocks can index).  T.need must be
// zero, and a barrier passed since it was zeroed, on entry (512 threads).
// Ends with a barrier; T.need then holds the call's NV_NEEDS_*.  between()
// runs after the first step's barrier (a profiling hook; nothing otherwise).
// The first step's two halves (threads 0-127: Y_c and D_c; threads 128-255:
// the codes' lower bounds) run on different waves, side by side.
template <typename Between>
__device__ __forceinline__ void nv_direct_table_build(NvDirectTable &T, float s_g, uint32_t rcrow,
                                                      uint32_t base, int i0, int i1,
                                                      Between between) {
    const int t = threadIdx.x;
    // step 1, per code: Y_c and D_c, or the code's lower bound
    if (t < 128) {
        float Y = 0.0f, D = 0.0f;
        uint32_t need = 0;
        const float a = t > 0 && t < 127 ? s_g * e4m3_pos_value((uint32_t)t) : 0.0f;
        if (a > 0.0f) {
            const uint32_t sel = (rcrow >> (2u * e4m3_frac_index((uint32_t)t))) & 3u;
            const float y0 = 1.0f / a;  // correctly rounded
            if (a < kDivScaleBelow || s_g < 0x1p-126f) {  // outside the table's rule: exact loop
                Y = y0;
                need = NV_NEEDS_EXACT;
            } else if (sel < 3u) {
                Y = sel == 0u ? y0 : u2f(f2u(y0) + (sel == 1u ? ~0u : 1u));
            } else if ((f2u(a) & 0xFFu) == 0u) {  // at most 16 significant bits
                const double r = 1.0 / (double)a;
                float yh = (float)r;
                if ((double)yh > r) yh = u2f(f2u(yh) - 1u);
                Y = yh;
                D = (float)(r - (double)yh);
                need = NV_NEEDS_TWO_OP;
            } else {
                Y = y0;
                need = NV_NEEDS_EXACT;
            }
        }
        T.yc[t] = Y;
        T.dc[t] = D;
        if (need) atomicOr(&T.need, need);
    } else if (t < 256) {
        const uint32_t c = (uint32_t)t - 128u;
        T.lo[c] = c == 0 ? 0u : (c == 127 ? 0xFFFFu : nv_lo_bf16(c, s_g));
    }
    __syncthreads();
    between();
    // step 2, per window entry: the code of a bf16 magnitude, from a guess
    // within one code of it settled by the two bounds around it.  All of a
    // thread's reads come before its stores, so its entries' LDS round trips
    // overlap (a store between them would order every later read after it).
    // Entries 0 and 1, then those in [i0, i1), 512 per round; rounds past
    // the range are skipped (uniformly).
    constexpr int NR = (RES_NIDX + 2 + 511) / 512;
    const CodeGuess G = make_code_guess(s_g);
    uint32_t code[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (i0 + r * 512 >= i1) break;
        const int i = i0 + t + r * 512;
        const uint32_t bits = min(base + (uint32_t)(i - 2), 0x7F7Fu);  // finite
        const uint32_t g = code_guess(u2f(bits << 16), G);
        code[r] = g + (bits >= T.lo[g + 1] ? 1u : 0u) - (bits < T.lo[g] ? 1u : 0u);
    }
    float y[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (i0 + r * 512 >= i1) break;
        y[r] = T.yc[code[r]];
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (i0 + r * 512 >= i1) break;
        const int i = i0 + t + r * 512;
        if (i < i1) {
            T.code[i] = (uint8_t)code[r];
            T.y[i] = y[r];
        }
    }
    if (t < 2) {
        T.code[t] = t == 0 ? 0x38u : 0u;
        T.y[t] = T.yc[t == 0 ? 0x38 : 0];
    }
    __syncthreads();
}

// ---- wave-level helpers ---------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, WAVE));
    return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    for (int off = 32; off >= 1; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off, WAVE));
    return v;
}

// OR the calling wave's condition flags into *status with one atomic.  Safe
// in divergent code (ballot counts active lanes only).
__device__ __forceinline__ void report_flags(int32_t *status, uint32_t flags) {
    uint32_t any = 0;
    for (uint32_t bit = 1; bit <= FLAG_BARRIER_TIMEOUT; bit <<= 1)
        if (__ballot((flags & bit) != 0)) any |= bit;
    if (any == 0 || status == nullptr) return;
    uint64_t active = __ballot(1);
    if (__lane_id() == (uint32_t)__builtin_ctzll(active)) atomicOr(status, (int32_t)any);
}

// ---- grid barrier ----------------------------------------------------------
// For kernels whose workgroups are normally all resident at once (at most one
// workgroup per CU, no more workgroups than CUs), but correct when they are
// not (another kernel holding CUs, e.g. a concurrent call on another stream):
// a workgroup that does not see the barrier complete within a bounded wait
// goes on without it, by a fallback that gives the same result (reading the
// missing workgroups' inputs itself), so nothing ever waits on a workgroup
// that cannot start.
//
// The workspace keeps an epoch word and one 64-bit slot (tag << 32 | value)
// per workgroup, zeroed before the first call and left alone between calls.
// A call's workgroups read the epoch when they start and tag their slots with
// epoch + 1 (never 0).  Rules:
//   complete  (every slot carried the tag) workgroup 0 stores epoch = tag;
//   timed out the workgroup stores epoch = tag, takes the fallback, and at
//             its end retracts its slot (stores 0).
// Invariant at the start of every call: no slot carries epoch + 1.  If some
// workgroup saw the barrier complete, every workgroup had read the same epoch
// E before any store to it, all tags were E + 1 and every store writes E + 1,
// so the surviving slots carry the epoch itself.  If none did, every
// workgroup timed out and retracted its slot.  So a slot only ever matches a
// tag when it was written in the same call, with that call's value; a
// workgroup that starts after a timed-out one advanced the epoch takes a tag
// nobody else has, times out too and takes the fallback.
__device__ __forceinline__ uint32_t barrier_tag(const uint32_t *epoch) {
    const uint32_t e = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return e + 1u == 0u ? 1u : e + 1u;
}

__device__ __forceinline__ void barrier_store_epoch(uint32_t *epoch, uint32_t tag) {
    __hip_atomic_store(epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void barrier_retract(uint64_t *slots) {
    __hip_atomic_store(&slots[blockIdx.y * gridDim.x + blockIdx.x], (uint64_t)0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool barrier_slot_tagged(const uint64_t *slots, int i, uint32_t tag,
                                                    uint32_t &value) {
    const uint64_t sl = __hip_atomic_load(&slots[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    value = (uint32_t)sl;
    return (uint32_t)(sl >> 32) == tag;
}

// Called by one whole wave of every workgroup: publishes (tag, value) in this
// workgroup's slot and polls, at most spin_limit + 1 times, until every slot
// of the grid carries the tag.  Returns whether it did; A is the largest
// value among the tagged slots (and this workgroup's own), which is every
// workgroup's when it returns true.  Stores no epoch: the caller follows the
// rules above.
__device__ __forceinline__ bool grid_barrier_max(uint64_t *slots, uint32_t tag, uint32_t value,
                                                 uint32_t spin_limit, uint32_t &A) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int G = gridDim.x * gridDim.y;
    const int wg = blockIdx.y * gridDim.x + blockIdx.x;
    if (lane == 0)
        __hip_atomic_store(&slots[wg], ((uint64_t)tag << 32) | value, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    // A poll issues a lane's slot loads four at a time before it looks at
    // any: one device-coherent round trip per poll for up to 256 workgroups,
    // not one per slot.
    for (uint32_t it = 0;; ++it) {
        bool ok = true;
        uint32_t mm = 0;
        for (int i0 = 0; i0 < G; i0 += 4 * WAVE) {
            uint64_t sl[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + lane + k * WAVE;
                sl[k] = i < G ? __hip_atomic_load(&slots[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : (uint64_t)tag << 32;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool t = (uint32_t)(sl[k] >> 32) == tag;
                ok = ok && t;
                mm = t ? max(mm, (uint32_t)sl[k]) : mm;
            }
        }
        const bool all = __ballot(!ok) == 0;
        if (all || it >= spin_limit) {
            A = max(wave_max_u32(mm), value);
            return all;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

}  // namespace fp4dev
