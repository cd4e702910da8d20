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

__device__ __forceinline__ void nv_table_build(NvScaleTable &T, float s_g) {
    for (int k = threadIdx.x; k < 128; k += blockDim.x) {
        T.lo[k] = nv_lo(k, s_g);
        T.th[k] = k == 0 ? -1.0 : (k == 127 ? __builtin_inf() : nv_threshold(k, s_g));
        if (k < 127) T.q[k] = nv_divisor(k, s_g);
    }
}

// Compact table for the one-pass bf16 kernel.  A block scale takes two
// dependent LDS reads: the guess g's thresholds, then the final code's entry:
//   lohi[g]  = {lo[g], lo[g+1]} as fp32 bit patterns (integer order equals
//              value order for these non-negative numbers), except that
//              lo[0] is 1: a zero amax then resolves to "code" -1; and
//              lohi[127] = {~0, ~0}, which resolves the converter's NaN code
//              (a guess past 448) to 126;
//   ent[c+1] = {Y_c, D_c, c, 0} for codes c = 0..126, and ent[0] = the
//              entry of code 0x38 (scale 1), which a zero block takes;
// where, for code c,
//   in general        Y = RN32(1/alpha'_c) (0 for alpha_c = 0) and
//                     D = alpha'_c, for the reciprocal-correction divide;
//   for a short s_g   Y = RD32(1/alpha_c) and D = RN32(1/alpha_c - Y) >= 0, a
//   (<= 12 bits)      two-float reciprocal for the two-operation divide;
//   sa[c] = {alpha'_c, sc_c}, always, for the compact full-divide pass.
// lo is staged in the last array.
struct NvGuessTable {
    uint2 lohi[128];
    float4 ent[128];
    float2 sa[127];
    float lo[127];
};

// An s_g with at most 12 significant bits: every alpha_c = s_g E4M3(c) then
// has at most 16, which the two-operation divide needs.
__device__ __forceinline__ bool short_tensor_scale(float s_g) {
    return s_g >= 0x1p-126f && (f2u(s_g) & 0xFFFu) == 0;
}

__device__ __forceinline__ float nv_signed_recip(int c, float s_g) {
    const float4 q = nv_divisor(c, s_g);
    return q.w != 1.0f ? -__builtin_fabsf(q.z) : q.z;
}

// Builds the table in two steps over the workgroup (per code, then per
// guess); returns to every thread whether some code needs operand scaling.
// Ends with a barrier.
__device__ __forceinline__ bool nv_guess_table_build(NvGuessTable &R, float s_g) {
    int scaled = 0;
    const int t = threadIdx.x;
    const bool shrt = short_tensor_scale(s_g);
    // step 1: per code c, sa[c] and ent[c + 1]; lo[k]
    if (t < 127) {
        const float a = s_g * e4m3_pos_value((uint32_t)t);
        const float sc = a > 0.0f && a < kDivScaleBelow ? kDivScale : 1.0f;  // code 0: alpha = 0
        const float ad = a * sc;  // exact
        float Y = a > 0.0f ? 1.0f / ad : 0.0f, D = ad;
        if (shrt && a > 0.0f) {
            // RD32 and the (non-negative) remainder of 1 / alpha
            const double r = 1.0 / (double)a;
            float yh = (float)r;
            if ((double)yh > r) yh = u2f(f2u(yh) - 1u);
            Y = yh;
            D = (float)(r - (double)yh);
        }
        R.sa[t] = make_float2(ad, sc);
        R.ent[t + 1] = make_float4(Y, D, u2f((uint32_t)t), 0.0f);
        if (t == 0x38) R.ent[0] = make_float4(Y, D, u2f(0x38u), 0.0f);
        scaled = sc != 1.0f;
    } else if (t >= 128 && t < 128 + 127) {
        R.lo[t - 128] = nv_lo(t - 128, s_g);
    }
    __syncthreads();
    // step 2: threshold pairs per guess g
    if (t < 127)
        R.lohi[t] = make_uint2(t == 0 ? 1u : f2u(R.lo[t]), t < 126 ? f2u(R.lo[t + 1]) : 0x7F800000u);
    else if (t == 127)
        R.lohi[t] = make_uint2(~0u, ~0u);
    return __syncthreads_or(scaled) != 0;
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

// The same guess from the FP8 converter: the E4M3 code of t 2^k rounded to
// nearest even (it divides t by its scale's power of two and keeps
// subnormals; past 464 it gives the NaN code 127, which a table must map to
// 126).  Within one code of the exact one, like the truncated guess.  The
// converter writes the low two bytes (t's code, then 0.0's) over t's own bits.
__device__ __forceinline__ uint32_t code_guess_cvt(float ag, const CodeGuess &G) {
    typedef short v2i16 __attribute__((ext_vector_type(2)));
    const float t = ag * G.r;
    const v2i16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2i16, t), t, 0.0f,
                                                             G.cs, false);
    return __builtin_bit_cast(uint32_t, r) & 0xFFu;
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

// ---- wave-level helpers ---------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, WAVE));
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
// For kernels whose whole grid is resident at once (at most one workgroup
// per CU, no more workgroups than CUs).  The workspace keeps an epoch word
// and one 64-bit slot per workgroup, zeroed before the first call and left
// alone between calls.  Each call tags its slots with epoch + 1 (never 0),
// read by every workgroup before any can pass the barrier; workgroup 0
// stores the new epoch once it has passed, for the next call in stream order.
__device__ __forceinline__ uint32_t barrier_tag(const uint32_t *epoch) {
    const uint32_t e = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return e + 1u == 0u ? 1u : e + 1u;
}

// Called by one whole wave of every workgroup: publishes (tag, value) in
// this workgroup's slot and polls until every slot of the grid carries the
// tag; returns the largest value.  A bounded wait: after spin_limit polls it
// sets FLAG_BARRIER_TIMEOUT in flags and returns what it has, never less than
// its own value (so a workgroup's own amax stays within the scale it uses).
__device__ __forceinline__ uint32_t grid_barrier_max(uint64_t *slots, uint32_t *epoch, uint32_t tag,
                                                     uint32_t value, uint32_t spin_limit,
                                                     uint32_t &flags) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int G = gridDim.x * gridDim.y;
    const int wg = blockIdx.y * gridDim.x + blockIdx.x;
    if (lane == 0)
        __hip_atomic_store(&slots[wg], ((uint64_t)tag << 32) | value, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    uint32_t A = 0;
    for (uint32_t it = 0;; ++it) {
        bool ok = true;
        uint32_t mm = 0;
        for (int i = lane; i < G; i += WAVE) {
            const uint64_t sl = __hip_atomic_load(&slots[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = ok && (uint32_t)(sl >> 32) == tag;
            mm = max(mm, (uint32_t)sl);
        }
        const bool all = __ballot(!ok) == 0;
        if (all || it >= spin_limit) {
            if (!all) flags |= FLAG_BARRIER_TIMEOUT;
            A = max(wave_max_u32(mm), value);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0 && wg == 0)
        __hip_atomic_store(epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return A;
}

}  // namespace fp4dev
