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

constexpr int WAVE = 64;
constexpr uint32_t FLAG_NONFINITE = 1;
constexpr uint32_t FLAG_SCALE_UNDERFLOW = 2;

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

// ---- DPP lane exchange inside quads -------------------------------------
constexpr int QP_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int QP_XOR2 = 0x4E;  // quad_perm [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
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
    uint32_t r = 0;
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

// Nearest code to a finite t >= 0 (ties to even, saturating); used only as a
// first guess that an exact comparison then corrects.
__device__ __forceinline__ uint32_t e4m3_code_guess(float t) {
    if (!(t < 448.0f)) return 126u;
    if (t < 0x1p-6f) return (uint32_t)__builtin_rintf(t * 512.0f);
    uint32_t b = f2u(t);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    uint32_t c = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
    return c > 126u ? 126u : c;
}

// E4M3 code nearest to the exact real num / (6 * sg), ties to the even code,
// saturating at 448 (code 126).  num >= 0 is exact in binary64 (an fp32
// value or the product of two); inv6sg = RN64(1 / (6 sg)).
// The guess from an approximate quotient can only be wrong when the exact
// quotient sits within ~2^-50 (relative) of the midpoint nearest the guess,
// so one exact comparison with that midpoint settles it: the sign of
// num - 6m * sg from a binary64 fma is exact (a single rounding of the exact
// difference; the operands are far above the binary64 underflow range).
__device__ __forceinline__ uint32_t e4m3_code_exact(double num, double sg, double inv6sg) {
    float t = (float)(num * inv6sg);
    uint32_t c = e4m3_code_guess(t);
    if (t >= e4m3_pos_value(c)) {
        if (c < 126u) {
            double d = __builtin_fma(-(double)e4m3_mid6(c), sg, num);
            if (d > 0.0 || (d == 0.0 && (c & 1u))) c += 1u;
        }
    } else {
        double d = __builtin_fma(-(double)e4m3_mid6(c - 1u), sg, num);
        if (d < 0.0 || (d == 0.0 && (c & 1u))) c -= 1u;
    }
    return c;
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
    uint64_t n = __ballot((flags & FLAG_NONFINITE) != 0);
    uint64_t u = __ballot((flags & FLAG_SCALE_UNDERFLOW) != 0);
    if ((n | u) == 0 || status == nullptr) return;
    uint64_t active = __ballot(1);
    if (__lane_id() == (uint32_t)__builtin_ctzll(active))
        atomicOr(status, (int32_t)((n ? FLAG_NONFINITE : 0u) | (u ? FLAG_SCALE_UNDERFLOW : 0u)));
}

}  // namespace fp4dev
