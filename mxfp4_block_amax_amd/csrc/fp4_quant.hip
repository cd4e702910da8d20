// fp4_quant.hip - MXFP4 / NVFP4 quantize, dequantize and MSE scale search
// kernels for gfx950.
//
// Data layout.  The input is treated as a flat sequence of E elements (every
// row holds whole blocks), cut into 16-byte "chunks" of 8 elements for bf16
// input (32 bytes for fp32).  Lane l of a wave owns chunk  tile*64*U + r*64 + l
// for r < U, so every load instruction of a wave reads 1 KiB of consecutive
// bf16 bytes and every code store writes 256 consecutive bytes.  Blocks are
// consecutive lanes: an NVFP4 block (16 elements) is a lane pair, an MXFP4
// block (32) a lane quad, and the block amax is finished with DPP quad
// permutes.  Scales are stored by one lane per block.
//
// Method ("NVFP4 / MXFP4 format" page, charlestar.github.io):
//   MXFP4 (sections 2 and 5): E8M0 exponent by the OCP floor rule,
//     e = floor(log2 amax) - 2, elements divided by 2^e and rounded to E2M1.
//   NVFP4 (section 3): s_g = A / 2688, s_b = E4M3(A_g / (6 s_g)) encoded before
//     it quantizes, alpha = RN32(s_g * s_b), q = RN32(x / alpha) -> E2M1.
//   Zero/tiny contract (section 3): an all-zero tensor takes s_g = 1, a zero
//     block takes s_b = 1 (0x38); a nonzero block whose s_b or alpha is 0, or
//     an s_g that underflows, raises FP4_FLAG_SCALE_UNDERFLOW.
// Scale search ("FP4 / NVFP4 math summary" page, devpress.csdn.net, section 9):
//   per block, the candidate E4M3 scale with the least fp32 squared error.
#include <mutex>
#include <type_traits>

#include "fp4_device.h"
#include "fp4_kernels.h"

namespace fp4dev {

constexpr int WG = 256;
constexpr int WAVES_PER_WG = WG / WAVE;

// ---------------------------------------------------------------------------
// chunk loads
// ---------------------------------------------------------------------------
template <bool BF16>
struct Chunk {
    uint4 lo, hi;  // hi used only for fp32 input
};

// STREAM: data read once (non-temporal); otherwise ordinary loads that may
// allocate in the caches, for data a second pass reads again.  fp32 input
// defaults to ordinary loads: a lane's chunk is two 16-byte loads 32 bytes
// apart, so each load instruction touches every line of its span for half
// of its bytes; non-temporal loads did not keep the line for the other half
// and it was fetched twice (measured: 8192 x 8192 fp32 MXFP4 quantize 67.0 ->
// 58.6 us, NVFP4 132 -> 107 us).
template <bool BF16, bool STREAM = BF16>
__device__ __forceinline__ Chunk<BF16> load_chunk(const uint4 *__restrict__ x, int64_t c, bool ok) {
    Chunk<BF16> k;
    const uint4 z = make_uint4(0, 0, 0, 0);
    if (BF16) {
        k.lo = ok ? (STREAM ? ld_stream(x + c) : x[c]) : z;
        k.hi = z;
    } else {
        k.lo = ok ? (STREAM ? ld_stream(x + 2 * c) : x[2 * c]) : z;
        k.hi = ok ? (STREAM ? ld_stream(x + 2 * c + 1) : x[2 * c + 1]) : z;
    }
    return k;
}

template <bool BF16>
__device__ __forceinline__ uint32_t chunk_amax(const Chunk<BF16> &k) {
    return BF16 ? amax_bf16x8(k.lo) : amax_f32x8(k.lo, k.hi);
}

// fp32 bit pattern of a chunk-amax pattern
template <bool BF16>
__device__ __forceinline__ uint32_t amax_as_f32_bits(uint32_t m) {
    return BF16 ? (m << 16) : m;
}

template <bool BF16>
__device__ __forceinline__ void chunk_values(const Chunk<BF16> &k, float (&v)[8]) {
    if (BF16) widen_bf16x8(k.lo, v);
    else widen_f32x8(k.lo, k.hi, v);
}

// ---------------------------------------------------------------------------
// MXFP4 quantize: one pass.  RULE picks the block exponent (format page,
// section 5: the format fixes the scale set, not the rule):
//   0  the OCP floor rule, e = floor(log2 amax) - 2;
//   1  the ceil rule, the smallest e with 6 * 2^e >= amax;
//   2  a squared-error search over e0 - 1, e0, e0 + 1 around the floor
//      rule's e0: e0 stays unless a neighbour has a strictly smaller fp32
//      loss (e0 - 1 tried first); exponents below -127 are not candidates.
// ---------------------------------------------------------------------------

// Codes of this lane's 8 values at E8M0 scale byte sb, and their squared
// error summed pairwise in index order: q = x / 2^e rounded to E2M1 by the
// converter, x_hat = E2M1(q) 2^e exactly, err = RN32(x - x_hat).
struct MxTry {
    uint32_t code;
    float loss;
};
__device__ __forceinline__ MxTry mx_try(const float (&v)[8], uint32_t sb) {
    const float so = e8m0_operand(sb);
    MxTry r;
    r.code = cvt_fp4x8_f32(v, so);
    float t[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x2_t p;
        switch (j) {  // the byte selector must be a constant
            case 0: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.code, so, 0); break;
            case 1: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.code, so, 1); break;
            case 2: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.code, so, 2); break;
            default: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.code, so, 3); break;
        }
        const float e0 = v[2 * j] - p.x, e1 = v[2 * j + 1] - p.y;
        t[2 * j] = e0 * e0;
        t[2 * j + 1] = e1 * e1;
    }
    const float part = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    // the block's four lanes: (L0 + L1) + (L2 + L3), the pairwise tree over 32
    const float pair = part + dppf<QP_XOR1>(part);
    r.loss = pair + dppf<QP_XOR2>(pair);
    return r;
}

template <bool BF16, int RULE>
__global__ __launch_bounds__(WG) void mx_quantize_kernel(const uint4 *__restrict__ x,
                                                         int64_t nchunks,
                                                         uint32_t *__restrict__ codes,
                                                         uint8_t *__restrict__ scales,
                                                         int32_t *status) {
    constexpr int U = 4;
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_WG + (threadIdx.x / WAVE);
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    const int64_t ntiles = (nchunks + WAVE * U - 1) / (WAVE * U);
    uint32_t flags = 0;
    for (int64_t t = wave; t < ntiles; t += nwaves) {
        Chunk<BF16> k[U];
#pragma unroll
        for (int r = 0; r < U; ++r) {
            int64_t c = t * (WAVE * U) + r * WAVE + lane;
            k[r] = load_chunk<BF16>(x, c, c < nchunks);
        }
#pragma unroll
        for (int r = 0; r < U; ++r) {
            int64_t c = t * (WAVE * U) + r * WAVE + lane;
            uint32_t m = chunk_amax<BF16>(k[r]);
            m = max(m, dpp<QP_XOR1>(m));
            m = max(m, dpp<QP_XOR2>(m));
            const int sh = BF16 ? 7 : 23;
            if ((m >> sh) >= 0xFFu) flags |= FLAG_NONFINITE;
            uint32_t sb = RULE == 1 ? mx_scale_byte_ceil(m, sh) : mx_scale_byte(m, sh);
            uint32_t q;
            if (RULE == 2) {
                float v[8];
                chunk_values<BF16>(k[r], v);
                const MxTry t0 = mx_try(v, sb);
                const MxTry tp = mx_try(v, sb + 1u);
                const MxTry tm = mx_try(v, sb > 0u ? sb - 1u : sb);
                q = t0.code;
                float best = t0.loss;
                uint32_t nb = sb;
                if (sb > 0u && tm.loss < best) {
                    best = tm.loss;
                    q = tm.code;
                    nb = sb - 1u;
                }
                if (tp.loss < best) {
                    q = tp.code;
                    nb = sb + 1u;
                }
                sb = nb;
            } else if (BF16) {
                q = cvt_fp4x8_bf16(k[r].lo, e8m0_operand(sb));
            } else {
                float v[8];
                chunk_values<BF16>(k[r], v);
                q = cvt_fp4x8_f32(v, e8m0_operand(sb));
            }
            if (c < nchunks) {
                codes[c] = q;
                if ((lane & 3) == 0) scales[c >> 2] = (uint8_t)sb;
            }
        }
    }
    report_flags(status, flags);
}

// ---------------------------------------------------------------------------
// MXFP4 quantize (OCP floor rule) written in MFMA operand order (the packed
// operand layout of the packed GEMM).  One wave per 1 KB code tile (row
// tile rt, K step ks): lane l quantizes block 2 ks + l / 32 of row
// 32 rt + l % 32 (32 values, its own amax) and stores its 16 code bytes at
// byte 16 l of the tile, so a wave writes one contiguous kilobyte; the
// scale byte goes to byte 8 l + ks % 8 of the tile's scale group ks / 8.
// Rows past the tensor read as zeros, whose blocks encode as the layout's
// padding (codes 0, scale byte 127).
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(WG) void mx_quantize_packed_kernel(const uint4 *__restrict__ x,
                                                                int64_t rows, int64_t K,
                                                                int64_t ntiles,
                                                                uint4 *__restrict__ codes,
                                                                uint8_t *__restrict__ scales,
                                                                int32_t *status) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_WG + (threadIdx.x / WAVE);
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    const int64_t nks = K / 64;
    uint32_t flags = 0;
    for (int64_t t = wave; t < ntiles; t += nwaves) {
        const int64_t rt = t / nks, ks = t % nks;
        const int64_t row = rt * 32 + (lane & 31);
        const bool ok = row < rows;
        // chunk index (8 values) of the block's first chunk
        const int64_t c0 = (row * K + (2 * ks + (lane >> 5)) * 32) / 8;
        Chunk<BF16> k[4];
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            k[i] = load_chunk<BF16>(x, c0 + i, ok);
            m = max(m, chunk_amax<BF16>(k[i]));
        }
        const int sh = BF16 ? 7 : 23;
        if ((m >> sh) >= 0xFFu) flags |= FLAG_NONFINITE;
        const uint32_t sb = mx_scale_byte(m, sh);
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (BF16) {
                q[i] = cvt_fp4x8_bf16(k[i].lo, e8m0_operand(sb));
            } else {
                float v[8];
                chunk_values<BF16>(k[i], v);
                q[i] = cvt_fp4x8_f32(v, e8m0_operand(sb));
            }
        }
        codes[t * 64 + lane] = make_uint4(q[0], q[1], q[2], q[3]);
        scales[((rt * (nks / 8) + ks / 8) * 64 + lane) * 8 + ks % 8] = (uint8_t)sb;
    }
    report_flags(status, flags);
}

// ---------------------------------------------------------------------------
// Stochastic element rounding (Ultralytics glossary "FP4", section
// "Inferenza e addestramento FP4": NVFP4 pretraining rounds gradients
// stochastically; the pages give no rule).  The quotient q is the
// deterministic encoder's; |q| rounds to the E2M1 magnitude below (lo) or
// above (hi) it, up with probability (|q| - lo) / (hi - lo) at 24-bit
// resolution: with r the element's 24 random bits, up iff
// r 2^-24 (hi - lo) < |q| - lo.  Both sides are exact in fp32 (r < 2^24,
// hi - lo a power of two, |q| - lo exact by Sterbenz), so the decision is
// exact.  Grid values never move, |q| >= 6 saturates, the sign is kept.
//
// Random bits: SplitMix64 (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014) evaluated at the counter
// seed + (i/2 + 1) 0x9E3779B97F4A7C15 for flat element index i, i.e. the
// (i/2 + 1)-th output of the generator started at state seed; element i
// takes the top 24 bits of the low (even i) or high (odd i) 32-bit half.
// Every element's bits depend on its index alone, so any grid, tiling or
// chunking gives the same codes.
//
// gfx950 also converts with stochastic rounding in hardware
// (v_cvt_scalef32_sr_pk_fp4_*), but how it consumes its random operand is
// not published, so the rounding is done here in VALU arithmetic and the
// converter only encodes the chosen (exact) grid value.
// ---------------------------------------------------------------------------
constexpr uint64_t kSplitMixGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t splitmix64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// The E2M1 grid value |q| rounds to, with q's sign, given 24 random bits r.
// |q| is clamped to 6 first (6 is a grid value, so it then stays).  For
// |q| >= 1, lo keeps the exponent and the top mantissa bit of |q| and hi - lo
// is half the exponent's power of two; below 1 the grid step is 0.5.  A NaN
// comes out as +-6 (its input is flagged non-finite).
__device__ __forceinline__ float sr_e2m1_value(float q, uint32_t r) {
    const float m = __builtin_fminf(__builtin_fabsf(q), 6.0f);
    const uint32_t b = f2u(m);
    const bool big = m >= 1.0f;
    const float lo = big ? u2f(b & 0xFFC00000u) : (m >= 0.5f ? 0.5f : 0.0f);
    const float gap = big ? u2f((b & 0x7F800000u) - 0x00800000u) : 0.5f;
    const float t = (float)r * 0x1p-24f * gap;  // exact
    const float v = t < m - lo ? lo + gap : lo;
    return __builtin_copysignf(v, q);
}

// Packed E2M1 codes of chunk c (elements 8c .. 8c+7, quotients q[0..7]).
__device__ __forceinline__ uint32_t sr_codes8(const float (&q)[8], uint64_t seed, int64_t c) {
    float v[8];
    uint64_t ctr = seed + (uint64_t)(4 * c + 1) * kSplitMixGamma;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint64_t z = splitmix64_mix(ctr);
        ctr += kSplitMixGamma;
        // the top 24 bits of each 32-bit half; the empty asm hides the
        // halves' origin so the conversion to float stays a 32-bit one (the
        // optimiser would otherwise convert z >> 40 as a 64-bit integer)
        uint32_t lo = (uint32_t)z, hi = (uint32_t)(z >> 32);
        asm volatile("" : "+v"(lo), "+v"(hi));
        v[2 * j] = sr_e2m1_value(q[2 * j], lo >> 8);
        v[2 * j + 1] = sr_e2m1_value(q[2 * j + 1], hi >> 8);
    }
    return cvt_fp4x8_f32(v, e8m0_operand(E8M0_ONE));  // exact: grid values
}

// MXFP4 quantize with stochastic rounding: block exponents by the OCP floor
// rule, q = x / 2^e (exact: a multiply by 2^-e, which is normal for every
// finite block since e <= 125), then the stochastic grid value.
template <bool BF16>
__global__ __launch_bounds__(WG) void mx_quantize_sr_kernel(const uint4 *__restrict__ x,
                                                            int64_t nchunks, uint64_t seed,
                                                            uint32_t *__restrict__ codes,
                                                            uint8_t *__restrict__ scales,
                                                            int32_t *status) {
    constexpr int U = 4;
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_WG + (threadIdx.x / WAVE);
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    const int64_t ntiles = (nchunks + WAVE * U - 1) / (WAVE * U);
    uint32_t flags = 0;
    for (int64_t t = wave; t < ntiles; t += nwaves) {
        Chunk<BF16> k[U];
#pragma unroll
        for (int r = 0; r < U; ++r) {
            int64_t c = t * (WAVE * U) + r * WAVE + lane;
            k[r] = load_chunk<BF16>(x, c, c < nchunks);
        }
#pragma unroll
        for (int r = 0; r < U; ++r) {
            int64_t c = t * (WAVE * U) + r * WAVE + lane;
            uint32_t m = chunk_amax<BF16>(k[r]);
            m = max(m, dpp<QP_XOR1>(m));
            m = max(m, dpp<QP_XOR2>(m));
            const int sh = BF16 ? 7 : 23;
            if ((m >> sh) >= 0xFFu) flags |= FLAG_NONFINITE;
            const uint32_t sb = mx_scale_byte(m, sh);
            const float inv = u2f((254u - sb) << 23);  // 2^-e
            float v[8];
            chunk_values<BF16>(k[r], v);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] *= inv;
            const uint32_t q = sr_codes8(v, seed, c);
            if (c < nchunks) {
                codes[c] = q;
                if ((lane & 3) == 0) scales[c >> 2] = (uint8_t)sb;
            }
        }
    }
    report_flags(status, flags);
}

// ---------------------------------------------------------------------------
// Tensor amax (NVFP4 and scale search, pass 1): one partial max of the
// sign-cleared bit patterns per workgroup.  No atomics, no initialisation.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(WG) void tensor_amax_kernel(const uint4 *__restrict__ x,
                                                         int64_t nchunks,
                                                         uint32_t *__restrict__ partials) {
    constexpr int U = 4;
    __shared__ uint32_t red[WAVES_PER_WG];
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * WG;
    for (int64_t c0 = (int64_t)blockIdx.x * WG + threadIdx.x; c0 < nchunks; c0 += stride * U) {
        Chunk<BF16> k[U];
#pragma unroll
        for (int r = 0; r < U; ++r) {
            int64_t c = c0 + r * stride;
            k[r] = load_chunk<BF16>(x, c, c < nchunks);
        }
#pragma unroll
        for (int r = 0; r < U; ++r) m = max(m, chunk_amax<BF16>(k[r]));
    }
    m = wave_max_u32(m);
    if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
        for (int i = 1; i < WAVES_PER_WG; ++i) r = max(r, red[i]);
        partials[blockIdx.x] = r;
    }
}

// Reduce the pass-1 partials (every workgroup does it; the array is tiny and
// L2-resident) and derive the tensor scale s_g = RN32(A / 2688), 1 for an
// all-zero tensor ("NVFP4 / MXFP4 format" page, section 3).
struct TensorScale {
    float s_g;
    uint32_t flags;
    uint32_t amax;  // fp32 bits of the tensor amax
};

// kRecipCorrection's row for a tensor (see nv_table_build), or -1.
template <bool BF16>
__device__ __forceinline__ int recip_row(const TensorScale &ts) {
    return BF16 && ts.s_g >= 0x1p-126f ? (int)((ts.amax >> 16) & 127u) : -1;
}

// s_g from the fp32 bit pattern of the tensor amax.
__device__ __forceinline__ TensorScale scale_from_amax(uint32_t A) {
    TensorScale ts;
    ts.flags = 0;
    ts.amax = A;
    if (A >= 0x7F800000u) {
        ts.flags = FLAG_NONFINITE;
        ts.s_g = 1.0f;
        return ts;
    }
    ts.s_g = (A == 0) ? 1.0f : u2f(A) / 2688.0f;  // correctly rounded fp32 divide
    if (ts.s_g == 0.0f) ts.flags = FLAG_SCALE_UNDERFLOW;
    return ts;
}

template <bool BF16>
__device__ TensorScale tensor_scale(const uint32_t *__restrict__ partials, int npart) {
    __shared__ uint32_t red[WAVES_PER_WG];
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npart; i += WG) m = max(m, partials[i]);
    m = wave_max_u32(m);
    if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = m;
    __syncthreads();
    m = red[0];
    for (int i = 1; i < WAVES_PER_WG; ++i) m = max(m, red[i]);
    return scale_from_amax(amax_as_f32_bits<BF16>(m));
}

// Per-block NVFP4 scale from the workgroup's table: the E4M3 code and the
// divide operands alpha', +-1/alpha', sc (x / alpha is done as
// (x sc) / alpha'; a negative reciprocal marks a scale whose one-multiply
// quotient may differ for some bf16 input), and yc, the reciprocal of the
// one-multiply quotient.  A zero block takes scale 1 (code 0x38).
struct BlockScale {
    float a, ad, y, sc;  // a: alpha itself
    float yc;
    uint32_t code;
};

__device__ __forceinline__ BlockScale nv_block_scale(const NvScaleTable &T, uint32_t ag_bits,
                                                     const CodeGuess &G, uint32_t &flags) {
    BlockScale b;
    const uint32_t c = nv_code(T, u2f(ag_bits), G);  // 0 for a zero amax
    b.code = ag_bits == 0 ? 0x38u : c;
    const float4 q = T.q[b.code];
    b.a = q.x;
    b.ad = q.y;
    b.y = q.z;
    b.sc = q.w;
    b.yc = T.yc[b.code];
    const bool under = (ag_bits != 0 && c == 0) || q.z == 0.0f;
    flags |= under ? FLAG_SCALE_UNDERFLOW : 0u;
    return b;
}

// x scaled by sc in place; sc is 1 except in tensors whose s_g is tiny, so the
// multiply sits behind a wave-uniform branch.
__device__ __forceinline__ void scale_values(float (&v)[8], float sc) {
    if (__ballot(sc != 1.0f)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= sc;
    }
}

// E2M1 codes of 8 values divided by alpha, the fp32 correctly rounded
// quotient, given alpha' = alpha sc, ys = +-RN32(1 / alpha'), sc and yc.
// BF16: the inputs have at most 8 significant bits, so unless some lane's
// scale is marked (ys < 0) the product with yc decides the same codes.
template <bool BF16>
__device__ __forceinline__ uint32_t nv_quant8(float (&v)[8], float ad, float ys, float sc,
                                              float yc) {
    scale_values(v, sc);
    const float y = __builtin_fabsf(ys);
    float q[8];
    if (BF16 && !__ballot(ys < 0.0f)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = v[i] * yc;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = div_rn(v[i], ad, y);
    }
    return cvt_fp4x8_f32(q, e8m0_operand(E8M0_ONE));
}

// Stochastic NVFP4 codes of 8 values with block scale alpha.  The quotient
// must be RN32(x / alpha) for every size of it (the decision reads it down to
// 2^-25, and below that whether it is zero).  It is taken as
// RN32(RN64(x * RN64(1 / alpha))): within 2^-52 (relative) of x / alpha, while
// for a normal quotient no fp32 rounding boundary lies closer than 2^-49
// (x - alpha m, m a midpoint, is a nonzero multiple of 2^(ea + eq - 47)), so the
// fp32 result is exact.  Below 2^-100 only zero versus nonzero matters, and
// RN32(x / alpha) is zero exactly when |x| <= alpha 2^-150, a comparison done
// exactly in fp64 (a wave-uniform branch, taken only for such tiny
// quotients).  alpha = 0 (a flagged scale underflow) gives zero quotients.
__device__ __forceinline__ uint32_t nv_sr8(const float (&v)[8], float alpha, uint64_t seed,
                                           int64_t c) {
    float q[8];
    const double ra = 1.0 / (double)alpha;
    bool tiny = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double p = (double)v[i] * ra;
        q[i] = (float)p;
        tiny |= v[i] != 0.0f && __builtin_fabs(p) < 0x1p-100;
    }
    if (__ballot(tiny)) {
        const double z = (double)alpha * 0x1p-150;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double p = (double)v[i] * ra;
            if (__builtin_fabs(p) < 0x1p-100)
                q[i] = __builtin_copysignf(__builtin_fabs((double)v[i]) > z ? 0x1p-149f : 0.0f, v[i]);
        }
    }
    if (alpha == 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = 0.0f;
    }
    return sr_codes8(q, seed, c);
}

// ---------------------------------------------------------------------------
// NVFP4 quantize, pass 2.  Each wave tile is two chunk-rows; a lane pair holds
// one block of each row.  The even lane derives row 0's block scale and the
// odd lane row 1's, and they swap results, so no block scale is computed
// twice.  SR: stochastic element rounding with the given seed (block scales
// and s_g unchanged).
// ---------------------------------------------------------------------------
template <bool BF16, bool SR>
__global__ __launch_bounds__(WG) void nv_quantize_kernel(const uint4 *__restrict__ x,
                                                         int64_t nchunks,
                                                         const uint32_t *__restrict__ partials,
                                                         int npart, uint64_t seed,
                                                         uint32_t *__restrict__ codes,
                                                         uint8_t *__restrict__ scales,
                                                         float *__restrict__ global_scale,
                                                         int32_t *status) {
    constexpr int U = 2;
    __shared__ NvScaleTable T;
    TensorScale ts = tensor_scale<BF16>(partials, npart);
    if (blockIdx.x == 0 && threadIdx.x == 0) *global_scale = ts.s_g;
    if (ts.flags) {  // uniform over the grid: outputs unspecified
        if (blockIdx.x == 0 && threadIdx.x == 0 && status) atomicOr(status, (int32_t)ts.flags);
        return;
    }
    nv_table_build(T, ts.s_g, recip_row<BF16>(ts));
    __syncthreads();
    const CodeGuess G = make_code_guess(ts.s_g);
    const int lane = threadIdx.x & (WAVE - 1);
    const bool odd = lane & 1;
    const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_WG + (threadIdx.x / WAVE);
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    const int64_t ntiles = (nchunks + WAVE * U - 1) / (WAVE * U);
    uint32_t flags = 0;
    for (int64_t tt = wave; tt < ntiles; tt += nwaves) {
        // fp32: back to front.  The amax pass read the input front to back,
        // so its tail is what the memory-side cache still holds when the
        // input is larger than that cache (8192 x 8192 fp32: 268 MB;
        // 100.8 -> 96.5 us per call, paired timing).
        const int64_t t = BF16 ? tt : ntiles - 1 - tt;
        const int64_t c0 = t * (WAVE * U) + lane, c1 = c0 + WAVE;
        Chunk<BF16> k0 = load_chunk<BF16>(x, c0, c0 < nchunks);
        Chunk<BF16> k1 = load_chunk<BF16>(x, c1, c1 < nchunks);
        uint32_t m0 = chunk_amax<BF16>(k0), m1 = chunk_amax<BF16>(k1);
        m0 = max(m0, dpp<QP_XOR1>(m0));
        m1 = max(m1, dpp<QP_XOR1>(m1));
        BlockScale mine = nv_block_scale(T, amax_as_f32_bits<BF16>(odd ? m1 : m0), G, flags);
        const float pa = dppf<QP_XOR1>(mine.ad), py = dppf<QP_XOR1>(mine.y),
                    ps = dppf<QP_XOR1>(mine.sc), pc = dppf<QP_XOR1>(mine.yc);
        // row 0 uses the even lane's scale, row 1 the odd lane's
        const float a0 = odd ? pa : mine.ad, y0 = odd ? py : mine.y, s0 = odd ? ps : mine.sc;
        const float a1 = odd ? mine.ad : pa, y1 = odd ? mine.y : py, s1 = odd ? mine.sc : ps;
        const float c0y = odd ? pc : mine.yc, c1y = odd ? mine.yc : pc;
        float v[8];
        uint32_t q0, q1;
        if (SR) {
            const float pal = dppf<QP_XOR1>(mine.a);
            chunk_values<BF16>(k0, v);
            q0 = nv_sr8(v, odd ? pal : mine.a, seed, c0);
            chunk_values<BF16>(k1, v);
            q1 = nv_sr8(v, odd ? mine.a : pal, seed, c1);
        } else {
            chunk_values<BF16>(k0, v);
            q0 = nv_quant8<BF16>(v, a0, y0, s0, c0y);
            chunk_values<BF16>(k1, v);
            q1 = nv_quant8<BF16>(v, a1, y1, s1, c1y);
        }
        if (c0 < nchunks) codes[c0] = q0;
        if (c1 < nchunks) codes[c1] = q1;
        const int64_t cs = odd ? c1 : c0;  // chunk whose block this lane's scale belongs to
        if (cs < nchunks) scales[cs >> 1] = (uint8_t)mine.code;
    }
    report_flags(status, flags);
}

// ---------------------------------------------------------------------------
// NVFP4 quantize of a bf16 tensor in one pass, the tensor held on chip.
//
// s_g needs the amax of the whole tensor before any block can be quantized,
// so the two-pass path reads the input from HBM twice.  Here one workgroup
// per CU (8 waves, two per SIMD) loads its slice once: up to 64 chunks of 16
// bytes per lane, the first RES_LDS_CHUNKS of them straight into LDS (the
// global->LDS load path; 144 KiB per workgroup, beside the ~14 KiB scale
// table) and the rest into VGPRs (184 registers).  It takes its partial
// amax, meets the other workgroups at a grid barrier and quantizes from
// registers and LDS.  256 CUs hold 128 MiB of bf16 this way, an 8192 x 8192
// tensor.
//
// Chunk j of lane t in workgroup w of G is  j*G*512 + w*512 + t  (rows j of
// all workgroups side by side), so each wave load reads 1 KiB of consecutive
// bytes, a lane pair holds one 16-element block, and rows j and j+1 pair up
// as in the two-pass kernel (even lane: row j's block scale, odd lane: row
// j+1's).  Loads past the end of the tensor re-read its last chunk (a
// duplicate cannot change the amax); stores past it are skipped.
//
// Grid barrier (grid_barrier_max).  Each workgroup publishes (tag << 32 |
// partial amax) in its own 64-bit slot with one device-coherent store, then
// polls every slot with device-coherent loads until all carry the tag.  The
// launcher starts this kernel only when one workgroup per CU fits and the
// grid is at most the CU count, so the workgroups are normally resident
// together.  When they are not (a concurrent kernel holds CUs), a workgroup
// stops waiting after spin_limit polls and takes the tensor amax itself: the
// tagged slots' values plus the amax of every other slice, read from x.  The
// result is the same; FLAG_BARRIER_TIMEOUT records that it happened.
// ---------------------------------------------------------------------------
// Amax bits (bf16 magnitude) of the block this lane derives the scale of,
// given its chunk amaxes m0 (row 0) and m1 (row 1): the even lane takes row
// 0's block and the odd lane row 1's; each lane also hands its partner its
// share of the partner's block.
__device__ __forceinline__ uint32_t pair_amax(uint32_t m0, uint32_t m1, bool odd) {
    const uint32_t own = odd ? m1 : m0, other = odd ? m0 : m1;
    return max(own, dpp<QP_XOR1>(other));
}

// Row 0's and row 1's Y for a tile of two chunk rows held by a lane pair
// (the even lane looked up row 0's block, the odd lane row 1's).
__device__ __forceinline__ void pair_rows(float v, float (&rows)[2]) {
    rows[0] = dppf<0xA0>(v);  // quad_perm [0,0,2,2]
    rows[1] = dppf<0xF5>(v);  // quad_perm [1,1,3,3]
}

constexpr int RES_WG = 512;
constexpr int RES_WAVES = RES_WG / WAVE;
constexpr int RES_LDS_CHUNKS = 18;
constexpr int RES_MAX_CHUNKS = 64;


typedef __attribute__((address_space(1))) const void *global_cptr;
typedef __attribute__((address_space(3))) void *lds_ptr;

// Tensor amax of a bf16 tensor by one large workgroup per CU (the grid of
// the one-pass quantize, no barrier): each lane issues all of its CPL chunk
// loads at once, the first RES_LDS_CHUNKS into LDS and the rest into VGPRs,
// then reduces.  Row j of the grid is one contiguous span of G*512 chunks
// dealt out in 512-byte pieces, piece (t / 32) G + w to lanes 32 (t / 32) ..
// + 31 of workgroup w, so an XCD's pieces are 512 bytes of every 4 KiB (the
// spread at which the XCDs' loads finish closest together).  Loads past the
// end re-read the lane's chunk of row 0 (a duplicate cannot change the max;
// the launcher keeps row 0 inside the tensor).  Writes one partial per
// workgroup, as tensor_amax_kernel does.
template <int CPL>
__global__ __launch_bounds__(RES_WG) void tensor_amax_wide_kernel(const uint4 *__restrict__ x,
                                                                  int64_t nchunks,
                                                                  uint32_t *__restrict__ partials) {
    constexpr int LC = CPL < RES_LDS_CHUNKS ? CPL : RES_LDS_CHUNKS;
    constexpr int RC = CPL - LC;
    __shared__ uint4 lds[LC * RES_WG];
    __shared__ uint32_t red[RES_WAVES];
    const int tid = threadIdx.x, wv = tid / WAVE;
    const int64_t stride = (int64_t)gridDim.x * RES_WG;
    const int64_t c00 = ((int64_t)(tid / 32) * gridDim.x + blockIdx.x) * 32 + tid % 32;
    auto chunk = [&](int j) {
        const int64_t c = j * stride + c00;
        return x + (c < nchunks ? c : c00);
    };
#pragma unroll
    for (int j = 0; j < LC; ++j)
        __builtin_amdgcn_global_load_lds((global_cptr)chunk(j), (lds_ptr)&lds[j * RES_WG + wv * WAVE],
                                         16, 0, 0);
    uint4 v[RC > 0 ? RC : 1];
#pragma unroll
    for (int r = 0; r < RC; ++r) v[r] = ld_stream(chunk(LC + r));
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < RC; ++r) m = max(m, amax_bf16x8(v[r]));
    __builtin_amdgcn_s_waitcnt(0);  // the global->LDS loads of this wave have landed
#pragma unroll
    for (int j = 0; j < LC; ++j) m = max(m, amax_bf16x8(lds[j * RES_WG + tid]));
    m = wave_max_u32(m);
    if ((tid & (WAVE - 1)) == 0) red[wv] = m;
    __syncthreads();
    if (tid == 0) {
        uint32_t r = red[0];
        for (int i = 1; i < RES_WAVES; ++i) r = max(r, red[i]);
        partials[blockIdx.x] = r;
    }
}

// ---------------------------------------------------------------------------
// NVFP4 quantize, pass 2, written in the packed NVFP4 operand layout: one
// wave per (row tile rt, K step ks) writes the tile's contiguous kilobyte of
// codes; lane l takes row 32 rt + l % 32, values 32 (2 ks + l / 32) .. + 31,
// which are two 16-blocks, and derives both block scales itself (the same
// per-block scale and divide as the row-major kernel, so the same codes and
// scale bytes).  The two E4M3 bytes go to bytes 16 l + 2 (ks % 8) + {0, 1}
// of the tile's scale group ks / 8.  Rows past the tensor are written as
// the layout's padding (codes 0, scale bytes 0).
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(WG) void nv_quantize_packed_kernel(
    const uint4 *__restrict__ x, int64_t rows, int64_t K, int64_t ntiles,
    const uint32_t *__restrict__ partials, int npart, uint4 *__restrict__ codes,
    uint16_t *__restrict__ scales, float *__restrict__ global_scale, int32_t *status) {
    __shared__ NvScaleTable T;
    TensorScale ts = tensor_scale<BF16>(partials, npart);
    if (blockIdx.x == 0 && threadIdx.x == 0) *global_scale = ts.s_g;
    if (ts.flags) {  // uniform over the grid: outputs unspecified
        if (blockIdx.x == 0 && threadIdx.x == 0 && status) atomicOr(status, (int32_t)ts.flags);
        return;
    }
    nv_table_build(T, ts.s_g, recip_row<BF16>(ts));
    __syncthreads();
    const CodeGuess G = make_code_guess(ts.s_g);
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_WG + (threadIdx.x / WAVE);
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    const int64_t nks = K / 64;
    uint32_t flags = 0;
    for (int64_t t = wave; t < ntiles; t += nwaves) {
        const int64_t rt = t / nks, ks = t % nks;
        const int64_t row = rt * 32 + (lane & 31);
        const bool ok = row < rows;
        const int64_t c0 = (row * K + (2 * ks + (lane >> 5)) * 32) / 8;
        Chunk<BF16> k[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = load_chunk<BF16>(x, c0 + i, ok);
        const uint32_t ma = max(chunk_amax<BF16>(k[0]), chunk_amax<BF16>(k[1]));
        const uint32_t mb = max(chunk_amax<BF16>(k[2]), chunk_amax<BF16>(k[3]));
        uint32_t fa = 0;
        const BlockScale sa = nv_block_scale(T, amax_as_f32_bits<BF16>(ma), G, fa);
        const BlockScale sb = nv_block_scale(T, amax_as_f32_bits<BF16>(mb), G, fa);
        if (ok) flags |= fa;
        uint32_t q[4];
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const BlockScale &b = i < 2 ? sa : sb;
            chunk_values<BF16>(k[i], v);
            q[i] = nv_quant8<BF16>(v, b.ad, b.y, b.sc, b.yc);
        }
        codes[t * 64 + lane] = ok ? make_uint4(q[0], q[1], q[2], q[3]) : make_uint4(0u, 0u, 0u, 0u);
        const uint16_t sc = ok ? (uint16_t)(sa.code | (sb.code << 8)) : (uint16_t)0;
        scales[((rt * (nks / 8) + ks / 8) * 64 + lane) * 8 + ks % 8] = sc;
    }
    report_flags(status, flags);
}

// Phase clock (a separate profiling build, -DFP4_PHASE_CLOCK): thread 0 of
// each workgroup of the one-pass kernel stamps the device's constant 100 MHz
// clock in slots 0..7 of its row: 0 its start, 1 after its loads and partial
// amax, 7 when its poll has seen every slot, 2 after the grid barrier, 5
// once s_g and the table window are known, 6 after the table's per-code
// step, 3 after the table, 4 at its end.
#ifdef FP4_PHASE_CLOCK
__device__ uint64_t g_phase_clock[kResidentSlots * 8];
#define FP4_PHASE(k)                                                                     \
    do {                                                                                 \
        if (threadIdx.x == 0) g_phase_clock[blockIdx.x * 8 + (k)] = __builtin_amdgcn_s_memrealtime(); \
    } while (0)
hipError_t read_phase_clock(uint64_t *host, size_t n) {
    if (n > (size_t)kResidentSlots * 8) n = (size_t)kResidentSlots * 8;
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_clock), n * sizeof(uint64_t), 0,
                               hipMemcpyDeviceToHost);
}
#else
#define FP4_PHASE(k) \
    do {             \
    } while (0)
#endif

// Cache policy of the code stores: non-temporal (the 33.6 MB of codes are
// not read again by this kernel; measured ~1 us faster per call at 8192^2).
// The scale bytes are stored non-temporally too (0.2 us).
constexpr int kStoreNT = 2;

// EXACT: the grid covers the tensor exactly (nchunks = gridDim.x * 512 * CPL),
// so no load is clamped and no store predicated.
template <int CPL, bool EXACT>
__global__ __launch_bounds__(RES_WG) void nv_resident_kernel(
    const uint4 *__restrict__ x, int nchunks, uint32_t *__restrict__ codes,
    uint8_t *__restrict__ scales, float *__restrict__ global_scale, uint64_t *slots,
    uint32_t *epoch, uint32_t spin_limit, int32_t *status) {
    constexpr int LC = CPL < RES_LDS_CHUNKS ? CPL : RES_LDS_CHUNKS;  // chunks per lane in LDS
    constexpr int RC = CPL - LC;                                     // ... and in VGPRs
    // one LDS block, table first: its addresses then fit the 16-bit
    // immediate offset of an LDS read, so no base is rebuilt per lookup
    struct Shared {
        NvDirectTable T;
        uint32_t red[RES_WAVES];
        uint32_t red_min[RES_WAVES];
        uint32_t tensor_amax;
        uint32_t late_tag;
        uint32_t wg_lo, wg_hi;  // this workgroup's smallest nonzero and largest block amax
        uint16_t rc[128];  // kRecipCorrection, staged during phase 1
        uint4 data[LC * RES_WG];
    };
    __shared__ Shared sh;
    NvDirectTable &T = sh.T;
    uint32_t(&red)[RES_WAVES] = sh.red;
    uint32_t &tensor_amax = sh.tensor_amax;
    uint4(&lds)[LC * RES_WG] = sh.data;

    FP4_PHASE(0);
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const int stride = gridDim.x * RES_WG;       // chunks covered by one step j of the grid
    const int c00 = blockIdx.x * RES_WG + tid;   // this lane's chunk at step 0
    const int last = nchunks - 1;
    // the table build's inputs that do not depend on s_g, ready before the
    // grid barrier (barriers below order these stores before their reads)
    if (tid < 128) sh.rc[tid] = kRecipCorrection[tid];
    if (tid == 0) T.need = 0u;

    // ---- phase 1: load the slice once, partial amax ----------------------
    // step j reads x[j*stride + c00]: a uniform base plus this lane's offset,
    // clamped to the last chunk
#pragma unroll
    for (int j = 0; j < LC; ++j) {
        const uint4 *xj = x + j * stride;
        __builtin_amdgcn_global_load_lds((global_cptr)(xj + (EXACT ? c00 : min(c00, last - j * stride))),
                                         (lds_ptr)&lds[j * RES_WG + wv * WAVE], 16, 0, 0);
    }
    uint4 v[RC > 0 ? RC : 1];
#pragma unroll
    for (int r = 0; r < RC; ++r) {
        const int j = LC + r;
        v[r] = ld_stream(x + j * stride + (EXACT ? c00 : min(c00, last - j * stride)));
    }
    const uint32_t tag = wv == 0 ? barrier_tag(epoch) : 0u;
    // The amaxes of the blocks this lane will derive scales for, while the
    // loads stream in: chunk rows 2p and 2p + 1 form pair p, whose block amax
    // (bf16 magnitude bits) is kept, two pairs per register, for phase 2.
    constexpr int NP = CPL / 2;
    const bool odd = lane & 1;
    uint32_t am[(NP + 1) / 2];
#pragma unroll
    for (int i = 0; i < (NP + 1) / 2; ++i) am[i] = 0;
    uint32_t m = 0;
    // and the smallest nonzero block amax (0xFFFF: none), which with m bounds
    // the table entries this workgroup's blocks index
    uint32_t mn = 0xFFFFu;
    auto keep_pair = [&](int p, uint32_t m0, uint32_t m1) {
        m = max(m, max(m0, m1));
        const uint32_t ag = pair_amax(m0, m1, odd);
        mn = min(mn, ag ? ag : 0xFFFFu);
        am[p >> 1] |= (p & 1) ? ag << 16 : ag;  // pairs are kept in no particular order
    };
#pragma unroll
    for (int r = 0; r < RC; r += 2) keep_pair((LC + r) / 2, amax_bf16x8(v[r]), amax_bf16x8(v[r + 1]));
    __builtin_amdgcn_s_waitcnt(0);  // the global->LDS loads of this wave have landed
#pragma unroll
    for (int j = 0; j < LC; j += 2)
        keep_pair(j / 2, amax_bf16x8(lds[j * RES_WG + tid]), amax_bf16x8(lds[(j + 1) * RES_WG + tid]));
    // opaque to the optimiser: the packed amaxes are final here (it would
    // otherwise carry the per-chunk maxima across the barrier instead)
#pragma unroll
    for (int i = 0; i < (NP + 1) / 2; ++i) asm volatile("" : "+v"(am[i]));
    m = wave_max_u32(m);
    mn = wave_min_u32(mn);
    if (lane == 0) {
        red[wv] = m;
        sh.red_min[wv] = mn;
    }
    __syncthreads();
    FP4_PHASE(1);

    // ---- grid barrier: wave 0 publishes the partial amax and polls --------
    uint32_t flags = 0;
    if (wv == 0) {
        uint32_t wm = lane < RES_WAVES ? red[lane] : 0u;
        uint32_t wn = lane < RES_WAVES ? sh.red_min[lane] : 0xFFFFu;
        wm = wave_max_u32(wm);
        wn = wave_min_u32(wn);
        if (lane == 0) {
            sh.wg_lo = wn;
            sh.wg_hi = wm;
        }
        uint32_t A;
        const bool done = grid_barrier_max(slots, tag, wm, spin_limit, A);
        FP4_PHASE(7);
        if (lane == 0) {
            tensor_amax = A;
            sh.late_tag = done ? 0u : tag;
            if (!done || blockIdx.x == 0) barrier_store_epoch(epoch, tag);
        }
    }
    __syncthreads();
    const uint32_t late = sh.late_tag;  // uniform: the tag, when the wait timed out
    if (late) {
        // Fallback: the tensor amax without the barrier.  A slot carrying the
        // tag holds its slice's amax from this call; every other slice is read
        // here from x (the same chunks its workgroup loads).
        uint32_t mf = 0;
        for (int w = wv; w < (int)gridDim.x; w += RES_WAVES) {
            uint32_t sv;
            const bool tagged = barrier_slot_tagged(slots, w, late, sv);
            if (__builtin_amdgcn_readfirstlane((int)tagged)) {
                mf = max(mf, (uint32_t)__builtin_amdgcn_readfirstlane((int)sv));
                continue;
            }
            for (int j = 0; j < CPL; ++j)
                for (int t = lane; t < RES_WG; t += WAVE) {
                    const int c = j * stride + w * RES_WG + t;
                    if (c < nchunks) mf = max(mf, amax_bf16x8(ld_stream(x + c)));
                }
        }
        mf = wave_max_u32(mf);
        if (lane == 0) red[wv] = mf;  // wave 0 read red before the barrier above
        __syncthreads();
        if (tid == 0) {
            uint32_t a = tensor_amax;
            for (int i = 0; i < RES_WAVES; ++i) a = max(a, red[i]);
            tensor_amax = a;
        }
        __syncthreads();
        flags |= FLAG_BARRIER_TIMEOUT;
    }
    FP4_PHASE(2);
    const TensorScale ts = scale_from_amax(tensor_amax << 16);
    if (blockIdx.x == 0 && tid == 0) *global_scale = ts.s_g;
    if (ts.flags) {  // uniform over the grid: outputs unspecified
        if (blockIdx.x == 0 && tid == 0 && status) atomicOr(status, (int32_t)ts.flags);
        if (late && tid == 0) barrier_retract(slots);
        report_flags(status, flags);
        return;
    }
    // The table's window starts at the smaller of the code-1 threshold and
    // this workgroup's smallest nonzero block amax, and ends at its largest
    // (entries past RES_NIDX + 1 all hold the saturated code).
    // Entries this workgroup's blocks can index: 0 and 1, and those of its
    // nonzero block amaxes in [wg_lo, wg_hi] (RES_NIDX + 1 for all at or
    // past the window's last magnitude).
    const uint32_t base = nv_window_base(ts.s_g);
    const int i0 = 2 + (int)min(max(sh.wg_lo, base) - base, (uint32_t)RES_NIDX - 1u);
    const int i1 = 2 + (int)min(max(sh.wg_hi + 1u, base) - base, (uint32_t)RES_NIDX);
    FP4_PHASE(5);
    nv_direct_table_build(T, ts.s_g, sh.rc[tensor_amax & 127u], base, i0, i1,
                          [] { FP4_PHASE(6); });  // ends with a barrier
    const uint32_t need = T.need;            // uniform
    FP4_PHASE(3);

    // ---- phase 2: quantize from LDS and registers -----------------------
    // Two chunk rows per iteration: a lane pair holds one 16-element block of
    // each; the even lane looks up row 0's block scale, the odd lane row 1's,
    // and they swap the divisor terms.
    // Opaque to the optimiser: phase 1's per-chunk results are not kept alive
    // across the barrier for reuse (there are no registers for them).
#pragma unroll
    for (int r = 0; r < RC; ++r) asm volatile("" : "+v"(v[r].x), "+v"(v[r].y), "+v"(v[r].z), "+v"(v[r].w));
    float ymin = __builtin_inff();  // the compact loop's smallest Y (0: a scale underflow)
    // code dwords go out as buffer stores: one resource, the lane's byte
    // offset in a VGPR and the uniform part of the address in an SGPR
    const uint32_t coff = (uint32_t)c00 * 4u;
    const __amdgpu_buffer_rsrc_t crs =
        __builtin_amdgcn_make_buffer_rsrc(codes, (short)0, nchunks * 4, kBufferRsrcWord3);
    const int cs = odd ? c00 + stride : c00;  // this lane's scale chunk, relative to row 0
    // a block amax (bf16 bits) -> its table entry: 0 for a zero block, else
    // base + i - 2 clamped to [1, RES_NIDX + 1] (one med3, whose lower bound
    // min(ag, 1) is 0 for the zero block)
    auto entry_of = [&](uint32_t ag) {
        const int k = (int)ag - (int)base + 2, lo = (int)min(ag, 1u), hi = RES_NIDX + 1;
        int e;
        asm("v_med3_i32 %0, %1, %2, %3" : "=v"(e) : "v"(k), "v"(lo), "s"(hi));
        return e;
    };
    // pair p's block amax -> its table entry
    auto entry = [&](int p) {
        const uint32_t ag = (p & 1) ? (am[p >> 1] >> 16) : (am[p >> 1] & 0xFFFFu);
        return entry_of(ag);
    };
    // The quotient x / alpha, chosen once per call (uniformly, from the table):
    //  - the product x * Y_c (every code's Y_c makes it exact for bf16 input);
    //  - fma(x, Y_c, x * D_c) when some code needs the two-operation form (D_c
    //    is 0 for the others, where it is the product again);
    //  - the exact compact loop otherwise (tiny tensors whose small codes need
    //    operand scaling; a code no form fits), re-reading the tiles from HBM.
    // Only the chosen loop is ever fetched: the unrolled loop's size, not its
    // arithmetic, is what limits it otherwise.  The table lookups of pair
    // p + 1 are issued before pair p's arithmetic.
    auto full_loop = [&](auto two_op_tag) {
        constexpr bool TWO = decltype(two_op_tag)::value;
        int idx = entry(0);
        float y = T.y[idx];
        uint32_t c = T.code[idx];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            __builtin_amdgcn_sched_barrier(0);  // keep iterations apart: registers are scarce
            float yn = 0.0f;
            uint32_t cn = 0;
            if (p + 1 < NP) {
                const int in = entry(p + 1);
                yn = T.y[in];
                cn = T.code[in];
            }
            const int j0 = 2 * p, j1 = j0 + 1;
            const uint4 w0 = j0 < LC ? lds[j0 * RES_WG + tid] : v[j0 - LC];
            const uint4 w1 = j1 < LC ? lds[j1 * RES_WG + tid] : v[j1 - LC];
            float ys[2], ds[2];
            pair_rows(y, ys);
            if (TWO) pair_rows(T.dc[c], ds);
            const int b0 = j0 * stride;
            if (EXACT || cs <= last - b0)
                __builtin_nontemporal_store((uint8_t)c, &(scales + (b0 >> 1))[(uint32_t)cs >> 1]);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                float f[8];
                widen_bf16x8(k == 0 ? w0 : w1, f);
#pragma unroll
                for (int i = 0; i < 8; ++i) f[i] = TWO ? __builtin_fmaf(f[i], ys[k], f[i] * ds[k]) : f[i] * ys[k];
                const uint32_t q = cvt_fp4x8_f32(f, e8m0_operand(E8M0_ONE));
                const int bk = (j0 + k) * stride;  // uniform
                if (EXACT || c00 <= last - bk) __builtin_amdgcn_raw_buffer_store_b32(q, crs, (int)coff, bk * 4, kStoreNT);
            }
            y = yn;
            c = cn;
        }
    };
    if (!(need & NV_NEEDS_EXACT)) {
        if (need & NV_NEEDS_TWO_OP) full_loop(std::true_type{});
        else full_loop(std::false_type{});
    } else {
        // the compact loop: (x sc) / (alpha sc), sc = 2^64 for alpha < 2^-90,
        // with the reciprocal-correction divide
        for (int j0 = 0; j0 < CPL; j0 += 2) {
            uint4 w[2];
            for (int k = 0; k < 2; ++k) {
                const int bk = (j0 + k) * stride;
                w[k] = ld_stream(x + bk + (EXACT ? c00 : min(c00, last - bk)));
            }
            // the block amax again from the tiles (a rolled loop cannot index am)
            const uint32_t ag = pair_amax(amax_bf16x8(w[0]), amax_bf16x8(w[1]), odd);
            const int idx = ag == 0 ? 0 : min(max((int)ag - (int)base + 2, 1), RES_NIDX + 1);
            const uint32_t c = T.code[idx];
            ymin = __builtin_fminf(ymin, T.y[idx]);
            const int b0 = j0 * stride;
            if (EXACT || cs <= last - b0)
                __builtin_nontemporal_store((uint8_t)c, &(scales + (b0 >> 1))[(uint32_t)cs >> 1]);
            const float a = ts.s_g * e4m3_pos_value(c);
            const float sc = a < kDivScaleBelow ? kDivScale : 1.0f;
            float ad[2], scr[2];
            pair_rows(a * sc, ad);  // exact
            pair_rows(sc, scr);
            for (int k = 0; k < 2; ++k) {
                float f[8];
                widen_bf16x8(w[k], f);
                const float y = ad[k] > 0.0f ? 1.0f / ad[k] : 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) f[i] = div_rn(f[i] * scr[k], ad[k], y);
                const uint32_t q = cvt_fp4x8_f32(f, e8m0_operand(E8M0_ONE));
                const int bk = (j0 + k) * stride;
                if (EXACT || c00 <= last - bk) __builtin_amdgcn_raw_buffer_store_b32(q, crs, (int)coff, bk * 4, kStoreNT);
            }
        }
    }
    flags |= ymin == 0.0f ? FLAG_SCALE_UNDERFLOW : 0u;
    // Some nonzero block took code 0 (its scale underflowed): codes never
    // fall as the block amax grows, so the workgroup's smallest nonzero block
    // amax has code 0 then.  (With s_g normal, as in the full loops, code 0 is
    // the only code whose Y is 0.)
    if (sh.wg_lo != 0xFFFFu && T.code[entry_of(sh.wg_lo)] == 0) flags |= FLAG_SCALE_UNDERFLOW;
    if (late && tid == 0) barrier_retract(slots);
    report_flags(status, flags);
#ifdef FP4_PHASE_CLOCK
    __builtin_amdgcn_s_waitcnt(0);  // this workgroup's stores have left
    __syncthreads();
    FP4_PHASE(4);
#endif
}

// ---------------------------------------------------------------------------
// Dequantize.  Lane = one chunk of 8 codes (one dword) -> 8 outputs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_any_value(uint32_t s) {
    uint32_t mag = s & 0x7Fu;
    if (mag == 0x7Fu) return __builtin_nanf("");
    float v = e4m3_pos_value(mag);
    return (s & 0x80u) ? -v : v;
}

// nearest-even fp32 -> bf16 (NaN kept quiet)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t b = f2u(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x40u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Decode one chunk (8 codes in a dword) to 8 outputs, written with streaming
// (non-temporal) stores: measured faster here than ordinary stores for this
// write-heavy kernel.
template <int FMT, bool OUT_BF16>
__device__ __forceinline__ void dequant_chunk(uint32_t q, uint32_t sb, float s_g, uint4 *y, int64_t c) {
    float v[8];
    if (FMT == 0) {
        const float so = e8m0_operand(sb);
        if (OUT_BF16) {
            uint32_t o[4];
            o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, so, 0));
            o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, so, 1));
            o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, so, 2));
            o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, so, 3));
            if (sb == 0xFFu) o[0] = o[1] = o[2] = o[3] = 0x7FC07FC0u;
            st_stream(y + c, make_uint4(o[0], o[1], o[2], o[3]));
            return;
        }
        f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, so, 0);
        f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, so, 1);
        f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, so, 2);
        f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, so, 3);
        v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
        v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
        if (sb == 0xFFu) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __builtin_nanf("");
        }
    } else {
        const float alpha = s_g * e4m3_any_value(sb);
        const float one = e8m0_operand(E8M0_ONE);
        f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, one, 0);
        f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, one, 1);
        f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, one, 2);
        f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, one, 3);
        v[0] = p0.x * alpha; v[1] = p0.y * alpha; v[2] = p1.x * alpha; v[3] = p1.y * alpha;
        v[4] = p2.x * alpha; v[5] = p2.y * alpha; v[6] = p3.x * alpha; v[7] = p3.y * alpha;
    }
    if (OUT_BF16) {
        uint4 o;
        o.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
        o.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
        o.z = bf16_rne(v[4]) | (bf16_rne(v[5]) << 16);
        o.w = bf16_rne(v[6]) | (bf16_rne(v[7]) << 16);
        st_stream(y + c, o);
    } else {
        st_stream(y + 2 * c, make_uint4(f2u(v[0]), f2u(v[1]), f2u(v[2]), f2u(v[3])));
        st_stream(y + 2 * c + 1, make_uint4(f2u(v[4]), f2u(v[5]), f2u(v[6]), f2u(v[7])));
    }
}

// Lane l of a wave tile decodes chunks tile*64*U + r*64 + l, r < U: every
// code load and output store of the wave is contiguous.  The waves stride
// over the tiles and load the next tile's codes and scale bytes before they
// decode and store the current one, so the loads are in flight under the
// stores instead of stalling the wave between tiles.  Tile (chunks per lane)
// and grid cap per path, measured on 8192 x 8192: the MXFP4 bf16 decode is
// two instructions per chunk and runs best on deep tiles and few waves; the
// NVFP4 one (multiply and bf16 rounding per value) needs more waves; fp32
// output writes 32 bytes a chunk and gains nothing from depth.
template <int FMT, bool OUT_BF16>
struct DequantShape {
    static constexpr int U = !OUT_BF16 ? 4 : (FMT == 0 ? 32 : 16);       // chunks per lane
    static constexpr int G = !OUT_BF16 ? 4096 : (FMT == 0 ? 512 : 1024);  // workgroup cap
};
template <int FMT, bool OUT_BF16>
__global__ __launch_bounds__(WG) void dequant_kernel(const uint32_t *__restrict__ codes,
                                                     const uint8_t *__restrict__ scales,
                                                     const float *__restrict__ global_scale,
                                                     int64_t nchunks, uint4 *__restrict__ y) {
    constexpr int U = DequantShape<FMT, OUT_BF16>::U;
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_WG + (threadIdx.x / WAVE);
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    const int64_t ntiles = (nchunks + WAVE * U - 1) / (WAVE * U);
    const float s_g = (FMT == 1) ? *global_scale : 1.0f;
    auto load = [&](int64_t t, uint32_t (&q)[U], uint32_t (&sb)[U]) {
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const int64_t c = t * (WAVE * U) + r * WAVE + lane;
            const bool ok = c < nchunks;
            q[r] = ok ? __builtin_nontemporal_load(codes + c) : 0u;
            sb[r] = ok ? (uint32_t)scales[FMT == 0 ? (c >> 2) : (c >> 1)] : 0u;
        }
    };
    uint32_t q[U], sb[U];
    load(wave, q, sb);
    for (int64_t t = wave; t < ntiles; t += nwaves) {
        uint32_t qn[U], sn[U];
        load(t + nwaves, qn, sn);  // past the last tile every lane is out of range
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const int64_t c = t * (WAVE * U) + r * WAVE + lane;
            if (c < nchunks) dequant_chunk<FMT, OUT_BF16>(q[r], sb[r], s_g, y, c);
        }
#pragma unroll
        for (int r = 0; r < U; ++r) {
            q[r] = qn[r];
            sb[r] = sn[r];
        }
    }
}

// ---------------------------------------------------------------------------
// MSE-optimal NVFP4 scale search.  A lane pair holds one block (8 elements
// each).  The distinct encoded candidates of a block are the consecutive
// E4M3 codes from E4M3(c_lo t) to E4M3(c_hi t), t = A_g / (6 s_g) (the host
// checks the candidate grid is fine enough for that), visited in increasing
// order, which is increasing candidate index; a strictly smaller loss
// replaces the incumbent, so the smallest index wins ties.
// Loss: each lane sums its 8 squared errors as ((t0+t1)+(t2+t3))+((t4+t5)+
// (t6+t7)) and the pair adds the two halves: the balanced pairwise tree over
// the 16 elements in index order.  |x| and |x_hat| give the same squared
// error as the signed values.
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ float half_block_loss(const float (&a)[8], float4 sq, float yc) {
    // sq = {alpha, alpha', +-1/alpha', sc}: divide as (a sc) / alpha' (one
    // multiply by yc for bf16 input when no lane's scale is marked), rebuild
    // with alpha.  Both choices are wave-uniform; operands are scaled (x sc,
    // exact) only when some lane of the wave needs it (tensors with a tiny s_g).
    const float alpha = sq.x;
    const float y = __builtin_fabsf(sq.z);
    const bool scaled = __ballot(sq.w != 1.0f) != 0;
    float q[8];
    if (BF16 && !__ballot(sq.z < 0.0f)) {
        if (!scaled) {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = a[i] * yc;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = (a[i] * sq.w) * yc;
        }
    } else {
        if (!scaled) {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = div_rn(a[i], sq.y, y);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = div_rn(a[i] * sq.w, sq.y, y);
        }
    }
    const float one = e8m0_operand(E8M0_ONE);
    uint32_t code = cvt_fp4x8_f32(q, one);
    float t[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x2_t p;
        switch (j) {  // the byte selector must be a constant
            case 0: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, one, 0); break;
            case 1: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, one, 1); break;
            case 2: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, one, 2); break;
            default: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, one, 3); break;
        }
        float e0 = a[2 * j] - p.x * alpha;
        float e1 = a[2 * j + 1] - p.y * alpha;
        t[2 * j] = e0 * e0;
        t[2 * j + 1] = e1 * e1;
    }
    return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

// ---- the bf16 search with per-code tables and a work queue -----------------
// For a bf16 tensor whose s_g is a normal number (and every divisor alpha_c,
// c >= 1, at least 2^-90) a workgroup tabulates per code c:
//   {alpha_c, tlo[c + 1], Y_c, D_c}: the block quotient of code c is
//   RN32(x Y_c) (D_c = 0) or fma(x, Y_c, x D_c), chosen per code as in the
//   one-pass quantize (kRecipCorrection): the E2M1 code of the correctly
//   rounded quotient for every bf16 x;
//   thi[c], tlo[c]: bf16 bits of the smallest block amax whose upper / lower
//   candidate code, the RN-even E4M3 code of c_hi amax / (6 s_g) (c_lo ...),
//   is at least c.  A block's upper code is its fp32 guess g (the truncated
//   code of amax RN32(c_hi / (6 s_g)), within one code below the exact one)
//   plus whether its amax reaches thi[g + 1]; code c is at or above the
//   lower code when the amax stays below tlo[c + 1].
// The loss is that of half_block_loss on the signed values (the quotient,
// the E2M1 code and the error are odd in x, and the squared error is even),
// so the code words of the best candidate are the block's output as they
// stand.
//
// Each lane holds one block (16 values).  The wave steps its tile's walks in
// place while many lanes still walk (at least the first two candidates);
// a block that still has one to evaluate then goes to its wave's queue in
// LDS (its 16 values and its walk state), and once 64 blocks wait the wave
// evaluates the next candidate of 64 of them at once, putting back those
// that go on.  Every block visits the same codes in the same order as
// a plain walk, so the result is the same; only the lanes' idle time changes
// (a wave no longer waits for its slowest block).
struct SearchTable {
    float4 e[128];      // per code: {alpha, tlo[c + 1] bits, Y, D}; code 0 and 127: alpha = 0
    uint16_t thi[128];  // thi[0] = 0, thi[127] = 0xFFFF (no amax reaches code 127)
};
// Between passes a queue holds < 64 blocks; a tile adds at most 32 (a tile
// with more steps its blocks in place until at most 32 remain).
constexpr int SQ_CAP = 96;
// A tile's blocks step in place while more than this many lanes walk: an
// in-place step is ~105 VALU instructions for the wave, a queue pass ~150
// for 64 blocks, so in place wins above ~45 walking lanes.
constexpr int SQ_INLINE = 40;
struct SearchQueue {
    uint4 data[SQ_CAP][2];  // the block's 16 bf16 values
    uint2 st[SQ_CAP];       // {block index, next code | best code << 8 | amax bits << 16}
    float bestL[SQ_CAP];    // the best loss so far
};
struct SearchShared {
    SearchTable tab;
    SearchQueue q[WAVES_PER_WG];
    int left[WAVES_PER_WG];  // blocks left in each wave's queue after its tiles
};

// The blocks waiting: pool index p lives in queue k at entry p - start_k.
// MULTI = false: one queue.  MULTI: the workgroup's queues back to back
// (queue k from s[k - 1]), drained together at the end.
template <bool MULTI>
struct QueuePool {
    SearchQueue *q;
    int s1, s2, s3;
    __device__ __forceinline__ SearchQueue &at(int p, int &j) const {
        if (!MULTI) {
            j = p;
            return q[0];
        }
        const int k = (p >= s1 ? 1 : 0) + (p >= s2 ? 1 : 0) + (p >= s3 ? 1 : 0);
        j = p - (k == 0 ? 0 : (k == 1 ? s1 : (k == 2 ? s2 : s3)));
        return q[k];
    }
};

// bits of the smallest positive bf16 magnitude v with candidate code >= c
// (1 <= c <= 126): c_mul v (exact in binary64) above the exact threshold
// 6 s_g midpoint(c - 1, c), or on it when c is even.  0x7F80: no finite v.
__device__ __forceinline__ uint32_t search_bound_bf16(uint32_t c, float s_g, float cmul) {
    const double th = nv_threshold((int)c, s_g);
    uint32_t b = f2u((float)(th / (double)cmul)) >> 16;  // within a unit of the answer
    b = b > 1u ? b - 1u : 0u;
    for (int k = 0; k < 4 && b < 0x7F80u; ++k) {
        const double z = (double)cmul * (double)u2f(b << 16);
        if (z > th || (z == th && (c & 1u) == 0)) break;
        ++b;
    }
    return min(b, 0x7F80u);
}

// Builds the table; returns (to every thread, after a barrier) whether the
// table's rule covers the call (else the generic walk runs).
template <bool ALL>
__device__ __forceinline__ bool search_table_build(SearchTable &S, const TensorScale &ts, float c_lo,
                                                   float c_hi) {
    const int t = threadIdx.x;
    int slow = 0;
    if (t < 128) {
        const float s_g = ts.s_g;
        const uint32_t M = (ts.amax >> 16) & 127u;
        float a = 0.0f, Y = 0.0f, D = 0.0f;
        if (t >= 1 && t <= 126) {
            a = s_g * e4m3_pos_value((uint32_t)t);
            const uint32_t sel = (kRecipCorrection[M] >> (2u * e4m3_frac_index((uint32_t)t))) & 3u;
            const float y0 = 1.0f / a;  // correctly rounded
            if (!(a >= kDivScaleBelow) || !(s_g >= 0x1p-126f)) {
                slow = 1;
            } else if (sel < 3u) {
                Y = sel == 0u ? y0 : u2f(f2u(y0) + (sel == 1u ? ~0u : 1u));
            } else if ((f2u(a) & 0xFFu) == 0u) {  // at most 16 significant bits
                const double r = 1.0 / (double)a;
                float yh = (float)r;
                if ((double)yh > r) yh = u2f(f2u(yh) - 1u);
                Y = yh;
                D = (float)(r - (double)yh);
            } else {
                slow = 1;
            }
        }
        // every code is at or above the lower code 1 of the exhaustive search
        const uint32_t c1 = (uint32_t)t + 1u;
        const uint32_t tlo = ALL || c1 >= 127u ? 0xFFFFu : search_bound_bf16(c1, s_g, c_lo);
        S.e[t] = make_float4(a, u2f(tlo), Y, D);
        if (!ALL) {
            const uint32_t c = (uint32_t)t;
            S.thi[t] = (uint16_t)(c == 0 ? 0u : (c == 127 ? 0xFFFFu : search_bound_bf16(c, s_g, c_hi)));
        }
    }
    return __syncthreads_or(slow) == 0;
}

// The code word of 8 values a[0..7] under a code's quotient (TWO: the
// two-operation one).
template <bool TWO>
__device__ __forceinline__ uint32_t cand_codes8(const float *a, float4 e) {
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = TWO ? __builtin_fmaf(a[i], e.z, a[i] * e.w) : a[i] * e.z;
    return cvt_fp4x8_f32(q, e8m0_operand(E8M0_ONE));
}

// Sum of the squared errors of a[0..7] with code word `code` under alpha:
// ((t0+t1)+(t2+t3))+((t4+t5)+(t6+t7)), one half of the block's pairwise tree.
__device__ __forceinline__ float half_sq_error(const float *a, uint32_t code, float alpha) {
    const float one = e8m0_operand(E8M0_ONE);
    float t[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x2_t p;
        switch (j) {  // the byte selector must be a constant
            case 0: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, one, 0); break;
            case 1: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, one, 1); break;
            case 2: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, one, 2); break;
            default: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(code, one, 3); break;
        }
        float e0 = a[2 * j] - p.x * alpha;
        float e1 = a[2 * j + 1] - p.y * alpha;
        t[2 * j] = e0 * e0;
        t[2 * j + 1] = e1 * e1;
    }
    return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

// The block's code words under a code (wave-uniform choice of quotient).
__device__ __forceinline__ uint2 cand_codes16(const float (&a)[16], float4 e, bool two) {
    if (two) return make_uint2(cand_codes8<true>(a, e), cand_codes8<true>(a + 8, e));
    return make_uint2(cand_codes8<false>(a, e), cand_codes8<false>(a + 8, e));
}

// The walk state of the lane's block.
struct Walk {
    int code;       // next candidate
    int best;
    float bestL;
    uint2 bq;       // code words at the best candidate (when known)
    float agf;      // block amax
    uint32_t agb;   // its bf16 bits
};

// Evaluates the lane's next candidate where `go`, then steps the walk.
__device__ __forceinline__ void walk_step(const SearchTable &S, const float (&a)[16], Walk &w, bool go) {
    const float4 e = S.e[max(w.code, 0)];
    const uint2 q = cand_codes16(a, e, __ballot(go && e.w != 0.0f) != 0);
    const float L = half_sq_error(a, q.x, e.x) + half_sq_error(a + 8, q.y, e.x);
    if (go && L <= w.bestL) {
        w.best = w.code;
        w.bestL = L;
        w.bq = q;
    }
    if (go) --w.code;
}

// Whether code w.code is a candidate: at least 1 and at or above the lower
// code (a zero block has its one code only).
__device__ __forceinline__ bool walk_in_range(float2 g, const Walk &w) {
    return w.code >= 1 && w.agb != 0u && w.agb < f2u(g.y);
}

// Whether the walk goes on: a next code in range that the early-stop bound
// (see scale_search_kernel) does not rule out.
__device__ __forceinline__ bool walk_goes_on(const SearchTable &S, const Walk &w) {
    const float2 g = *reinterpret_cast<const float2 *>(&S.e[max(w.code, 0)]);
    const float x6 = 6.0f * g.x;
    const float e6 = w.agf - x6;
    const float bound = w.agf >= x6 ? e6 * e6 : 0.0f;
    return walk_in_range(g, w) && !(bound > w.bestL);
}

__device__ __forceinline__ void walk_finish(const Walk &w, int64_t b, uint32_t *__restrict__ codes,
                                            uint8_t *__restrict__ scales, uint32_t &flags) {
    reinterpret_cast<uint2 *>(codes)[b] = w.bq;
    scales[b] = (uint8_t)w.best;
    if (w.best == 0 && w.agb != 0u) flags |= FLAG_SCALE_UNDERFLOW;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (f2u(hi) & 0xFFFF0000u) | (f2u(lo) >> 16);
}

// Pushes the lanes with `more` onto the pool; n: its length (uniform).
template <bool MULTI>
__device__ __forceinline__ void queue_push(const QueuePool<MULTI> &P, int &n, bool more,
                                           const float (&a)[16], const Walk &w, int64_t b) {
    const uint64_t bal = __ballot(more);
    const int p = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (more) {
        int slot;
        SearchQueue &Q = P.at(p, slot);
        Q.data[slot][0] = make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                     pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7]));
        Q.data[slot][1] = make_uint4(pack_bf16x2(a[8], a[9]), pack_bf16x2(a[10], a[11]),
                                     pack_bf16x2(a[12], a[13]), pack_bf16x2(a[14], a[15]));
        Q.st[slot] = make_uint2((uint32_t)b, (uint32_t)w.code | ((uint32_t)w.best << 8) | (w.agb << 16));
        Q.bestL[slot] = w.bestL;
    }
    n += __builtin_popcountll(bal);
}

__device__ __forceinline__ void widen_block(uint4 k0, uint4 k1, float (&a)[16]) {
    float (&lo)[8] = *reinterpret_cast<float (*)[8]>(&a[0]);
    float (&hi)[8] = *reinterpret_cast<float (*)[8]>(&a[8]);
    widen_bf16x8(k0, lo);
    widen_bf16x8(k1, hi);
}

// One pass over the top m (<= 64) blocks of the pool: each evaluates its
// next candidate; those whose walk goes on are pushed back, the rest written
// (their code words recomputed where the best candidate is an earlier one).
template <bool MULTI>
__device__ __forceinline__ void queue_pass(const SearchTable &S, const QueuePool<MULTI> &P, int &n,
                                           int m, uint32_t *__restrict__ codes,
                                           uint8_t *__restrict__ scales, uint32_t &flags) {
    const int lane = __lane_id();
    const bool act = lane < m;
    int j;
    SearchQueue &Q = P.at(n - m + (act ? lane : 0), j);
    const uint2 st = Q.st[j];
    Walk w;
    w.bestL = Q.bestL[j];
    w.code = (int)(st.y & 0xFFu);
    w.best = (int)((st.y >> 8) & 0xFFu);
    w.agb = st.y >> 16;
    w.agf = u2f(w.agb << 16);
    w.bq = make_uint2(0, 0);
    float a[16];
    widen_block(Q.data[j][0], Q.data[j][1], a);
    const int evaluated = w.code;
    walk_step(S, a, w, act);
    const bool more = act && walk_goes_on(S, w);
    const bool fin = act && !more;
    if (__ballot(fin && w.best != evaluated)) {
        const float4 e = S.e[w.best];
        const uint2 q = cand_codes16(a, e, __ballot(fin && w.best != evaluated && e.w != 0.0f) != 0);
        if (w.best != evaluated) w.bq = q;
    }
    if (fin) walk_finish(w, st.x, codes, scales, flags);
    n -= m;
    queue_push(P, n, more, a, w, st.x);
}

// k0, k1: the wave's first tile, loaded by the caller before the table build.
template <bool ALL>
__device__ __forceinline__ void search_bf16_tiles(SearchShared &SS,
                                                  const uint4 *__restrict__ x, int64_t nblocks,
                                                  uint4 k0, uint4 k1, float r_hi,
                                                  uint32_t *__restrict__ codes,
                                                  uint8_t *__restrict__ scales, uint32_t &flags) {
    const SearchTable &S = SS.tab;
    const int lane = __lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const QueuePool<false> P{&SS.q[wv], 0, 0, 0};
    const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_WG + wv;
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    const int64_t ntiles = (nblocks + WAVE - 1) / WAVE;
    int n = 0;  // blocks waiting in the queue
    for (int64_t t = wave; t < ntiles; t += nwaves) {
        const int64_t b = t * WAVE + lane;
        const bool ok = b < nblocks;
        // the next tile's block, loaded while this one is searched (past the
        // end: the last block again, never used)
        const int64_t bn = min(b + nwaves * WAVE, nblocks - 1);
        const uint4 n0 = x[2 * bn], n1 = x[2 * bn + 1];  // ordinary loads: see load_chunk
        Walk w;
        w.agb = max(amax_bf16x8(k0), amax_bf16x8(k1));
        w.agf = u2f(w.agb << 16);
        if (w.agb == 0) {
            w.code = 0x38;  // a zero block: scale 1, all codes zero
        } else if (ALL) {
            w.code = 126;
        } else {
            const uint32_t gh = e4m3_trunc_code(w.agf * r_hi);
            const uint32_t hi = gh + (w.agb >= S.thi[gh + 1] ? 1u : 0u);
            // none in range (hi is 0 or below the lower code): code 0, a scale underflow
            w.code = hi >= 1u && w.agb < f2u(S.e[hi].y) ? (int)hi : 0;
        }
        w.best = 0;
        w.bestL = __builtin_inff();
        w.bq = make_uint2(0, 0);
        float a[16];
        widen_block(k0, k1, a);
        walk_step(S, a, w, true);  // the first candidate always exists
        // the second without the early-stop test: a code the bound rules out
        // has a loss above the best and is not taken, and the test after it
        // stops the walk
        bool more = walk_in_range(*reinterpret_cast<const float2 *>(&S.e[max(w.code, 0)]), w);
        // In place while many lanes still walk (a step then costs less than
        // a queue pass per block), and while the queue has no room.
        int k = __builtin_popcountll(__ballot(more));
        while (k > 0 && (k > SQ_INLINE || n + k > SQ_CAP)) {
            walk_step(S, a, w, more);
            more = more && walk_goes_on(S, w);
            k = __builtin_popcountll(__ballot(more));
        }
        if (ok && !more) walk_finish(w, b, codes, scales, flags);
        queue_push(P, n, ok && more, a, w, b);
        n = __builtin_amdgcn_readfirstlane(n);
        while (n >= WAVE) {
            queue_pass(S, P, n, WAVE, codes, scales, flags);
            n = __builtin_amdgcn_readfirstlane(n);
        }
        k0 = n0;
        k1 = n1;
    }
    // the blocks left in the four queues (< 64 each) are drained by one wave,
    // in passes over all of them
    if (lane == 0) SS.left[wv] = n;
    __syncthreads();
    if (wv != 0) return;
    const int s1 = SS.left[0], s2 = s1 + SS.left[1], s3 = s2 + SS.left[2];
    const QueuePool<true> all{&SS.q[0], s1, s2, s3};
    int left = s3 + SS.left[3];
    while (left > 0) {
        queue_pass(S, all, left, min(left, WAVE), codes, scales, flags);
        left = __builtin_amdgcn_readfirstlane(left);
    }
}

// ALL: every E4M3 code 1..126 is a candidate (the format page's brute force,
// section 4), instead of the codes the candidate range c_lo..c_hi reaches.
template <bool BF16, bool ALL>
__global__ __launch_bounds__(WG, 8) void scale_search_kernel(
    const uint4 *__restrict__ x, int64_t nchunks, const uint32_t *__restrict__ partials,
    int npart, float c_lo, float c_hi, uint32_t *__restrict__ codes,
    uint8_t *__restrict__ scales, float *__restrict__ global_scale, int32_t *status) {
    constexpr size_t kShared = BF16 && sizeof(SearchShared) > sizeof(NvScaleTable) ? sizeof(SearchShared)
                                                                                    : sizeof(NvScaleTable);
    __shared__ __align__(16) uint8_t smem[kShared];
    // bf16: the wave's first tile (a block per lane), in flight during the set-up
    uint4 k0 = make_uint4(0, 0, 0, 0), k1 = k0;
    if (BF16) {
        const int64_t b0 = min(((int64_t)blockIdx.x * WAVES_PER_WG + threadIdx.x / WAVE) * WAVE +
                                   (threadIdx.x & (WAVE - 1)),
                               nchunks / 2 - 1);  // past the end: the last block, never used
        k0 = x[2 * b0];
        k1 = x[2 * b0 + 1];
    }
    TensorScale ts = tensor_scale<BF16>(partials, npart);
    if (blockIdx.x == 0 && threadIdx.x == 0) *global_scale = ts.s_g;
    if (ts.flags) {
        if (blockIdx.x == 0 && threadIdx.x == 0 && status) atomicOr(status, (int32_t)ts.flags);
        return;
    }
    uint32_t flags = 0;
    if constexpr (BF16) {
        SearchShared &S = *reinterpret_cast<SearchShared *>(smem);
        // the queue stores block indices in 32 bits
        if (search_table_build<ALL>(S.tab, ts, c_lo, c_hi) && (nchunks >> 33) == 0) {
            search_bf16_tiles<ALL>(S, x, nchunks / 2, k0, k1,
                                   (float)((double)c_hi / (6.0 * (double)ts.s_g)), codes, scales, flags);
            report_flags(status, flags);
            return;
        }
        // (uniform: no thread reads the search table again)
    }
    NvScaleTable &T = *reinterpret_cast<NvScaleTable *>(smem);
    nv_table_build(T, ts.s_g, recip_row<BF16>(ts));
    __syncthreads();
    const double inv6sg = 1.0 / (6.0 * (double)ts.s_g);
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_WG + (threadIdx.x / WAVE);
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    const int64_t ntiles = (nchunks + WAVE - 1) / WAVE;
    for (int64_t t = wave; t < ntiles; t += nwaves) {
        const int64_t c = t * WAVE + lane;
        Chunk<BF16> k = load_chunk<BF16>(x, c, c < nchunks);
        uint32_t m = chunk_amax<BF16>(k);
        m = max(m, dpp<QP_XOR1>(m));
        const uint32_t ag_bits = amax_as_f32_bits<BF16>(m);
        float a[8];
        chunk_values<BF16>(k, a);
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = __builtin_fabsf(a[i]);
        uint32_t best = 0x38u;
        if (ag_bits != 0) {
            const double ag = (double)u2f(ag_bits);
            uint32_t lo = ALL ? 1u : nv_code_real(T, (double)c_lo * ag, inv6sg);
            const uint32_t hi = ALL ? 126u : nv_code_real(T, (double)c_hi * ag, inv6sg);
            lo = lo < 1u ? 1u : lo;
            // Codes from the largest down; a loss equal to the incumbent's
            // replaces it, so the smallest code wins ties, as in increasing
            // order with strict improvement.  Every term of the loss is >= 0
            // and the fp32 pairwise sum of such terms is at least each of
            // them, so once the block maximum saturates (amax >= RN(6 alpha),
            // hence its quotient exceeds 5 and it quantizes to 6 alpha) its
            // own term RN(RN(amax - RN(6 alpha))^2) bounds the loss from
            // below; that bound only grows as the code falls, so the walk
            // stops at the first code whose bound exceeds the best loss.
            const float agf = u2f(ag_bits);
            float bestL = __builtin_inff();
            bool have = false;
            for (uint32_t code = hi; code >= lo; --code) {
                const float4 sq = T.q[code];
                const float x6 = 6.0f * sq.x;
                const float e6 = agf - x6;
                const float bound = agf >= x6 ? e6 * e6 : 0.0f;
                if (bound > bestL) break;
                // a code whose alpha underflowed to 0 is evaluated (its loss
                // is finite) but never taken
                float part = half_block_loss<BF16>(a, sq, T.yc[code]);
                float L = part + dppf<QP_XOR1>(part);
                if (sq.x != 0.0f && L <= bestL) {
                    best = code;
                    bestL = L;
                    have = true;
                }
            }
            if (!have) {
                flags |= FLAG_SCALE_UNDERFLOW;
                best = 0;
            }
        }
        const float4 sq = T.q[best];
        chunk_values<BF16>(k, a);
        uint32_t q = nv_quant8<BF16>(a, sq.y, sq.z, sq.w, T.yc[best]);
        if (c < nchunks) {
            codes[c] = q;
            if ((lane & 1) == 0) scales[c >> 1] = (uint8_t)best;
        }
    }
    report_flags(status, flags);
}

// ---------------------------------------------------------------------------
// Row-padded layout ("NVFP4 / MXFP4 format" page, section 8): each row of
// cols values is padded with zeros to whole blocks of the format, and codes
// and scales are those of the padded [rows, pcols] matrix; decoding crops
// each row back to cols.  Padded chunk c (8 values) is row c / cpr, columns
// (c % cpr) * 8 .. + 8 (cpr = pcols / 8); columns at or past cols read as 0.
// Rows need not be aligned, so values move one by one (this layout is for
// shapes the block-aligned kernels do not take).
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ uint32_t padded_values(const void *__restrict__ x, int64_t cols,
                                                  int64_t cpr, int64_t c, bool ok, float (&v)[8]) {
    const int64_t r = ok ? c / cpr : 0, j0 = ok ? (c % cpr) * 8 : 0;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t j = j0 + i;
        uint32_t b = 0;
        if (ok && j < cols)
            b = BF16 ? (uint32_t)((const uint16_t *)x)[r * cols + j] << 16
                     : ((const uint32_t *)x)[r * cols + j];
        v[i] = u2f(b);
        m = max(m, b & 0x7FFFFFFFu);
    }
    return m;  // fp32 pattern of the chunk amax (non-finite patterns sort above)
}

template <bool BF16>
__global__ __launch_bounds__(WG) void mx_quantize_padded_kernel(const void *__restrict__ x,
                                                                int64_t cols, int64_t cpr,
                                                                int64_t nchunks,
                                                                uint32_t *__restrict__ codes,
                                                                uint8_t *__restrict__ scales,
                                                                int32_t *status) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_WG + (threadIdx.x / WAVE);
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    uint32_t flags = 0;
    for (int64_t t = wave; t * WAVE < nchunks; t += nwaves) {
        const int64_t c = t * WAVE + lane;  // four lanes hold a block (cpr is a multiple of 4)
        float v[8];
        uint32_t m = padded_values<BF16>(x, cols, cpr, c, c < nchunks, v);
        m = max(m, dpp<QP_XOR1>(m));
        m = max(m, dpp<QP_XOR2>(m));
        if ((m >> 23) >= 0xFFu) flags |= FLAG_NONFINITE;
        const uint32_t sb = mx_scale_byte(m, 23);
        const uint32_t q = cvt_fp4x8_f32(v, e8m0_operand(sb));
        if (c < nchunks) {
            codes[c] = q;
            if ((lane & 3) == 0) scales[c >> 2] = (uint8_t)sb;
        }
    }
    report_flags(status, flags);
}

// NVFP4 pass 1 on the padded layout: one partial max (fp32 pattern) per
// workgroup; the zero padding changes no amax.
template <bool BF16>
__global__ __launch_bounds__(WG) void padded_amax_kernel(const void *__restrict__ x, int64_t cols,
                                                         int64_t cpr, int64_t nchunks,
                                                         uint32_t *__restrict__ partials) {
    __shared__ uint32_t red[WAVES_PER_WG];
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * WG;
    for (int64_t c = (int64_t)blockIdx.x * WG + threadIdx.x; c < nchunks; c += stride) {
        float v[8];
        m = max(m, padded_values<BF16>(x, cols, cpr, c, true, v));
    }
    m = wave_max_u32(m);
    if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
        for (int i = 1; i < WAVES_PER_WG; ++i) r = max(r, red[i]);
        partials[blockIdx.x] = r;
    }
}

// NVFP4 pass 2 on the padded layout: a lane pair holds a block; each lane
// derives the block scale (the same in both) and divides with the
// reciprocal-correction divide.
template <bool BF16>
__global__ __launch_bounds__(WG) void nv_quantize_padded_kernel(
    const void *__restrict__ x, int64_t cols, int64_t cpr, int64_t nchunks,
    const uint32_t *__restrict__ partials, int npart, uint32_t *__restrict__ codes,
    uint8_t *__restrict__ scales, float *__restrict__ global_scale, int32_t *status) {
    __shared__ NvScaleTable T;
    TensorScale ts = tensor_scale<false>(partials, npart);  // fp32 patterns
    if (blockIdx.x == 0 && threadIdx.x == 0) *global_scale = ts.s_g;
    if (ts.flags) {
        if (blockIdx.x == 0 && threadIdx.x == 0 && status) atomicOr(status, (int32_t)ts.flags);
        return;
    }
    nv_table_build(T, ts.s_g, -1);
    __syncthreads();
    const CodeGuess G = make_code_guess(ts.s_g);
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t wave = (int64_t)blockIdx.x * WAVES_PER_WG + (threadIdx.x / WAVE);
    const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
    uint32_t flags = 0;
    for (int64_t t = wave; t * WAVE < nchunks; t += nwaves) {
        const int64_t c = t * WAVE + lane;
        float v[8];
        uint32_t m = padded_values<BF16>(x, cols, cpr, c, c < nchunks, v);
        m = max(m, dpp<QP_XOR1>(m));
        const BlockScale b = nv_block_scale(T, m, G, flags);
        const uint32_t q = nv_quant8<false>(v, b.ad, b.y, b.sc, b.yc);
        if (c < nchunks) {
            codes[c] = q;
            if ((lane & 1) == 0) scales[c >> 1] = (uint8_t)b.code;
        }
    }
    report_flags(status, flags);
}

// Decode of the padded layout, cropped to cols per row: the values of
// dequant_chunk, stored one by one.
template <int FMT, bool OUT_BF16>
__global__ __launch_bounds__(WG) void dequant_padded_kernel(const uint32_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            const float *__restrict__ global_scale,
                                                            int64_t cols, int64_t cpr,
                                                            int64_t nchunks, void *__restrict__ y) {
    const float s_g = (FMT == 1) ? *global_scale : 1.0f;
    const int64_t stride = (int64_t)gridDim.x * WG;
    for (int64_t c = (int64_t)blockIdx.x * WG + threadIdx.x; c < nchunks; c += stride) {
        const uint32_t q = codes[c];
        const uint32_t sb = scales[FMT == 0 ? (c >> 2) : (c >> 1)];
        const float so = FMT == 0 ? e8m0_operand(sb) : e8m0_operand(E8M0_ONE);
        const float alpha = FMT == 0 ? 1.0f : s_g * e4m3_any_value(sb);
        float v[8];
        const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, so, 0);
        const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, so, 1);
        const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, so, 2);
        const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, so, 3);
        v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
        v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
        const int64_t r = c / cpr, j0 = (c % cpr) * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float o = FMT == 0 ? v[i] : v[i] * alpha;
            if (FMT == 0 && sb == 0xFFu) o = __builtin_nanf("");
            const int64_t j = j0 + i;
            if (j < cols) {
                if (OUT_BF16) ((uint16_t *)y)[r * cols + j] = (uint16_t)bf16_rne(o);
                else ((float *)y)[r * cols + j] = o;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline int grid_for(int64_t waves_needed, int max_wg) {
    int64_t g = (waves_needed + WAVES_PER_WG - 1) / WAVES_PER_WG;
    if (g > max_wg) g = max_wg;
    return (int)(g < 1 ? 1 : g);
}

hipError_t launch_mx_quantize(const void *x, bool bf16, int64_t n, int rule, uint8_t *codes,
                              uint8_t *scales, int32_t *status, hipStream_t s) {
    const int64_t nchunks = n / 8;
    const int g = grid_for((nchunks + WAVE * 4 - 1) / (WAVE * 4), kMaxGrid);
    using K = void (*)(const uint4 *, int64_t, uint32_t *, uint8_t *, int32_t *);
    static const K kernels[2][3] = {
        {mx_quantize_kernel<false, 0>, mx_quantize_kernel<false, 1>, mx_quantize_kernel<false, 2>},
        {mx_quantize_kernel<true, 0>, mx_quantize_kernel<true, 1>, mx_quantize_kernel<true, 2>}};
    hipLaunchKernelGGL(kernels[bf16 ? 1 : 0][rule], dim3(g), dim3(WG), 0, s, (const uint4 *)x,
                       nchunks, (uint32_t *)codes, scales, status);
    return hipGetLastError();
}

hipError_t launch_mx_quantize_packed(const void *x, bool bf16, int64_t rows, int64_t cols,
                                     uint8_t *packed, int32_t *status, hipStream_t s) {
    const int64_t nrt = (rows + 31) / 32, ntiles = nrt * (cols / 64);
    int64_t g = (ntiles + WAVES_PER_WG - 1) / WAVES_PER_WG;
    if (g > kMaxGrid) g = kMaxGrid;
    uint8_t *scales = packed + nrt * 32 * (cols / 2);
    auto k = bf16 ? mx_quantize_packed_kernel<true> : mx_quantize_packed_kernel<false>;
    hipLaunchKernelGGL(k, dim3((unsigned)g), dim3(WG), 0, s, (const uint4 *)x, rows, cols, ntiles,
                       (uint4 *)packed, scales, status);
    return hipGetLastError();
}

// CUs of the current device, probed once per device (0 if unknown).
static int device_cus() {
    static int cus[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::call_once(once[dev], [dev] {
        int c = 0;
        cus[dev] = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                           c > 0 ? c : 0;
    });
    return cus[dev];
}

// Workgroups of the tensor-amax pass, each looping over its share four
// chunks per lane at a time: up to kAmaxPartials, or with two_per_cu at
// most two per CU.  The two-pass fp32 NVFP4 quantize takes the latter
// (8192 x 8192: 105.1 -> 100.2 us, paired timing).  Two per CU make the
// pass alone faster for bf16 too (117 MB in 18.7 us against 21.4 us), but
// the scale search and the stochastic NVFP4 quantize that follow it then
// measured ~6 us slower per call, so the other passes keep the wide grid.
static int amax_grid(int64_t nchunks, bool two_per_cu) {
    int64_t g = (nchunks + WG * 4 - 1) / (WG * 4);
    const int cus = two_per_cu ? device_cus() : 0;
    if (cus > 0 && g > 2 * (int64_t)cus) g = 2 * (int64_t)cus;
    if (g > kAmaxPartials) g = kAmaxPartials;
    return (int)(g < 1 ? 1 : g);
}


// Whether the one-pass resident kernel can run on the current device, and on
// how many CUs: one workgroup per CU must fit (so the whole grid is resident
// at once).  Probed once per device.
struct ResidentInfo {
    int cus;  // 0: not available
};

static ResidentInfo resident_info() {
    static ResidentInfo info[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ResidentInfo{0};
    std::call_once(once[dev], [dev] {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        // the largest instance bounds the resources of all of them
        auto largest = nv_resident_kernel<RES_MAX_CHUNKS, false>;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, largest,
                                                         RES_WG, 0) != hipSuccess ||
            per_cu < 1)
            cus = 0;
        info[dev].cus = cus > kResidentSlots ? 0 : cus;
    });
    return info[dev];
}

// The tensor-amax pass: the wide kernel (one workgroup per CU, every load
// issued at once) for a bf16 tensor of 8 to 64 chunks per lane on the CUs
// the one-pass quantize may use, else tensor_amax_kernel.  g is the number
// of partials it writes.
struct AmaxPlan {
    int g;
    int cpl;  // chunks per lane of the wide kernel, a multiple of 8; 0: the other kernel
};

static AmaxPlan amax_plan(int64_t nchunks, bool bf16, bool two_per_cu) {
    if (bf16) {
        const int cus = resident_info().cus;
        const int64_t per = (int64_t)cus * RES_WG;  // chunks one row of the grid covers
        if (cus > 0 && cus <= kAmaxPartials && nchunks >= per * 8 && nchunks <= per * RES_MAX_CHUNKS) {
            const int cpl = (int)((nchunks + per * 8 - 1) / (per * 8)) * 8;
            const int g = (int)((nchunks + (int64_t)cpl * RES_WG - 1) / ((int64_t)cpl * RES_WG));
            return {g, cpl};
        }
    }
    return {amax_grid(nchunks, two_per_cu), 0};
}

static hipError_t launch_amax(const void *x, bool bf16, int64_t nchunks, uint32_t *partials,
                              const AmaxPlan &p, hipStream_t s) {
    const dim3 g((unsigned)p.g);
    const uint4 *xv = (const uint4 *)x;
    switch (p.cpl) {
        case 0:
            if (bf16) hipLaunchKernelGGL(tensor_amax_kernel<true>, g, dim3(WG), 0, s, xv, nchunks, partials);
            else hipLaunchKernelGGL(tensor_amax_kernel<false>, g, dim3(WG), 0, s, xv, nchunks, partials);
            break;
#define FP4_WIDE(C) \
    case C: hipLaunchKernelGGL(tensor_amax_wide_kernel<C>, g, dim3(RES_WG), 0, s, xv, nchunks, partials); break
        FP4_WIDE(8); FP4_WIDE(16); FP4_WIDE(24); FP4_WIDE(32);
        FP4_WIDE(40); FP4_WIDE(48); FP4_WIDE(56); FP4_WIDE(64);
#undef FP4_WIDE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}


hipError_t launch_nv_quantize_packed(const void *x, bool bf16, int64_t rows, int64_t cols,
                                     uint8_t *packed, float *global_scale, void *workspace,
                                     int32_t *status, hipStream_t s) {
    const int64_t nrt = (rows + 31) / 32, ntiles = nrt * (cols / 64);
    uint32_t *partials = (uint32_t *)workspace;
    const AmaxPlan ap = amax_plan(rows * cols / 8, bf16, false);
    const int g1 = ap.g;
    hipError_t e = launch_amax(x, bf16, rows * cols / 8, partials, ap, s);
    if (e != hipSuccess) return e;
    int64_t g = (ntiles + WAVES_PER_WG - 1) / WAVES_PER_WG;
    if (g > kMaxGrid) g = kMaxGrid;
    uint16_t *scales = (uint16_t *)(packed + nrt * 32 * (cols / 2));
    auto k = bf16 ? nv_quantize_packed_kernel<true> : nv_quantize_packed_kernel<false>;
    hipLaunchKernelGGL(k, dim3((unsigned)g), dim3(WG), 0, s, (const uint4 *)x, rows, cols, ntiles,
                       partials, g1, (uint4 *)packed, scales, global_scale, status);
    return hipGetLastError();
}

template <int CPL>
static void launch_resident(int g, const void *x, int64_t nchunks, uint8_t *codes,
                            uint8_t *scales, float *global_scale, uint8_t *ws, int32_t *status,
                            hipStream_t s, uint32_t spin_limit) {
    const bool exact = nchunks == (int64_t)g * CPL * RES_WG;
    auto kernel = exact ? nv_resident_kernel<CPL, true> : nv_resident_kernel<CPL, false>;
    hipLaunchKernelGGL(kernel, dim3(g), dim3(RES_WG), 0, s, (const uint4 *)x,
                       (int)nchunks, (uint32_t *)codes, scales, global_scale,
                       (uint64_t *)(ws + kResidentSlotsOffset),
                       (uint32_t *)(ws + kResidentEpochOffset), spin_limit, status);
}

hipError_t launch_nv_quantize(const void *x, bool bf16, int64_t n, uint8_t *codes,
                              uint8_t *scales, float *global_scale, void *workspace,
                              int32_t *status, hipStream_t s, uint32_t spin_limit) {
    const int64_t nchunks = n / 8;
    if (bf16) {
        const ResidentInfo ri = resident_info();
        const int64_t per_step = (int64_t)ri.cus * RES_WG;  // chunks one step of a full grid covers
        if (ri.cus > 0 && nchunks <= per_step * RES_MAX_CHUNKS) {
            // fewest chunks per lane (a row pair at least) that fit on the CUs
            int cpl = 8;
            while ((int64_t)cpl * per_step < nchunks) cpl *= 2;
            const int g = (int)((nchunks + (int64_t)cpl * RES_WG - 1) / ((int64_t)cpl * RES_WG));
            uint8_t *ws = (uint8_t *)workspace;
            switch (cpl) {
                case 8: launch_resident<8>(g, x, nchunks, codes, scales, global_scale, ws, status, s, spin_limit); break;
                case 16: launch_resident<16>(g, x, nchunks, codes, scales, global_scale, ws, status, s, spin_limit); break;
                case 32: launch_resident<32>(g, x, nchunks, codes, scales, global_scale, ws, status, s, spin_limit); break;
                default: launch_resident<64>(g, x, nchunks, codes, scales, global_scale, ws, status, s, spin_limit); break;
            }
            return hipGetLastError();
        }
    }
    uint32_t *partials = (uint32_t *)workspace;
    const AmaxPlan ap = amax_plan(nchunks, bf16, !bf16);
    const int g1 = ap.g;
    hipError_t e = launch_amax(x, bf16, nchunks, partials, ap, s);
    if (e != hipSuccess) return e;
    const int g = grid_for((nchunks + WAVE * 2 - 1) / (WAVE * 2), kMaxGrid);
    auto kernel = bf16 ? nv_quantize_kernel<true, false> : nv_quantize_kernel<false, false>;
    hipLaunchKernelGGL(kernel, dim3(g), dim3(WG), 0, s, (const uint4 *)x, nchunks, partials, g1,
                       (uint64_t)0, (uint32_t *)codes, scales, global_scale, status);
    return hipGetLastError();
}

hipError_t launch_quantize_sr(int fmt, const void *x, bool bf16, int64_t n, uint64_t seed,
                              uint8_t *codes, uint8_t *scales, float *global_scale,
                              void *workspace, int32_t *status, hipStream_t s) {
    const int64_t nchunks = n / 8;
    if (fmt == 0) {
        const int g = grid_for((nchunks + WAVE * 4 - 1) / (WAVE * 4), kMaxGrid);
        auto kernel = bf16 ? mx_quantize_sr_kernel<true> : mx_quantize_sr_kernel<false>;
        hipLaunchKernelGGL(kernel, dim3(g), dim3(WG), 0, s, (const uint4 *)x, nchunks, seed,
                           (uint32_t *)codes, scales, status);
        return hipGetLastError();
    }
    uint32_t *partials = (uint32_t *)workspace;
    const AmaxPlan ap = amax_plan(nchunks, bf16, false);
    const int g1 = ap.g;
    hipError_t e = launch_amax(x, bf16, nchunks, partials, ap, s);
    if (e != hipSuccess) return e;
    const int g = grid_for((nchunks + WAVE * 2 - 1) / (WAVE * 2), kMaxGrid);
    auto kernel = bf16 ? nv_quantize_kernel<true, true> : nv_quantize_kernel<false, true>;
    hipLaunchKernelGGL(kernel, dim3(g), dim3(WG), 0, s, (const uint4 *)x, nchunks, partials, g1,
                       seed, (uint32_t *)codes, scales, global_scale, status);
    return hipGetLastError();
}

// Workgroups of the bf16 search resident at once on the current device
// (kMaxGrid if the device cannot be queried).  Probed once per device.
static int search_grid_cap() {
    static int cap[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kMaxGrid;
    std::call_once(once[dev], [dev] {
        int cus = 0, per_cu = 0;
        cap[dev] = kMaxGrid;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scale_search_kernel<true, false>, WG,
                                                         0) == hipSuccess &&
            cus > 0 && per_cu > 0)
            cap[dev] = cus * per_cu < kMaxGrid ? cus * per_cu : kMaxGrid;
    });
    return cap[dev];
}

hipError_t launch_scale_search(const void *x, bool bf16, int64_t n, bool all, float c_lo,
                               float c_hi, uint8_t *codes, uint8_t *scales, float *global_scale,
                               void *workspace, int32_t *status, hipStream_t s) {
    const int64_t nchunks = n / 8;
    uint32_t *partials = (uint32_t *)workspace;
    const AmaxPlan ap = amax_plan(nchunks, bf16, false);
    const int g1 = ap.g;
    hipError_t e = launch_amax(x, bf16, nchunks, partials, ap, s);
    if (e != hipSuccess) return e;
    using K = void (*)(const uint4 *, int64_t, const uint32_t *, int, float, float, uint32_t *,
                       uint8_t *, float *, int32_t *);
    static const K kernels[2][2] = {
        {scale_search_kernel<false, false>, scale_search_kernel<false, true>},
        {scale_search_kernel<true, false>, scale_search_kernel<true, true>}};
    // bf16: at most the workgroups the device holds at once (each sets up its
    // tables once and its waves drain their queues once)
    const int g = grid_for((nchunks + WAVE - 1) / WAVE, bf16 ? search_grid_cap() : kMaxGrid);
    hipLaunchKernelGGL(kernels[bf16 ? 1 : 0][all ? 1 : 0], dim3(g), dim3(WG), 0, s,
                       (const uint4 *)x, nchunks, partials, g1, c_lo, c_hi, (uint32_t *)codes,
                       scales, global_scale, status);
    return hipGetLastError();
}

hipError_t launch_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales,
                             const float *global_scale, int64_t n, void *y, bool out_bf16,
                             hipStream_t s) {
    const int64_t nchunks = n / 8;
#define FP4_DQ(F, B)                                                                          \
    hipLaunchKernelGGL((dequant_kernel<F, B>),                                                \
                       dim3(grid_for((nchunks + WAVE * DequantShape<F, B>::U - 1) /            \
                                         (WAVE * DequantShape<F, B>::U),                       \
                                     DequantShape<F, B>::G)),                                  \
                       dim3(WG), 0, s, (const uint32_t *)codes, scales, global_scale, nchunks, \
                       (uint4 *)y)
    if (fmt == 0) {
        if (out_bf16) FP4_DQ(0, true);
        else FP4_DQ(0, false);
    } else {
        if (out_bf16) FP4_DQ(1, true);
        else FP4_DQ(1, false);
    }
#undef FP4_DQ
    return hipGetLastError();
}

hipError_t launch_quantize_padded(int fmt, const void *x, bool bf16, int64_t rows, int64_t cols,
                                  uint8_t *codes, uint8_t *scales, float *global_scale,
                                  void *workspace, int32_t *status, hipStream_t s) {
    const int block = fmt == 0 ? 32 : 16;
    const int64_t pcols = (cols + block - 1) / block * block;
    const int64_t cpr = pcols / 8, nchunks = rows * cpr;
    const int g = grid_for((nchunks + WAVE - 1) / WAVE, kMaxGrid);
    if (fmt == 0) {
        auto k = bf16 ? mx_quantize_padded_kernel<true> : mx_quantize_padded_kernel<false>;
        hipLaunchKernelGGL(k, dim3(g), dim3(WG), 0, s, x, cols, cpr, nchunks, (uint32_t *)codes,
                           scales, status);
        return hipGetLastError();
    }
    uint32_t *partials = (uint32_t *)workspace;
    const int g1 = amax_grid(nchunks, false);
    auto ka = bf16 ? padded_amax_kernel<true> : padded_amax_kernel<false>;
    hipLaunchKernelGGL(ka, dim3(g1), dim3(WG), 0, s, x, cols, cpr, nchunks, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    auto kq = bf16 ? nv_quantize_padded_kernel<true> : nv_quantize_padded_kernel<false>;
    hipLaunchKernelGGL(kq, dim3(g), dim3(WG), 0, s, x, cols, cpr, nchunks, partials, g1,
                       (uint32_t *)codes, scales, global_scale, status);
    return hipGetLastError();
}

hipError_t launch_dequantize_padded(int fmt, const uint8_t *codes, const uint8_t *scales,
                                    const float *global_scale, int64_t rows, int64_t cols,
                                    void *y, bool out_bf16, hipStream_t s) {
    const int block = fmt == 0 ? 32 : 16;
    const int64_t cpr = (cols + block - 1) / block * block / 8, nchunks = rows * cpr;
    const int g = grid_for((nchunks + WAVE - 1) / WAVE, kMaxGrid);
    using K = void (*)(const uint32_t *, const uint8_t *, const float *, int64_t, int64_t,
                       int64_t, void *);
    static const K kernels[2][2] = {{dequant_padded_kernel<0, false>, dequant_padded_kernel<0, true>},
                                    {dequant_padded_kernel<1, false>, dequant_padded_kernel<1, true>}};
    hipLaunchKernelGGL(kernels[fmt][out_bf16 ? 1 : 0], dim3(g), dim3(WG), 0, s,
                       (const uint32_t *)codes, scales, global_scale, cols, cpr, nchunks, y);
    return hipGetLastError();
}

}  // namespace fp4dev
