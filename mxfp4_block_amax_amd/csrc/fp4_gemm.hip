// fp4_gemm.hip - MXFP4 x MXFP4 block-scaled GEMM on gfx950 scaled MFMA.
//
// C[m, n] = sum over 32-blocks t of 2^(ea[m,t]-127) 2^(eb[n,t]-127)
//           * sum_{k in t} pA[m, k] pB[n, k]
// ("FP4, FP8 and INT8/INT4" page, tom-jerr.github.io, section 5.1: each K
// block multiplies its own pair of scales, accumulation in fp32; "NVFP4 /
// MXFP4 format" page, section 6: B stored as N x K so its last-dimension
// blocks are the K blocks).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E2M1 (cbsz = blgp = 4)
// takes a 32 x 64 slice of A and a 64 x 32 slice of B.  Lane l supplies row
// (or column) l % 32 and the 32 consecutive K values starting at 32 (l / 32):
// exactly one MX block, 16 packed bytes, with that block's E8M0 byte as the
// lane's scale operand.  The hardware applies each lane's scale to its own
// block, so the per-block scaling of the formula happens inside the MFMA and
// the fp32 accumulator spans all of K.
//
// Work split: a workgroup (4 waves) owns a 128 x 32 tile of C and walks all
// of K; wave w owns rows 32w..32w+31.  B (N x K, the large operand at M=128)
// is read from HBM once in total; A is re-read by every workgroup from L2.
// The K loop is unrolled with a register prefetch of the next steps' codes.
#include "fp4_device.h"
#include "fp4_kernels.h"

namespace fp4dev {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int GEMM_WG = 256;
constexpr int GEMM_TM = 128;  // rows of C per workgroup
constexpr int GEMM_TN = 32;   // columns of C per workgroup
constexpr int GEMM_PD = 8;    // K steps (of 64) loaded ahead

__device__ __forceinline__ i32x8_t as_operand(uint4 v) {
    i32x8_t r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    return r;
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x40u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(GEMM_WG) void mxfp4_gemm_kernel(
    const uint4 *__restrict__ A, const uint8_t *__restrict__ As, const uint4 *__restrict__ Bt,
    const uint8_t *__restrict__ Bs, int M, int N, int K, void *__restrict__ C) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r32 = lane & 31;  // operand row / column within the 32-slice
    const int kh = lane >> 5;   // which 32-block of the 64-wide K step
    const int am = blockIdx.y * GEMM_TM + w * 32 + r32;
    const int bn = blockIdx.x * GEMM_TN + r32;
    const bool aok = am < M, bok = bn < N;
    const int nblk = K / 32;                 // K blocks per row
    const int nsteps = (nblk + 1) / 2;       // 64-wide K steps
    const uint4 *arow = A + (int64_t)(aok ? am : 0) * nblk;
    const uint4 *brow = Bt + (int64_t)(bok ? bn : 0) * nblk;
    const uint8_t *asr = As + (int64_t)(aok ? am : 0) * nblk;
    const uint8_t *bsr = Bs + (int64_t)(bok ? bn : 0) * nblk;

    f32x16_t acc = {};
    uint4 ra[GEMM_PD], rb[GEMM_PD];
    uint32_t sa[GEMM_PD], sb[GEMM_PD];
    const uint4 z = make_uint4(0, 0, 0, 0);

    auto fetch = [&](int s, int slot) {
        const int blk = 2 * s + kh;
        const bool in = blk < nblk;
        ra[slot] = (aok && in) ? arow[blk] : z;
        rb[slot] = (bok && in) ? ld_stream(brow + blk) : z;
        sa[slot] = (aok && in) ? (uint32_t)asr[blk] : 127u;
        sb[slot] = (bok && in) ? (uint32_t)bsr[blk] : 127u;
    };

#pragma unroll
    for (int p = 0; p < GEMM_PD; ++p) fetch(p, p);

    for (int s0 = 0; s0 < nsteps; s0 += GEMM_PD) {
#pragma unroll
        for (int p = 0; p < GEMM_PD; ++p) {
            const int s = s0 + p;
            if (s < nsteps) {
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    as_operand(ra[p]), as_operand(rb[p]), acc, 4, 4, 0, (int)sa[p], 0, (int)sb[p]);
            }
            if (s + GEMM_PD < nsteps) fetch(s + GEMM_PD, p);
        }
    }

    // accumulator layout of the 32x32 MFMA: lane l holds column l % 32 and
    // rows 8 (j / 4) + 4 (l / 32) + (j % 4), j = 0..15
    const int col = blockIdx.x * GEMM_TN + r32;
    if (col >= N) return;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int row = blockIdx.y * GEMM_TM + w * 32 + 8 * (j / 4) + 4 * kh + (j % 4);
        if (row < M) {
            if (OUT_BF16)
                ((uint16_t *)C)[(int64_t)row * N + col] = (uint16_t)bf16_rne_bits(acc[j]);
            else
                ((float *)C)[(int64_t)row * N + col] = acc[j];
        }
    }
}

// ---------------------------------------------------------------------------
// Fast path (K a multiple of 2048; code rows 16-byte and scale rows 8-byte
// aligned).  A workgroup still owns a 128 x 32 tile of C, but its four waves
// split K into quarters instead of splitting M: each wave runs all four
// 32-row slices of A against the one 32-column slice of B over its quarter,
// so every A and B byte the workgroup needs is loaded exactly once, by one
// lane.  Loads are unpredicated (rows past M / columns past N are clamped to
// the last valid one and their results discarded) and software-pipelined
// two groups of four K steps deep in registers.  The four partial tiles are
// summed through LDS in a fixed order (wave 0 + 1 + 2 + 3), so results are
// deterministic.
// ---------------------------------------------------------------------------
constexpr int GF_G = 4;  // K steps per load group

struct GemmGroup {
    uint4 a[GF_G][4];  // [step][32-row slice]
    uint4 b[GF_G];
    uint2 sa[4];       // 8 scale bytes = 4 steps x 2 K-halves, per row slice
    uint2 sb;
};

__device__ __forceinline__ void gemm_load_group(GemmGroup &g, const uint4 *const (&pa)[4],
                                                const uint4 *pb, const uint2 *const (&psa)[4],
                                                const uint2 *psb, int s, int rot, int steps_w) {
    // visit this wave's K range starting at a workgroup-dependent offset
    s += rot;
    if (s >= steps_w) s -= steps_w;
    // step s (a multiple of GF_G): lane reads block 2s' + kh of its rows
#pragma unroll
    for (int p = 0; p < GF_G; ++p) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) g.a[p][mi] = pa[mi][2 * (s + p)];
        g.b[p] = ld_stream(pb + 2 * (s + p));
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) g.sa[mi] = psa[mi][s / GF_G];
    g.sb = psb[s / GF_G];
}

__device__ __forceinline__ uint32_t scale_byte(uint2 w, int p, int kh) {
    // byte 2p + kh of the 8-byte group; the MFMA reads the low byte
    const int i = 2 * p + kh;
    return (i < 4 ? w.x : w.y) >> (8 * (i & 3));
}

__device__ __forceinline__ void gemm_mma_group(f32x16_t (&acc)[4], const GemmGroup &g, int kh) {
#pragma unroll
    for (int p = 0; p < GF_G; ++p) {
        const int sb = (int)scale_byte(g.sb, p, kh);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                as_operand(g.a[p][mi]), as_operand(g.b[p]), acc[mi], 4, 4, 0,
                (int)scale_byte(g.sa[mi], p, kh), 0, sb);
    }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(GEMM_WG) void mxfp4_gemm_fast_kernel(
    const uint4 *__restrict__ A, const uint8_t *__restrict__ As, const uint4 *__restrict__ Bt,
    const uint8_t *__restrict__ Bs, int M, int N, int K, void *__restrict__ C) {
    __shared__ float part[4][4][16][64];  // [wave][row slice][acc element][lane]
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r32 = lane & 31;
    const int kh = lane >> 5;
    const int nblk = K / 32;
    const int steps_w = K / 64 / 4;  // K steps per wave (a multiple of 2 * GF_G)
    const int s0 = w * steps_w;
    const int bn = min((int)blockIdx.x * GEMM_TN + r32, N - 1);

    const uint4 *pa[4];
    const uint2 *psa[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int am = min((int)blockIdx.y * GEMM_TM + 32 * mi + r32, M - 1);
        pa[mi] = A + (int64_t)am * nblk + 2 * s0 + kh;
        psa[mi] = (const uint2 *)(As + (int64_t)am * nblk + 2 * s0);
    }
    const uint4 *pb = Bt + (int64_t)bn * nblk + 2 * s0 + kh;
    const uint2 *psb = (const uint2 *)(Bs + (int64_t)bn * nblk + 2 * s0);

    // Workgroups start their K walk at different groups so that they do not
    // all read the same lines of A (L2-resident, shared by every workgroup)
    // at the same time.  The order is a fixed function of the tile.
    const int ngroups2 = steps_w / (2 * GF_G);
    const int rot = (int)((blockIdx.x + 3u * blockIdx.y) % (unsigned)ngroups2) * (2 * GF_G);

    f32x16_t acc[4] = {};
    GemmGroup g0, g1;
    gemm_load_group(g0, pa, pb, psa, psb, 0, rot, steps_w);
    for (int s = 0; s < steps_w; s += 2 * GF_G) {
        gemm_load_group(g1, pa, pb, psa, psb, s + GF_G, rot, steps_w);
        // keep each group's loads ahead of the MFMAs that do not need them:
        // without the fence the scheduler sinks them next to their uses
        __builtin_amdgcn_sched_barrier(0);
        gemm_mma_group(acc, g0, kh);
        // unconditional prefetch (the last round re-reads group 0, in bounds),
        // so no branch splits the load counting of the pipeline
        const int sn = (s + 2 * GF_G < steps_w) ? s + 2 * GF_G : 0;
        gemm_load_group(g0, pa, pb, psa, psb, sn, rot, steps_w);
        __builtin_amdgcn_sched_barrier(0);
        gemm_mma_group(acc, g1, kh);
    }

    // fixed-order reduction of the four K-quarter partials
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 16; ++j) part[w][mi][j][lane] = acc[mi][j];
    __syncthreads();
    const int mi = w;  // wave w finishes row slice w
    const int col = blockIdx.x * GEMM_TN + r32;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float v = part[0][mi][j][lane];
        v = v + part[1][mi][j][lane];
        v = v + part[2][mi][j][lane];
        v = v + part[3][mi][j][lane];
        const int row = blockIdx.y * GEMM_TM + 32 * mi + 8 * (j / 4) + 4 * kh + (j % 4);
        if (row < M && col < N) {
            if (OUT_BF16)
                ((uint16_t *)C)[(int64_t)row * N + col] = (uint16_t)bf16_rne_bits(v);
            else
                ((float *)C)[(int64_t)row * N + col] = v;
        }
    }
}

static bool gemm_fast_ok(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *bt_codes,
                         const uint8_t *bt_scales, int64_t K) {
    auto al = [](const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; };
    return K % 2048 == 0 && al(a_codes, 16) && al(bt_codes, 16) && al(a_scales, 8) &&
           al(bt_scales, 8);
}

hipError_t launch_gemm_mxfp4(const uint8_t *a_codes, const uint8_t *a_scales,
                             const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t M,
                             int64_t N, int64_t K, void *c, bool out_bf16, hipStream_t s) {
    dim3 grid((unsigned)((N + GEMM_TN - 1) / GEMM_TN), (unsigned)((M + GEMM_TM - 1) / GEMM_TM));
    if (gemm_fast_ok(a_codes, a_scales, bt_codes, bt_scales, K)) {
        if (out_bf16)
            hipLaunchKernelGGL(mxfp4_gemm_fast_kernel<true>, grid, dim3(GEMM_WG), 0, s,
                               (const uint4 *)a_codes, a_scales, (const uint4 *)bt_codes,
                               bt_scales, (int)M, (int)N, (int)K, c);
        else
            hipLaunchKernelGGL(mxfp4_gemm_fast_kernel<false>, grid, dim3(GEMM_WG), 0, s,
                               (const uint4 *)a_codes, a_scales, (const uint4 *)bt_codes,
                               bt_scales, (int)M, (int)N, (int)K, c);
        return hipGetLastError();
    }
    if (out_bf16)
        hipLaunchKernelGGL(mxfp4_gemm_kernel<true>, grid, dim3(GEMM_WG), 0, s,
                           (const uint4 *)a_codes, a_scales, (const uint4 *)bt_codes, bt_scales,
                           (int)M, (int)N, (int)K, c);
    else
        hipLaunchKernelGGL(mxfp4_gemm_kernel<false>, grid, dim3(GEMM_WG), 0, s,
                           (const uint4 *)a_codes, a_scales, (const uint4 *)bt_codes, bt_scales,
                           (int)M, (int)N, (int)K, c);
    return hipGetLastError();
}

}  // namespace fp4dev
