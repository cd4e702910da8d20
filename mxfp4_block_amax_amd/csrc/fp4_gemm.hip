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
// Kernels here:
//  - mxfp4_gemm_lds_kernel: a workgroup (4 waves) owns a 128 x 32 tile of C
//    and walks all of K, staged through an LDS ring; wave w owns rows
//    32w..32w+31.  B (N x K, the large operand at M = 128) is read from HBM
//    once in total; A is re-read by every workgroup from L2.
//  - mxfp4_gemm_fast_kernel (register-fed) and mxfp4_gemm_kernel (one K step
//    at a time): the same product for shapes the staged kernel does not take.
//  - mxfp4_gemm_splitk_kernel + splitk_reduce_kernel: 128 x 128 tiles over
//    K ranges, fp32 partials, a fixed-order reduction.
//  - nvfp4_gemm_lds_kernel / nvfp4_gemm_simple_kernel: NVFP4 x NVFP4 on the
//    fp16 MFMA.
//  - mxfp4_linear_kernel: activation quantize + the staged GEMM in one launch.
#include <mutex>
#include <type_traits>

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

// ---------------------------------------------------------------------------
// MFMA operand order ("packed" layout).  An MXFP4 matrix X with R rows and K
// values per row is rearranged so that one 64-lane load of 16 bytes per lane
// is exactly one operand of the scaled MFMA:
//   codes:  row tile rt (32 rows; rows past R are zero), K step ks (64
//           values): 1024 bytes in which lane l holds row 32 rt + l % 32,
//           K block 2 ks + l / 32 (that block's 16 code bytes);
//   scales: after all codes; per row tile and group q of eight K steps, 512
//           bytes in which byte 8 l + i is the E8M0 byte of lane l's row and
//           K half in step 8 q + i, i.e. of block 2 (8 q + i) + l / 32 (127
//           on padding rows).
// Weights are packed once; each operand load of the GEMM below is then one
// contiguous kilobyte, instead of 32 rows x 32 bytes at the row stride, the
// pattern that keeps the address unit of the register-fed kernel above busy.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint4 *__restrict__ codes,
                                                         int64_t rows, int64_t nks,
                                                         int64_t total, uint4 *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int l = (int)(i & 63);
        const int64_t t = i >> 6, ks = t % nks, rt = t / nks;
        const int64_t r = rt * 32 + (l & 31);
        out[i] = r < rows ? codes[r * (2 * nks) + 2 * ks + (l >> 5)] : make_uint4(0, 0, 0, 0);
    }
}

__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t *__restrict__ scales,
                                                          int64_t rows, int64_t nks,
                                                          int64_t total, uint32_t *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t nkq = nks / 8;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int j = (int)(i & 1), l = (int)((i >> 1) & 63);
        const int64_t t = i >> 7, q = t % nkq, rt = t / nkq;
        const int64_t r = rt * 32 + (l & 31);
        uint32_t v = 0x7F7F7F7Fu;
        if (r < rows) {
            // steps 8 q + 4 j + b, b = 0..3: blocks 2 step + l / 32
            const uint8_t *s = scales + r * (2 * nks) + 2 * (8 * q + 4 * j) + (l >> 5);
            v = (uint32_t)s[0] | ((uint32_t)s[2] << 8) | ((uint32_t)s[4] << 16) | ((uint32_t)s[6] << 24);
        }
        out[i] = v;
    }
}

constexpr int PK_RING = 8;  // K steps in flight per wave

// The GEMM on packed operands.  A workgroup owns a 128 x 32 tile of C; wave w
// takes the w-th quarter of the K steps (SW = K / 256 of them) for all four
// 32-row slices of A against the 32 columns of B.  The K walk is unrolled:
// step st's five code loads (four A slices, one B) sit in ring slot st % 8,
// issued eight steps ahead, so the load waits are exact constants; each
// wave's scales (one 8-byte load per operand per eight steps) stay in
// registers.  The four partial tiles are summed through LDS in a fixed order
// (wave 0 + 1 + 2 + 3), so results are deterministic.
template <bool OUT_BF16, int SW>
__global__ __launch_bounds__(GEMM_WG) void mxfp4_gemm_packed_kernel(
    const uint4 *__restrict__ Ap, const uint4 *__restrict__ Asp, const uint4 *__restrict__ Bp,
    const uint4 *__restrict__ Bsp, int M, int N, void *__restrict__ C) {
    constexpr int R = PK_RING;
    constexpr int NQ = SW / 8;  // scale loads (8 steps each) per operand
    constexpr int nks = 4 * SW, nkq = nks / 8;
    __shared__ float part[4][4][16][64];  // [wave][row slice][acc element][lane]
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31;
    const int kh = lane >> 5;
    const int s0 = w * SW;
    const int nrt_a = (M + 31) / 32, nrt_b = (N + 31) / 32;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)Ap, (short)0, nrt_a * nks * 1024, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)Bp, (short)0, nrt_b * nks * 1024, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void *)Asp, (short)0, nrt_a * nkq * 512, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void *)Bsp, (short)0, nrt_b * nkq * 512, kBufferRsrcWord3);
    const int vo = lane * 16;
    int oa[4], osa[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int rt = min((int)blockIdx.y * 4 + mi, nrt_a - 1);
        oa[mi] = (rt * nks + s0) * 1024;
        osa[mi] = (rt * nkq + s0 / 8) * 512;
    }
    const int ob = ((int)blockIdx.x * nks + s0) * 1024;
    const int osb = ((int)blockIdx.x * nkq + s0 / 8) * 512;
    auto ld = [&](__amdgpu_buffer_rsrc_t r, int off) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, vo, off, 0);
        return make_uint4(v.x, v.y, v.z, v.w);
    };

    auto ld2 = [&](__amdgpu_buffer_rsrc_t r, int off) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8, off, 0);
        return make_uint2(v.x, v.y);
    };
    // this wave's scales: NQ 8-byte loads per operand, kept in registers
    uint2 sca[4][NQ], scb[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) sca[mi][q] = ld2(rsa, osa[mi] + q * 512);
        scb[q] = ld2(rsb, osb + q * 512);
    }
    // the code ring: step st lives in slot st % R, loaded R steps ahead
    uint4 ga[R][4], gb[R];
    auto issue = [&](int slot, int st) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) ga[slot][mi] = ld(ra, oa[mi] + st * 1024);
        gb[slot] = ld(rb, ob + st * 1024);
    };
#pragma unroll
    for (int i = 0; i < R; ++i) issue(i, i);
    auto sel = [](uint2 v, int j) { return j == 0 ? v.x : v.y; };

    f32x16_t acc[4] = {};
#pragma unroll
    for (int st = 0; st < SW; ++st) {
        const int slot = st % R, q = st / 8, j = (st / 4) % 2, sh = 8 * (st % 4);
        const int sb = (int)(sel(scb[q], j) >> sh);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                as_operand(ga[slot][mi]), as_operand(gb[slot]), acc[mi], 4, 4, 0,
                (int)(sel(sca[mi][q], j) >> sh), 0, sb);
        if (st + R < SW) issue(slot, st + R);
        // keep each step's loads right after its MFMAs (sunk together they
        // would empty the ring)
        __builtin_amdgcn_sched_barrier(0);
    }

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

// ---------------------------------------------------------------------------
// LDS-staged kernel (K a multiple of 512; code and scale rows 16-byte
// aligned).  The operand layout of the scaled MFMA wants, per load
// instruction, 32 rows x 32 bytes at the row stride, which keeps the address
// unit busy most of the time.  Here every load instruction instead reads
// eight full 128-byte row segments, straight into LDS (global->LDS loads, no
// registers), and the MFMA operands are read back from LDS.
//
// Tile: a workgroup (4 waves) owns 128 x 32 of C; wave w owns rows
// 32w..32w+31 and walks all of K in order (deterministic).  K is cut into
// stages of 4 MFMA steps (256 K values, 128 bytes of codes per row): per
// stage the workgroup stages A 128 x 128 B and B 32 x 128 B, GEMM_S stages in
// flight.  Each wave loads its own 32 rows of A and 8 of the 32 rows of B;
// a barrier per stage makes the shared B rows visible.  Within a row the
// 16-byte chunk c of row r of a stage sits at chunk c ^ ((r >> 1) & 7) of its
// LDS row: a ds_read_b128 serves 16 lanes per pass, rows r and r + 1 fall in
// different halves of the 64 banks, so the 16 rows of a pass of the
// MFMA-layout reads (one chunk each) hit 16 distinct 4-bank groups.
// The scale bytes of a K segment of up to GEMM_MAX_K are preloaded into LDS
// in whole 16-byte row chunks (a per-stage scale load would cost the L2 a
// request per row for 8 bytes, and the kernel is bound by its per-CU fetch
// requests); a longer K runs its segments one after another into the same
// accumulators.
// ---------------------------------------------------------------------------
constexpr int GEMM_S = 5;                   // stages in flight
constexpr int GEMM_STAGE_K = 256;           // K values per stage (4 MFMA steps)
constexpr int GEMM_A_CHUNKS = GEMM_TM * 8;  // 16-byte chunks of A codes per stage
constexpr int GEMM_B_CHUNKS = GEMM_TN * 8;
constexpr int GEMM_STAGE_CHUNKS = GEMM_A_CHUNKS + GEMM_B_CHUNKS;
constexpr int GEMM_LOADS = 5;               // code loads per wave per stage
constexpr int GEMM_MAX_K = 8192;            // K of one segment (its scales held in LDS)
constexpr int GEMM_SCALE_COLS = GEMM_MAX_K / 32 / 16;  // 16-byte scale chunks per row

typedef __attribute__((address_space(1))) const void *gemm_gptr;
typedef __attribute__((address_space(3))) void *gemm_lptr;

__device__ __forceinline__ int gemm_swizzle(int row) { return (row >> 1) & 7; }

// One K segment (at most GEMM_MAX_K, a multiple of 512, starting at block
// kb0 of the rows) of one workgroup's 128 x 32 tile of C (blockIdx.y,
// blockIdx.x), added to the accumulators.
__device__ __forceinline__ void gemm_lds_segment(const uint4 *__restrict__ A,
                                                 const uint8_t *__restrict__ As,
                                                 const uint4 *__restrict__ Bt,
                                                 const uint8_t *__restrict__ Bs, int M, int N,
                                                 int nblk, int kb0, int Kseg, f32x16_t &acc0,
                                                 f32x16_t &acc1) {
    // ring of code stages: A [128 rows][8 chunks], B [32][8];
    // the segment's scales, transposed: A [16-byte chunk][128 rows], B [chunk][32 rows]
    __shared__ uint4 ring[GEMM_S][GEMM_STAGE_CHUNKS];
    __shared__ uint4 a_scales[GEMM_SCALE_COLS][GEMM_TM];
    __shared__ uint4 b_scales[GEMM_SCALE_COLS][GEMM_TN];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r32 = lane & 31;
    const int kh = lane >> 5;
    const int nst = Kseg / GEMM_STAGE_K;
    const int ncols = Kseg / 32 / 16;  // 16-byte scale chunks per row (2 stages each)
    const int m0 = blockIdx.y * GEMM_TM, n0 = blockIdx.x * GEMM_TN;

    // ---- the scales, once: lane l of a load moves 16 bytes (2 stages) of one
    // row; A: chunk column c, rows 64h + l; B: columns 2j + l / 32, rows l % 32
    for (int i = w; i < 2 * ncols; i += 4) {
        const int c = i >> 1, row = 64 * (i & 1) + lane;
        const uint8_t *src = As + (int64_t)min(m0 + row, M - 1) * nblk + kb0 + 16 * c;
        __builtin_amdgcn_global_load_lds((gemm_gptr)src, (gemm_lptr)&a_scales[c][64 * (i & 1)], 16, 0, 0);
    }
    for (int j = w; 2 * j < ncols; j += 4) {
        const int c = 2 * j + kh;
        const uint8_t *src = Bs + (int64_t)min(n0 + r32, N - 1) * nblk + kb0 + 16 * min(c, ncols - 1);
        __builtin_amdgcn_global_load_lds((gemm_gptr)src, (gemm_lptr)&b_scales[2 * j][0], 16, 0, 0);
    }

    // code loads: lane l of a load covers row (8i + l / 8) of its group and
    // LDS chunk l % 8, which holds the row's chunk (l % 8) ^ swizzle
    const int lrow = lane >> 3, lpc = lane & 7;
    const uint4 *ga[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 32 * w + 8 * i + lrow;  // row within the A tile
        const int am = min(m0 + row, M - 1);
        ga[i] = A + (int64_t)am * nblk + kb0 + (lpc ^ gemm_swizzle(row));
    }
    const int brow = 8 * w + lrow;
    const uint4 *gb = Bt + (int64_t)min(n0 + brow, N - 1) * nblk + kb0 + (lpc ^ gemm_swizzle(brow));

    // Five code loads per wave per stage: its 32 rows of A and 8 of the 32
    // rows of B, global -> LDS.  Stages past the end re-read the last one
    // (cache hits) into a slot that is never read, so every iteration issues
    // the same loads and the wait below is one constant.
    auto issue = [&](int st, uint32_t slot) {
        st = min(st, nst - 1);
        uint4 *sb = &ring[0][0] + slot * GEMM_STAGE_CHUNKS;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((gemm_gptr)(ga[i] + st * 8),
                                             (gemm_lptr)&sb[(32 * w + 8 * i) * 8], 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gemm_gptr)(gb + st * 8),
                                         (gemm_lptr)&sb[GEMM_A_CHUNKS + 8 * w * 8], 16, 0, 0);
    };

    const int arow = 32 * w + r32;  // this lane's A operand row in the tile
    const int sw = gemm_swizzle(r32);  // its swizzle (= that of arow and of the B row r32)
    // LDS byte addresses of this lane's operands in slot 0: chunk
    // (2 s4 + kh) ^ swizzle of its A row and of its B row for steps s4 = 0..3
    uint32_t la[4], lb[4];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(gemm_lptr)&ring[0][0];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const uint32_t c = (uint32_t)((2 * s4 + kh) ^ sw);
        la[s4] = lds0 + (uint32_t)(arow * 8 + c) * 16u;
        lb[s4] = lds0 + (uint32_t)(GEMM_A_CHUNKS + r32 * 8 + c) * 16u;
    }
    // this lane's scale rows: stage st's 8 bytes are half (st & 1) of chunk st / 2
    const uint32_t lsa = (uint32_t)(uintptr_t)(gemm_lptr)&a_scales[0][arow];
    const uint32_t lsb = (uint32_t)(uintptr_t)(gemm_lptr)&b_scales[0][r32];
    constexpr uint32_t kSlotBytes = GEMM_STAGE_CHUNKS * 16u;

#pragma unroll
    for (int st = 0; st < GEMM_S - 1; ++st) issue(st, (uint32_t)st);
    uint32_t slot = 0, fill = GEMM_S - 1;  // slot of stage st, and of stage st + S - 1
    for (int st = 0; st < nst; ++st) {
        // stage st landed once only the later S - 2 stages' loads are in
        // flight (the scale loads, issued first, have landed by then too)
        constexpr int kLater = GEMM_LOADS * (GEMM_S - 2);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kLater & 15) | ((kLater >> 4) << 14));
        __builtin_amdgcn_s_barrier();  // every wave's part visible; slot `fill` is free
        issue(st + GEMM_S - 1, fill);
        // One asm block reads the stage's operands and waits for them: the
        // compiler cannot tell which LDS the global->LDS loads of later
        // stages write, and would otherwise wait for all of them here.
        const uint32_t off = slot * kSlotBytes;
        const uint32_t soff = (uint32_t)(st >> 1) * 16u * GEMM_TM + (uint32_t)(st & 1) * 8u;
        const uint32_t soffb = (uint32_t)(st >> 1) * 16u * GEMM_TN + (uint32_t)(st & 1) * 8u;
        u32x4_t a0, a1, a2, a3, b0, b1, b2, b3;
        uint2 sa, sb;
        asm volatile(
            "ds_read_b128 %0, %10\n\t"
            "ds_read_b128 %4, %14\n\t"
            "ds_read_b128 %1, %11\n\t"
            "ds_read_b128 %5, %15\n\t"
            "ds_read_b128 %2, %12\n\t"
            "ds_read_b128 %6, %16\n\t"
            "ds_read_b128 %3, %13\n\t"
            "ds_read_b128 %7, %17\n\t"
            "ds_read_b64 %8, %18\n\t"
            "ds_read_b64 %9, %19\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1), "=&v"(b2),
              "=&v"(b3), "=&v"(sa), "=&v"(sb)
            : "v"(la[0] + off), "v"(la[1] + off), "v"(la[2] + off), "v"(la[3] + off),
              "v"(lb[0] + off), "v"(lb[1] + off), "v"(lb[2] + off), "v"(lb[3] + off),
              "v"(lsa + soff), "v"(lsb + soffb)
            : "memory");
        slot = slot + 1 == GEMM_S ? 0 : slot + 1;
        fill = fill + 1 == GEMM_S ? 0 : fill + 1;
        const u32x4_t av[4] = {a0, a1, a2, a3}, bv[4] = {b0, b1, b2, b3};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int i = 2 * s4 + kh;  // scale byte of this step and half
            const uint32_t ea = (i < 4 ? sa.x : sa.y) >> (8 * (i & 3));
            const uint32_t eb = (i < 4 ? sb.x : sb.y) >> (8 * (i & 3));
            const i32x8_t ao = {(int)av[s4].x, (int)av[s4].y, (int)av[s4].z, (int)av[s4].w, 0, 0, 0, 0};
            const i32x8_t bo = {(int)bv[s4].x, (int)bv[s4].y, (int)bv[s4].z, (int)bv[s4].w, 0, 0, 0, 0};
            if (s4 & 1)
                acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ao, bo, acc1, 4, 4, 0, (int)ea,
                                                                      0, (int)eb);
            else
                acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ao, bo, acc0, 4, 4, 0, (int)ea,
                                                                      0, (int)eb);
        }
    }
    // the trailing re-reads land, and every wave is done with the segment's
    // LDS, before the next segment or the end of the workgroup
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_s_barrier();
}

// One workgroup's 128 x 32 tile of C (blockIdx.y, blockIdx.x), all of K: the
// K segments in order, each with its scales preloaded.
template <bool OUT_BF16>
__device__ __forceinline__ void gemm_lds_tile(const uint4 *__restrict__ A,
                                              const uint8_t *__restrict__ As,
                                              const uint4 *__restrict__ Bt,
                                              const uint8_t *__restrict__ Bs, int M, int N,
                                              int K, void *__restrict__ C) {
    // two accumulators (alternate MFMA steps) so that consecutive MFMAs do
    // not wait for each other; summed once at the end, in a fixed order
    f32x16_t acc0 = {}, acc1 = {};
    const int nblk = K / 32;
    for (int k0 = 0; k0 < K; k0 += GEMM_MAX_K)
        gemm_lds_segment(A, As, Bt, Bs, M, N, nblk, k0 / 32, min(K - k0, GEMM_MAX_K), acc0, acc1);
    const f32x16_t acc = acc0 + acc1;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r32 = lane & 31;
    const int kh = lane >> 5;
    const int m0 = blockIdx.y * GEMM_TM, n0 = blockIdx.x * GEMM_TN;

    // accumulator layout of the 32x32 MFMA: lane l holds column l % 32 and
    // rows 8 (j / 4) + 4 (l / 32) + (j % 4), j = 0..15
    const int col = n0 + r32;
    if (col >= N) return;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int row = m0 + 32 * w + 8 * (j / 4) + 4 * kh + (j % 4);
        if (row < M) {
            if (OUT_BF16)
                ((uint16_t *)C)[(int64_t)row * N + col] = (uint16_t)bf16_rne_bits(acc[j]);
            else
                ((float *)C)[(int64_t)row * N + col] = acc[j];
        }
    }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(GEMM_WG) void mxfp4_gemm_lds_kernel(
    const uint4 *__restrict__ A, const uint8_t *__restrict__ As, const uint4 *__restrict__ Bt,
    const uint8_t *__restrict__ Bs, int M, int N, int K, void *__restrict__ C) {
    gemm_lds_tile<OUT_BF16>(A, As, Bt, Bs, M, N, K, C);
}

// ---------------------------------------------------------------------------
// Split-K MXFP4 GEMM, for short A (the 128 x 32 tiling above makes every CU
// read all of A, 512 KB at K = 8192, against 128 KB of its own B).
//
// A workgroup owns a 128 x 128 tile of C and one of S equal K ranges (at most
// 2048 K, a multiple of 512): 128 KB of A and 128 KB of B at K = 8192, S = 4.
// Eight waves, two per SIMD so that one's LDS reads overlap the other's
// MFMAs: wave w computes rows 32 (w % 4) .. + 32 against columns 64 (w / 4)
// .. + 64, two 32 x 32 MFMA tiles sharing each A operand read.  K is staged
// through LDS (256 K per stage, four stages in flight, 32 KB per stage, the
// swizzle above), and the E8M0 scales of the workgroup's K range are
// preloaded transposed ([16-byte chunk][row], 16 KB).  The fp32 partial sums go
// to the workspace, P[s][m][n]; a second kernel adds the S partials of each
// output in increasing s, ((P0 + P1) + P2) + ..., and rounds once to the
// output type, so the result does not depend on scheduling.  The kernel
// boundary between the two makes the partials written on one XCD visible to
// the others without in-kernel cache maintenance.
// ---------------------------------------------------------------------------
constexpr int SK_WG = 512;
constexpr int SK_TN = 128;                                 // columns of C per workgroup
constexpr int SK_RING = 4;                                 // stages in flight
constexpr int SK_KS_MAX = 2048;                            // K values of one split, at most
constexpr int SK_SCALE_COLS = SK_KS_MAX / 32 / 16;         // 16-byte scale chunks per row
constexpr int SK_A_CHUNKS = GEMM_TM * 8;                   // 16-byte chunks of A per stage
constexpr int SK_B_CHUNKS = SK_TN * 8;
constexpr int SK_STAGE_CHUNKS = SK_A_CHUNKS + SK_B_CHUNKS;
constexpr int SK_LOADS = 4;                                // code loads per wave per stage

__global__ __launch_bounds__(SK_WG) void mxfp4_gemm_splitk_kernel(
    const uint4 *__restrict__ A, const uint8_t *__restrict__ As, const uint4 *__restrict__ Bt,
    const uint8_t *__restrict__ Bs, int M, int N, int K, int ks, float *__restrict__ P) {
    __shared__ uint4 ring[SK_RING][SK_STAGE_CHUNKS];
    __shared__ uint4 a_scales[SK_SCALE_COLS][GEMM_TM];
    __shared__ uint4 b_scales[SK_SCALE_COLS][SK_TN];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int wr = w & 3, wc = w >> 2;     // row tile, column half
    const int r32 = lane & 31;
    const int kh = lane >> 5;
    const int nblk = K / 32;               // blocks (16-byte chunks) per row
    const int split = blockIdx.y;
    const int kb0 = split * (ks / 32);     // the split's first block
    const int nst = ks / GEMM_STAGE_K;
    const int ncols = ks / 512;            // 16-byte scale chunks per row in the split
    const int m0 = blockIdx.z * GEMM_TM, n0 = blockIdx.x * SK_TN;

    // ---- the split's scales, once: lane l of a load moves 16 bytes (two
    // stages) of row 64h + l of chunk column c
    for (int i = w; i < 2 * ncols; i += SK_WG / 64) {
        const int c = i >> 1, h = i & 1, row = 64 * h + lane;
        const uint8_t *sa = As + (int64_t)min(m0 + row, M - 1) * nblk + kb0 + 16 * c;
        const uint8_t *sb = Bs + (int64_t)min(n0 + row, N - 1) * nblk + kb0 + 16 * c;
        __builtin_amdgcn_global_load_lds((gemm_gptr)sa, (gemm_lptr)&a_scales[c][64 * h], 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gemm_gptr)sb, (gemm_lptr)&b_scales[c][64 * h], 16, 0, 0);
    }

    // code loads: lane l of a load covers row (8i + l / 8) of the wave's 16
    // rows and LDS chunk l % 8, which holds the row's chunk (l % 8) ^ swizzle
    const int lrow = lane >> 3, lpc = lane & 7;
    const uint4 *ga[2], *gb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 16 * w + 8 * i + lrow;
        const int c = lpc ^ gemm_swizzle(row);
        ga[i] = A + (int64_t)min(m0 + row, M - 1) * nblk + kb0 + c;
        gb[i] = Bt + (int64_t)min(n0 + row, N - 1) * nblk + kb0 + c;
    }
    // Four code loads per wave per stage: its 16 rows of A and of B.  Stages
    // past the end re-read the last one into a slot that is never read, so
    // every iteration issues the same loads and the wait is one constant.
    auto issue = [&](int st, uint32_t slot) {
        st = min(st, nst - 1);
        uint4 *sb = &ring[0][0] + slot * SK_STAGE_CHUNKS;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds((gemm_gptr)(ga[i] + st * 8),
                                             (gemm_lptr)&sb[(16 * w + 8 * i) * 8], 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds((gemm_gptr)(gb[i] + st * 8),
                                             (gemm_lptr)&sb[SK_A_CHUNKS + (16 * w + 8 * i) * 8],
                                             16, 0, 0);
    };

    f32x16_t acc0 = {}, acc1 = {};  // column tiles 2 wc and 2 wc + 1
    const int arow = 32 * wr + r32;
    const int brow = 64 * wc + r32;  // tile 1: brow + 32 (same swizzle)
    const int sw = gemm_swizzle(r32);  // = that of arow, brow and brow + 32
    uint32_t la[4], lb[4];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(gemm_lptr)&ring[0][0];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const uint32_t c = (uint32_t)((2 * s4 + kh) ^ sw);
        la[s4] = lds0 + (uint32_t)(arow * 8 + c) * 16u;
        lb[s4] = lds0 + (uint32_t)(SK_A_CHUNKS + brow * 8 + c) * 16u;
    }
    const uint32_t lsa = (uint32_t)(uintptr_t)(gemm_lptr)&a_scales[0][arow];
    const uint32_t lsb = (uint32_t)(uintptr_t)(gemm_lptr)&b_scales[0][brow];
    constexpr uint32_t kSlotBytes = SK_STAGE_CHUNKS * 16u;
    constexpr uint32_t kTileB = 32u * 8u * 16u;   // 32 rows of a stage
    constexpr uint32_t kTileS = 32u * 16u;        // 32 rows of a scale column

#pragma unroll
    for (int st = 0; st < SK_RING - 1; ++st) issue(st, (uint32_t)st);
    uint32_t slot = 0, fill = SK_RING - 1;
    for (int st = 0; st < nst; ++st) {
        constexpr int kLater = SK_LOADS * (SK_RING - 2);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kLater & 15) | ((kLater >> 4) << 14));
        __builtin_amdgcn_s_barrier();  // every wave's part visible; slot `fill` is free
        issue(st + SK_RING - 1, fill);
        const uint32_t off = slot * kSlotBytes;
        const uint32_t soff = (uint32_t)(st >> 1) * 16u * GEMM_TM + (uint32_t)(st & 1) * 8u;
        const uint32_t soffb = (uint32_t)(st >> 1) * 16u * SK_TN + (uint32_t)(st & 1) * 8u;
        uint2 sa, sb0, sb1;
        asm volatile(
            "ds_read_b64 %0, %3\n\t"
            "ds_read_b64 %1, %4\n\t"
            "ds_read_b64 %2, %5\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(sa), "=&v"(sb0), "=&v"(sb1)
            : "v"(lsa + soff), "v"(lsb + soffb), "v"(lsb + soffb + kTileS)
            : "memory");
        slot = slot + 1 == SK_RING ? 0 : slot + 1;
        fill = fill + 1 == SK_RING ? 0 : fill + 1;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            u32x4_t a, b0, b1;
            asm volatile(
                "ds_read_b128 %0, %3\n\t"
                "ds_read_b128 %1, %4\n\t"
                "ds_read_b128 %2, %5\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(a), "=&v"(b0), "=&v"(b1)
                : "v"(la[s4] + off), "v"(lb[s4] + off), "v"(lb[s4] + off + kTileB)
                : "memory");
            const int i = 2 * s4 + kh;  // scale byte of this step and half
            const int sh = 8 * (i & 3);
            const int ea = (int)((i < 4 ? sa.x : sa.y) >> sh);
            const i32x8_t ao = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
            const i32x8_t bo0 = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
            const i32x8_t bo1 = {(int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w, 0, 0, 0, 0};
            acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                ao, bo0, acc0, 4, 4, 0, ea, 0, (int)((i < 4 ? sb0.x : sb0.y) >> sh));
            acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                ao, bo1, acc1, 4, 4, 0, ea, 0, (int)((i < 4 ? sb1.x : sb1.y) >> sh));
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the trailing re-reads land before the workgroup ends

    // accumulator layout of the 32x32 MFMA: lane l holds column l % 32 and
    // rows 8 (j / 4) + 4 (l / 32) + (j % 4), j = 0..15
    float *Ps = P + (int64_t)split * M * N;
    const f32x16_t acc[2] = {acc0, acc1};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int col = n0 + 64 * wc + 32 * t + r32;
        if (col < N) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int row = m0 + 32 * wr + 8 * (j / 4) + 4 * kh + (j % 4);
                if (row < M) Ps[(int64_t)row * N + col] = acc[t][j];
            }
        }
    }
}

// C = the S partials of each output added in increasing s, rounded once.
// Four outputs per thread (M N is a multiple of 4).
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const uint4 *__restrict__ P,
                                                            int64_t n4, int S,
                                                            void *__restrict__ C) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const uint4 p = ld_stream(P + i);
        float4 acc = make_float4(u2f(p.x), u2f(p.y), u2f(p.z), u2f(p.w));
        for (int k = 1; k < S; ++k) {
            const uint4 q = ld_stream(P + (int64_t)k * n4 + i);
            acc.x += u2f(q.x);
            acc.y += u2f(q.y);
            acc.z += u2f(q.z);
            acc.w += u2f(q.w);
        }
        if (OUT_BF16) {
            uint2 o;
            o.x = bf16_rne_bits(acc.x) | (bf16_rne_bits(acc.y) << 16);
            o.y = bf16_rne_bits(acc.z) | (bf16_rne_bits(acc.w) << 16);
            ((uint2 *)C)[i] = o;
        } else {
            ((float4 *)C)[i] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// NVFP4 x NVFP4 GEMM ("NVFP4 / MXFP4 format" page, section 6:
// Y = a_X a_W sum_g b^X_g b^W_g sum_{k in g} p^X_k p^W_k over 16-element
// groups).  The scaled MFMA applies one power of two per 32 K values; an
// E4M3 block scale is not a power of two and p * b needs up to 6 significant
// bits, which no FP8/FP6/FP4 operand holds but fp16 does.  So each operand
// value is decoded to fp16 (the FP4 converter), multiplied by its block's
// E4M3 value (one packed fp16 multiply per pair, exact), and fed to the fp16
// MFMA 32x32x16 with fp32 accumulation; the two tensor scales multiply the
// fp32 result once: C = RN32(acc * RN32(a_X a_W)).
//
// Tiling as the MXFP4 kernel: a 128 x 32 tile per workgroup, K staged
// through an XOR-swizzled ring in LDS (three stages of 256 K), the E4M3
// scales of all K preloaded (16 K per byte: 80 KB for K = 8192).  Lane half h
// takes the stage's K values [128h, 128h + 128): its 64 code bytes are
// contiguous, and MFMA step j uses bytes 4j..4j+3 (K 128h + 8j .. + 8), which
// lie in one 16-block (8h + j/2).  A and B lanes use the same permutation of
// K, so the sum is unchanged.
// ---------------------------------------------------------------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

constexpr int NVG_S = 3;                                // stages in flight
constexpr int NVG_SCALE_COLS = GEMM_MAX_K / 16 / 16;    // 16-byte chunks of E4M3 scales per row

// Eight fp16 operand values: the 8 codes of dword w times the block scale
// held in half `hi` of s2 (selected per MFMA step, a constant).
__device__ __forceinline__ half8_t nv_operand(uint32_t w, half2_t s2, bool hi) {
    const _Float16 s = hi ? s2.y : s2.x;
    const half2_t b = {s, s};
    const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * b;
    const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * b;
    const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * b;
    const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * b;
    const half8_t r = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    return r;
}

// ---------------------------------------------------------------------------
// NVFP4 operands in fp16-MFMA operand order ("packed" NVFP4 layout).  Codes as
// in the MXFP4 packed layout: per 32-row tile and 64-value K step, 1 KB in
// which lane l holds the 32 codes of row l % 32 in the step's K half l / 32.
// Scales after all codes: per tile and group q of eight K steps, 1 KB in which
// byte 2 i + b of lane l is the E4M3 scale of its row and 16-block
// 4 (8 q + i) + 2 (l / 32) + b (padding rows: 0).  The fp16 MFMA's 16 K slots
// may take any K values as long as A and B agree: in sub-step u of a step,
// lane half h feeds K values 32 h + 8 u .. + 8, which lie in one 16-block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_nv_scales_kernel(const uint8_t *__restrict__ scales,
                                                             int64_t rows, int64_t nks,
                                                             int64_t total,
                                                             uint4 *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t nkq = nks / 8;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
        const int l = (int)(t & 63);
        const int64_t g = t >> 6, q = g % nkq, rt = g / nkq;
        const int64_t r = rt * 32 + (l & 31);
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (r < rows) {
            const uint8_t *s = scales + r * (nks * 4) + 32 * q + 2 * (l >> 5);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                w[i / 2] |= ((uint32_t)s[4 * i] | ((uint32_t)s[4 * i + 1] << 8)) << (16 * (i & 1));
        }
        out[t] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

constexpr int NVPK_RING = 8;  // K steps in flight per wave

// The NVFP4 GEMM on packed operands: a workgroup owns a 128 x 32 tile of C,
// its four waves take the four quarters of the K steps (SW each, unrolled,
// step st's loads in ring slot st % NVPK_RING, issued NVPK_RING steps ahead); each wave
// decodes its own operands once (FP4 -> fp16 times the E4M3 scale, exact),
// 16 fp16 MFMAs per step; the partial tiles are added through LDS in a fixed
// order and C = RN32(sum * RN32(s_gA s_gB)).
template <bool OUT_BF16, int SW>
__global__ __launch_bounds__(GEMM_WG) void nvfp4_gemm_packed_kernel(
    const uint4 *__restrict__ Ap, const uint4 *__restrict__ Asp, const float *__restrict__ sgA,
    const uint4 *__restrict__ Bp, const uint4 *__restrict__ Bsp, const float *__restrict__ sgB,
    int M, int N, void *__restrict__ C) {
    constexpr int R = NVPK_RING;
    constexpr int NQ = SW / 8;
    constexpr int nks = 4 * SW, nkq = nks / 8;
    __shared__ float part[4][4][16][64];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31;
    const int kh = lane >> 5;
    const int s0 = w * SW;
    const int nrt_a = (M + 31) / 32, nrt_b = (N + 31) / 32;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)Ap, (short)0, nrt_a * nks * 1024, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)Bp, (short)0, nrt_b * nks * 1024, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void *)Asp, (short)0, nrt_a * nkq * 1024, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void *)Bsp, (short)0, nrt_b * nkq * 1024, kBufferRsrcWord3);
    const int vo = lane * 16;
    int oa[4], osa[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int rt = min((int)blockIdx.y * 4 + mi, nrt_a - 1);
        oa[mi] = (rt * nks + s0) * 1024;
        osa[mi] = (rt * nkq + s0 / 8) * 1024;
    }
    const int ob = ((int)blockIdx.x * nks + s0) * 1024;
    const int osb = ((int)blockIdx.x * nkq + s0 / 8) * 1024;
    auto ld = [&](__amdgpu_buffer_rsrc_t r, int off) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, vo, off, 0);
        return make_uint4(v.x, v.y, v.z, v.w);
    };
    // scales, one 16-byte load per operand per eight steps, double-buffered:
    // group q + 1 is requested when group q starts
    uint4 sca[2][4], scb[2];
    auto issue_scales = [&](int q) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) sca[q & 1][mi] = ld(rsa, osa[mi] + q * 1024);
        scb[q & 1] = ld(rsb, osb + q * 1024);
    };
    uint4 ga[R][4], gb[R];
    auto issue = [&](int slot, int st) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) ga[slot][mi] = ld(ra, oa[mi] + st * 1024);
        gb[slot] = ld(rb, ob + st * 1024);
    };
    issue_scales(0);
#pragma unroll
    for (int i = 0; i < R; ++i) issue(i, i);
    auto word = [](uint4 v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; };
    // E4M3 bytes 2 (i % 2), 2 (i % 2) + 1 of a word as an fp16 pair
    auto scale2 = [](uint32_t v, bool hi) {
        return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, true)
                  : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
    };

    f32x16_t acc[4] = {};
#pragma unroll
    for (int st = 0; st < SW; ++st) {
        const int slot = st % R, q = st / 8, i = st % 8;
        if (i == 0 && q + 1 < NQ) issue_scales(q + 1);
        const half2_t bs2 = scale2(word(scb[q & 1], i / 2), (i & 1) != 0);
        half2_t as2[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) as2[mi] = scale2(word(sca[q & 1][mi], i / 2), (i & 1) != 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const half8_t bo = nv_operand(word(gb[slot], u), bs2, u >= 2);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    nv_operand(word(ga[slot][mi], u), as2[mi], u >= 2), bo, acc[mi], 0, 0, 0);
        }
        if (st + R < SW) issue(slot, st + R);
        __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int j = 0; j < 16; ++j) part[w][mi][j][lane] = acc[mi][j];
    __syncthreads();
    const int mi = w;
    const float g = sgA[0] * sgB[0];
    const int col = blockIdx.x * GEMM_TN + r32;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float v = part[0][mi][j][lane];
        v = v + part[1][mi][j][lane];
        v = v + part[2][mi][j][lane];
        v = v + part[3][mi][j][lane];
        v = v * g;
        const int row = blockIdx.y * GEMM_TM + 32 * mi + 8 * (j / 4) + 4 * kh + (j % 4);
        if (row < M && col < N) {
            if (OUT_BF16)
                ((uint16_t *)C)[(int64_t)row * N + col] = (uint16_t)bf16_rne_bits(v);
            else
                ((float *)C)[(int64_t)row * N + col] = v;
        }
    }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(GEMM_WG) void nvfp4_gemm_lds_kernel(
    const uint4 *__restrict__ A, const uint8_t *__restrict__ As, const float *__restrict__ sgA,
    const uint4 *__restrict__ Bt, const uint8_t *__restrict__ Bs, const float *__restrict__ sgB,
    int M, int N, int K, void *__restrict__ C) {
    __shared__ uint4 ring[NVG_S][GEMM_STAGE_CHUNKS];
    __shared__ uint4 a_scales[NVG_SCALE_COLS][GEMM_TM];
    __shared__ uint4 b_scales[NVG_SCALE_COLS][GEMM_TN];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int r32 = lane & 31;
    const int kh = lane >> 5;
    const int nblk = K / 32;       // 16-byte code chunks per row
    const int nst = K / GEMM_STAGE_K;
    const int ncols = K / 256;     // 16-byte scale chunks per row (one per stage)
    const int srow = K / 16;       // scale bytes per row
    const int m0 = blockIdx.y * GEMM_TM, n0 = blockIdx.x * GEMM_TN;

    // ---- the scales, once, transposed: A [chunk][128 rows], B [chunk][32 rows]
    for (int i = w; i < 2 * ncols; i += 4) {
        const int c = i >> 1, row = 64 * (i & 1) + lane;
        const uint8_t *src = As + (int64_t)min(m0 + row, M - 1) * srow + 16 * c;
        __builtin_amdgcn_global_load_lds((gemm_gptr)src, (gemm_lptr)&a_scales[c][64 * (i & 1)], 16, 0, 0);
    }
    for (int j = w; 2 * j < ncols; j += 4) {
        const int c = 2 * j + kh;
        const uint8_t *src = Bs + (int64_t)min(n0 + r32, N - 1) * srow + 16 * min(c, ncols - 1);
        __builtin_amdgcn_global_load_lds((gemm_gptr)src, (gemm_lptr)&b_scales[2 * j][0], 16, 0, 0);
    }

    // code loads, as the MXFP4 kernel: lane l of a load covers row
    // (8i + l / 8) of its group and LDS chunk l % 8, holding the row's chunk
    // (l % 8) ^ swizzle
    const int lrow = lane >> 3, lpc = lane & 7;
    const uint4 *ga[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 32 * w + 8 * i + lrow;
        ga[i] = A + (int64_t)min(m0 + row, M - 1) * nblk + (lpc ^ gemm_swizzle(row));
    }
    const int brow = 8 * w + lrow;
    const uint4 *gb = Bt + (int64_t)min(n0 + brow, N - 1) * nblk + (lpc ^ gemm_swizzle(brow));
    auto issue = [&](int st, uint32_t slot) {
        st = min(st, nst - 1);
        uint4 *sb = &ring[0][0] + slot * GEMM_STAGE_CHUNKS;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((gemm_gptr)(ga[i] + st * 8),
                                             (gemm_lptr)&sb[(32 * w + 8 * i) * 8], 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gemm_gptr)(gb + st * 8),
                                         (gemm_lptr)&sb[GEMM_A_CHUNKS + 8 * w * 8], 16, 0, 0);
    };

    f32x16_t acc0 = {}, acc1 = {};
    const int arow = 32 * w + r32;
    const int sw = gemm_swizzle(r32);  // = that of arow and of the B row r32
    // this lane's operand chunks in slot 0: (4 kh + i) ^ swizzle, i = 0..3
    uint32_t la[4], lb[4];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(gemm_lptr)&ring[0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t c = (uint32_t)((4 * kh + i) ^ sw);
        la[i] = lds0 + (uint32_t)(arow * 8 + c) * 16u;
        lb[i] = lds0 + (uint32_t)(GEMM_A_CHUNKS + r32 * 8 + c) * 16u;
    }
    // the lane's 8 scale bytes of stage st: blocks 8 kh .. 8 kh + 7
    const uint32_t lsa = (uint32_t)(uintptr_t)(gemm_lptr)&a_scales[0][arow] + 8u * kh;
    const uint32_t lsb = (uint32_t)(uintptr_t)(gemm_lptr)&b_scales[0][r32] + 8u * kh;
    constexpr uint32_t kSlotBytes = GEMM_STAGE_CHUNKS * 16u;

#pragma unroll
    for (int st = 0; st < NVG_S - 1; ++st) issue(st, (uint32_t)st);
    uint32_t slot = 0, fill = NVG_S - 1;
    for (int st = 0; st < nst; ++st) {
        constexpr int kLater = GEMM_LOADS * (NVG_S - 2);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kLater & 15) | ((kLater >> 4) << 14));
        __builtin_amdgcn_s_barrier();
        issue(st + NVG_S - 1, fill);
        const uint32_t off = slot * kSlotBytes;
        const uint32_t soa = (uint32_t)st * 16u * GEMM_TM, sob = (uint32_t)st * 16u * GEMM_TN;
        u32x4_t a0, a1, a2, a3, b0, b1, b2, b3;
        uint2 sa, sb;
        asm volatile(
            "ds_read_b128 %0, %10\n\t"
            "ds_read_b128 %4, %14\n\t"
            "ds_read_b128 %1, %11\n\t"
            "ds_read_b128 %5, %15\n\t"
            "ds_read_b128 %2, %12\n\t"
            "ds_read_b128 %6, %16\n\t"
            "ds_read_b128 %3, %13\n\t"
            "ds_read_b128 %7, %17\n\t"
            "ds_read_b64 %8, %18\n\t"
            "ds_read_b64 %9, %19\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(b0), "=&v"(b1), "=&v"(b2),
              "=&v"(b3), "=&v"(sa), "=&v"(sb)
            : "v"(la[0] + off), "v"(la[1] + off), "v"(la[2] + off), "v"(la[3] + off),
              "v"(lb[0] + off), "v"(lb[1] + off), "v"(lb[2] + off), "v"(lb[3] + off),
              "v"(lsa + soa), "v"(lsb + sob)
            : "memory");
        slot = slot + 1 == NVG_S ? 0 : slot + 1;
        fill = fill + 1 == NVG_S ? 0 : fill + 1;
        // block scales as fp16 pairs: blocks (0,1) (2,3) (4,5) (6,7)
        const half2_t as2[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa.x, 1.0f, false),
                                __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa.x, 1.0f, true),
                                __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa.y, 1.0f, false),
                                __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa.y, 1.0f, true)};
        const half2_t bs2[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb.x, 1.0f, false),
                                __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb.x, 1.0f, true),
                                __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb.y, 1.0f, false),
                                __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb.y, 1.0f, true)};
        const u32x4_t av[4] = {a0, a1, a2, a3}, bv[4] = {b0, b1, b2, b3};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t wa = av[j >> 2][j & 3], wb = bv[j >> 2][j & 3];
            const int blk = j >> 1;  // 16-block within the lane's eight
            const half8_t ao = nv_operand(wa, as2[blk >> 1], blk & 1);
            const half8_t bo = nv_operand(wb, bs2[blk >> 1], blk & 1);
            if (j & 1)
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ao, bo, acc1, 0, 0, 0);
            else
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ao, bo, acc0, 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    const f32x16_t acc = acc0 + acc1;
    const float g = sgA[0] * sgB[0];
    const int col = n0 + r32;
    if (col >= N) return;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int row = m0 + 32 * w + 8 * (j / 4) + 4 * kh + (j % 4);
        if (row < M) {
            const float v = acc[j] * g;
            if (OUT_BF16)
                ((uint16_t *)C)[(int64_t)row * N + col] = (uint16_t)bf16_rne_bits(v);
            else
                ((float *)C)[(int64_t)row * N + col] = v;
        }
    }
}

// Value of any E4M3FN byte: sign bit, magnitude code; 0x7F is NaN.
__device__ __forceinline__ float e4m3_any_value_g(uint32_t s) {
    const uint32_t mag = s & 0x7Fu;
    const float v = mag == 0x7Fu ? __builtin_nanf("") : e4m3_pos_value(mag);
    return (s & 0x80u) ? -v : v;
}

// Any K (a multiple of 16) and alignment: one output per thread, the
// equation's sums in fp32 block by block.  For shapes the staged kernel does
// not take; slow.
template <bool OUT_BF16>
__global__ __launch_bounds__(GEMM_WG) void nvfp4_gemm_simple_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ As, const float *__restrict__ sgA,
    const uint8_t *__restrict__ Bt, const uint8_t *__restrict__ Bs, const float *__restrict__ sgB,
    int M, int N, int K, void *__restrict__ C) {
    const int64_t idx = (int64_t)blockIdx.x * GEMM_WG + threadIdx.x;
    if (idx >= (int64_t)M * N) return;
    const int m = (int)(idx / N), n = (int)(idx % N);
    const uint8_t *pa = A + (int64_t)m * (K / 2), *pb = Bt + (int64_t)n * (K / 2);
    float acc = 0.0f;
    for (int t = 0; t < K / 16; ++t) {
        float dot = 0.0f;
        for (int i = 0; i < 8; ++i) {
            const uint32_t ca = pa[8 * t + i], cb = pb[8 * t + i];
            const f32x2_t va = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ca, 1.0f, 0);
            const f32x2_t vb = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cb, 1.0f, 0);
            dot = __builtin_fmaf(va.x, vb.x, dot);
            dot = __builtin_fmaf(va.y, vb.y, dot);
        }
        const float s = e4m3_any_value_g(As[(int64_t)m * (K / 16) + t]) *
                        e4m3_any_value_g(Bs[(int64_t)n * (K / 16) + t]);
        acc = __builtin_fmaf(s, dot, acc);
    }
    const float v = acc * (sgA[0] * sgB[0]);
    if (OUT_BF16)
        ((uint16_t *)C)[idx] = (uint16_t)bf16_rne_bits(v);
    else
        ((float *)C)[idx] = v;
}

// ---------------------------------------------------------------------------
// W4A4 linear: the activations [M, K] quantized to MXFP4 (OCP floor rule) in
// the GEMM's own launch ("FP4, FP8 and INT8/INT4" page, section 5: the
// quantize and MMA costs of a low-bit linear layer).  Every workgroup needs
// all of A, so each quantizes a 1/G share and writes it out (a_codes,
// a_scales are outputs too), the grid meets at a barrier, and the tiles then
// read A as the plain GEMM does.  The grid must be resident at once.
// ---------------------------------------------------------------------------
// MXFP4 quantize of the wave tiles wave, wave + nwaves, ... of A: a share of
// the grid's (the fused path) or all of A by one workgroup (its fallback).
template <bool XBF16>
__device__ __forceinline__ uint32_t quantize_share(const uint4 *__restrict__ x, int64_t nchunks,
                                                   uint32_t *__restrict__ a_codes,
                                                   uint8_t *__restrict__ a_scales, int64_t wave,
                                                   int64_t nwaves) {
    const int lane = threadIdx.x & (WAVE - 1);
    uint32_t flags = 0;
    // a wave takes 64 consecutive chunks of 8 values; four lanes hold a block
    for (int64_t t = wave; t * WAVE < nchunks; t += nwaves) {
        const int64_t c = t * WAVE + lane;
        const bool ok = c < nchunks;
        const uint4 z = make_uint4(0, 0, 0, 0);
        // fp32: two loads 32 bytes apart per lane, ordinary (cached) so the
        // second finds the line the first brought in
        const uint4 lo = ok ? (XBF16 ? ld_stream(x + c) : x[2 * c]) : z;
        const uint4 hi = (!XBF16 && ok) ? x[2 * c + 1] : z;
        uint32_t m = XBF16 ? amax_bf16x8(lo) : amax_f32x8(lo, hi);
        m = max(m, dpp<QP_XOR1>(m));
        m = max(m, dpp<QP_XOR2>(m));
        const int sh = XBF16 ? 7 : 23;
        if ((m >> sh) >= 0xFFu) flags |= FLAG_NONFINITE;
        const uint32_t sb = mx_scale_byte(m, sh);
        uint32_t q;
        if (XBF16) {
            q = cvt_fp4x8_bf16(lo, e8m0_operand(sb));
        } else {
            float v[8];
            widen_f32x8(lo, hi, v);
            q = cvt_fp4x8_f32(v, e8m0_operand(sb));
        }
        if (ok) {
            a_codes[c] = q;
            if ((lane & 3) == 0) a_scales[c >> 2] = (uint8_t)sb;
        }
    }
    return flags;
}

template <bool OUT_BF16, bool XBF16>
__global__ __launch_bounds__(GEMM_WG) void mxfp4_linear_kernel(
    const uint4 *__restrict__ x, uint32_t *__restrict__ a_codes, uint8_t *__restrict__ a_scales,
    const uint4 *__restrict__ Bt, const uint8_t *__restrict__ Bs, int M, int N, int K,
    void *__restrict__ C, uint64_t *slots, uint32_t *epoch, uint32_t spin_limit,
    int32_t *status) {
    const int wv = threadIdx.x / WAVE;
    constexpr int WPG = GEMM_WG / WAVE;
    const int64_t nchunks = (int64_t)M * K / 8;
    const uint32_t tag = wv == 0 ? barrier_tag(epoch) : 0u;
    uint32_t flags = quantize_share<XBF16>(x, nchunks, a_codes, a_scales,
                                           (int64_t)(blockIdx.y * gridDim.x + blockIdx.x) * WPG + wv,
                                           (int64_t)gridDim.x * gridDim.y * WPG);
    // Every wave's stores of its share have completed at the workgroup
    // barrier; then one wave makes them visible to the device (the release
    // writes back this XCD's L2) before it publishes its slot, and after the
    // grid barrier drops stale copies of the other shares (the acquire
    // invalidates the caches) before any wave reads A.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ uint32_t late_tag;
    if (wv == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        uint32_t A;
        const bool done = grid_barrier_max(slots, tag, 0u, spin_limit, A);
        if ((threadIdx.x & (WAVE - 1)) == 0) {
            late_tag = done ? 0u : tag;
            if (!done || (blockIdx.x == 0 && blockIdx.y == 0)) barrier_store_epoch(epoch, tag);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    const bool late = late_tag != 0u;
    if (late) {
        // Fallback: the wait timed out, so other shares of A may not be
        // written yet.  This workgroup quantizes all of A itself; where
        // another workgroup writes the same bytes it writes the same values.
        flags |= quantize_share<XBF16>(x, nchunks, a_codes, a_scales, wv, WPG);
        flags |= FLAG_BARRIER_TIMEOUT;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wv == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
    }
    report_flags(status, flags);
    gemm_lds_tile<OUT_BF16>((const uint4 *)a_codes, a_scales, Bt, Bs, M, N, K, C);
    if (late && threadIdx.x == 0) barrier_retract(slots);
}

// Workgroups one CU holds of the linear kernel's largest instance (its LDS
// allows one), and the CU count: the grid of a fused call may not exceed
// their product.  Probed once per device.
static int linear_capacity() {
    static int cap[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::call_once(once[dev], [dev] {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        auto k = mxfp4_linear_kernel<false, false>;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, GEMM_WG, 0) != hipSuccess)
            per_cu = 0;
        const int c = cus * per_cu;
        cap[dev] = c > kResidentSlots ? kResidentSlots : c;
    });
    return cap[dev];
}

static bool gemm_lds_ok(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *bt_codes,
                        const uint8_t *bt_scales, int64_t K) {
    auto al = [](const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; };
    return K % (2 * GEMM_STAGE_K) == 0 && al(a_codes, 16) && al(bt_codes, 16) &&
           al(a_scales, 16) && al(bt_scales, 16);
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
    if (gemm_lds_ok(a_codes, a_scales, bt_codes, bt_scales, K)) {
        if (out_bf16)
            hipLaunchKernelGGL(mxfp4_gemm_lds_kernel<true>, grid, dim3(GEMM_WG), 0, s,
                               (const uint4 *)a_codes, a_scales, (const uint4 *)bt_codes,
                               bt_scales, (int)M, (int)N, (int)K, c);
        else
            hipLaunchKernelGGL(mxfp4_gemm_lds_kernel<false>, grid, dim3(GEMM_WG), 0, s,
                               (const uint4 *)a_codes, a_scales, (const uint4 *)bt_codes,
                               bt_scales, (int)M, (int)N, (int)K, c);
        return hipGetLastError();
    }
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

int64_t packed_operand_bytes(int64_t rows, int64_t K) {
    if (rows < 1 || K < 512 || K % 512 != 0) return 0;
    const int64_t padded = (rows + 31) / 32 * 32;
    return padded * (K / 2) + padded * (K / 32);
}

hipError_t launch_pack_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                             uint8_t *packed, hipStream_t s) {
    const int64_t nrt = (rows + 31) / 32, nks = K / 64;
    const int64_t nc = nrt * nks * 64, ns = nrt * (nks / 8) * 128;
    auto grid = [](int64_t n) {
        int64_t g = (n + 255) / 256;
        return (unsigned)(g > kMaxGrid ? kMaxGrid : g);
    };
    hipLaunchKernelGGL(pack_codes_kernel, dim3(grid(nc)), dim3(256), 0, s, (const uint4 *)codes,
                       rows, nks, nc, (uint4 *)packed);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pack_scales_kernel, dim3(grid(ns)), dim3(256), 0, s, scales, rows, nks, ns,
                       (uint32_t *)(packed + nrt * 32 * (K / 2)));
    return hipGetLastError();
}

hipError_t launch_gemm_mxfp4_packed(const uint8_t *a_packed, const uint8_t *bt_packed, int64_t M,
                                    int64_t N, int64_t K, void *c, bool out_bf16, hipStream_t s) {
    const int64_t nrt_a = (M + 31) / 32, nrt_b = (N + 31) / 32;
    const uint4 *ap = (const uint4 *)a_packed, *bp = (const uint4 *)bt_packed;
    const uint4 *asp = (const uint4 *)(a_packed + nrt_a * 32 * (K / 2));
    const uint4 *bsp = (const uint4 *)(bt_packed + nrt_b * 32 * (K / 2));
    dim3 grid((unsigned)nrt_b, (unsigned)((M + GEMM_TM - 1) / GEMM_TM));
    using Kn = void (*)(const uint4 *, const uint4 *, const uint4 *, const uint4 *, int, int, void *);
    // K steps per wave = K / 256: one instance per multiple of 2048 up to 16384
    static const Kn kernels[2][8] = {
        {mxfp4_gemm_packed_kernel<false, 8>, mxfp4_gemm_packed_kernel<false, 16>,
         mxfp4_gemm_packed_kernel<false, 24>, mxfp4_gemm_packed_kernel<false, 32>,
         mxfp4_gemm_packed_kernel<false, 40>, mxfp4_gemm_packed_kernel<false, 48>,
         mxfp4_gemm_packed_kernel<false, 56>, mxfp4_gemm_packed_kernel<false, 64>},
        {mxfp4_gemm_packed_kernel<true, 8>, mxfp4_gemm_packed_kernel<true, 16>,
         mxfp4_gemm_packed_kernel<true, 24>, mxfp4_gemm_packed_kernel<true, 32>,
         mxfp4_gemm_packed_kernel<true, 40>, mxfp4_gemm_packed_kernel<true, 48>,
         mxfp4_gemm_packed_kernel<true, 56>, mxfp4_gemm_packed_kernel<true, 64>}};
    const int idx = (int)(K / 2048) - 1;
    if (idx < 0 || idx > 7 || K % 2048 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kernels[out_bf16 ? 1 : 0][idx], grid, dim3(GEMM_WG), 0, s, ap, asp, bp, bsp,
                       (int)M, (int)N, c);
    return hipGetLastError();
}

int64_t nv_packed_operand_bytes(int64_t rows, int64_t K) {
    if (rows < 1 || K < 512 || K % 512 != 0) return 0;
    const int64_t padded = (rows + 31) / 32 * 32;
    return padded * (K / 2) + padded * (K / 16);
}

hipError_t launch_pack_nvfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                             uint8_t *packed, hipStream_t s) {
    const int64_t nrt = (rows + 31) / 32, nks = K / 64;
    const int64_t nc = nrt * nks * 64, ns = nrt * (nks / 8) * 64;
    auto grid = [](int64_t n) {
        int64_t g = (n + 255) / 256;
        return (unsigned)(g > kMaxGrid ? kMaxGrid : g);
    };
    hipLaunchKernelGGL(pack_codes_kernel, dim3(grid(nc)), dim3(256), 0, s, (const uint4 *)codes,
                       rows, nks, nc, (uint4 *)packed);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pack_nv_scales_kernel, dim3(grid(ns)), dim3(256), 0, s, scales, rows, nks,
                       ns, (uint4 *)(packed + nrt * 32 * (K / 2)));
    return hipGetLastError();
}

hipError_t launch_gemm_nvfp4_packed(const uint8_t *a_packed, const float *sg_a,
                                    const uint8_t *bt_packed, const float *sg_b, int64_t M,
                                    int64_t N, int64_t K, void *c, bool out_bf16, hipStream_t s) {
    const int64_t nrt_a = (M + 31) / 32, nrt_b = (N + 31) / 32;
    const uint4 *ap = (const uint4 *)a_packed, *bp = (const uint4 *)bt_packed;
    const uint4 *asp = (const uint4 *)(a_packed + nrt_a * 32 * (K / 2));
    const uint4 *bsp = (const uint4 *)(bt_packed + nrt_b * 32 * (K / 2));
    dim3 grid((unsigned)nrt_b, (unsigned)((M + GEMM_TM - 1) / GEMM_TM));
    using Kn = void (*)(const uint4 *, const uint4 *, const float *, const uint4 *, const uint4 *,
                        const float *, int, int, void *);
    // K steps per wave = K / 256: one instance per multiple of 2048 up to 16384
    static const Kn kernels[2][8] = {
        {nvfp4_gemm_packed_kernel<false, 8>, nvfp4_gemm_packed_kernel<false, 16>,
         nvfp4_gemm_packed_kernel<false, 24>, nvfp4_gemm_packed_kernel<false, 32>,
         nvfp4_gemm_packed_kernel<false, 40>, nvfp4_gemm_packed_kernel<false, 48>,
         nvfp4_gemm_packed_kernel<false, 56>, nvfp4_gemm_packed_kernel<false, 64>},
        {nvfp4_gemm_packed_kernel<true, 8>, nvfp4_gemm_packed_kernel<true, 16>,
         nvfp4_gemm_packed_kernel<true, 24>, nvfp4_gemm_packed_kernel<true, 32>,
         nvfp4_gemm_packed_kernel<true, 40>, nvfp4_gemm_packed_kernel<true, 48>,
         nvfp4_gemm_packed_kernel<true, 56>, nvfp4_gemm_packed_kernel<true, 64>}};
    const int idx = (int)(K / 2048) - 1;
    if (idx < 0 || idx > 7 || K % 2048 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kernels[out_bf16 ? 1 : 0][idx], grid, dim3(GEMM_WG), 0, s, ap, asp, sg_a, bp,
                       bsp, sg_b, (int)M, (int)N, c);
    return hipGetLastError();
}

int gemm_splitk_parts(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || N % 4 != 0 || K < 512 || K % 512 != 0) return 0;
    // the fewest equal splits of at most SK_KS_MAX K, each a multiple of 512
    for (int64_t S = (K + SK_KS_MAX - 1) / SK_KS_MAX; S <= K / 512; ++S)
        if (K % S == 0 && (K / S) % 512 == 0) return (int)S;
    return 0;
}

hipError_t launch_gemm_mxfp4_splitk(const uint8_t *a_codes, const uint8_t *a_scales,
                                    const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t M,
                                    int64_t N, int64_t K, void *c, bool out_bf16, float *workspace,
                                    hipStream_t s) {
    const int S = gemm_splitk_parts(M, N, K);
    if (S < 1) return hipErrorInvalidValue;
    dim3 grid((unsigned)((N + SK_TN - 1) / SK_TN), (unsigned)S,
              (unsigned)((M + GEMM_TM - 1) / GEMM_TM));
    hipLaunchKernelGGL(mxfp4_gemm_splitk_kernel, grid, dim3(SK_WG), 0, s, (const uint4 *)a_codes,
                       a_scales, (const uint4 *)bt_codes, bt_scales, (int)M, (int)N, (int)K,
                       (int)(K / S), workspace);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n4 = M * N / 4;
    int64_t g = (n4 + 255) / 256;
    if (g > kMaxGrid) g = kMaxGrid;
    auto k = out_bf16 ? splitk_reduce_kernel<true> : splitk_reduce_kernel<false>;
    hipLaunchKernelGGL(k, dim3((unsigned)g), dim3(256), 0, s, (const uint4 *)workspace, n4, S, c);
    return hipGetLastError();
}

hipError_t launch_linear_mxfp4(const void *x, bool x_bf16, const uint8_t *bt_codes,
                               const uint8_t *bt_scales, int64_t M, int64_t N, int64_t K,
                               uint8_t *a_codes, uint8_t *a_scales, void *c, bool out_bf16,
                               bool one_launch, void *workspace, int32_t *status, hipStream_t s,
                               uint32_t spin_limit) {
    dim3 grid((unsigned)((N + GEMM_TN - 1) / GEMM_TN), (unsigned)((M + GEMM_TM - 1) / GEMM_TM));
    const int64_t G = (int64_t)grid.x * grid.y;
    if (one_launch && gemm_lds_ok(a_codes, a_scales, bt_codes, bt_scales, K) &&
        G <= linear_capacity()) {
        using Kn = void (*)(const uint4 *, uint32_t *, uint8_t *, const uint4 *, const uint8_t *,
                            int, int, int, void *, uint64_t *, uint32_t *, uint32_t, int32_t *);
        static const Kn kernels[2][2] = {
            {mxfp4_linear_kernel<false, false>, mxfp4_linear_kernel<false, true>},
            {mxfp4_linear_kernel<true, false>, mxfp4_linear_kernel<true, true>}};
        uint8_t *ws = (uint8_t *)workspace;
        hipLaunchKernelGGL(kernels[out_bf16 ? 1 : 0][x_bf16 ? 1 : 0], grid, dim3(GEMM_WG), 0, s,
                           (const uint4 *)x, (uint32_t *)a_codes, a_scales,
                           (const uint4 *)bt_codes, bt_scales, (int)M, (int)N, (int)K, c,
                           (uint64_t *)(ws + kResidentSlotsOffset),
                           (uint32_t *)(ws + kResidentEpochOffset), spin_limit, status);
        return hipGetLastError();
    }
    // the grid cannot be resident at once (or the shape takes another GEMM
    // kernel): the same two steps as separate launches
    hipError_t e = launch_mx_quantize(x, x_bf16, M * K, 0, a_codes, a_scales, status, s);
    if (e != hipSuccess) return e;
    return launch_gemm_mxfp4(a_codes, a_scales, bt_codes, bt_scales, M, N, K, c, out_bf16, s);
}

hipError_t launch_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *sg_a,
                             const uint8_t *bt_codes, const uint8_t *bt_scales, const float *sg_b,
                             int64_t M, int64_t N, int64_t K, void *c, bool out_bf16,
                             hipStream_t s) {
    auto al = [](const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; };
    if (K % 256 == 0 && K <= GEMM_MAX_K && al(a_codes, 16) && al(bt_codes, 16) &&
        al(a_scales, 16) && al(bt_scales, 16)) {
        dim3 grid((unsigned)((N + GEMM_TN - 1) / GEMM_TN), (unsigned)((M + GEMM_TM - 1) / GEMM_TM));
        auto k = out_bf16 ? nvfp4_gemm_lds_kernel<true> : nvfp4_gemm_lds_kernel<false>;
        hipLaunchKernelGGL(k, grid, dim3(GEMM_WG), 0, s, (const uint4 *)a_codes, a_scales, sg_a,
                           (const uint4 *)bt_codes, bt_scales, sg_b, (int)M, (int)N, (int)K, c);
        return hipGetLastError();
    }
    const int64_t nout = M * N;
    auto k = out_bf16 ? nvfp4_gemm_simple_kernel<true> : nvfp4_gemm_simple_kernel<false>;
    hipLaunchKernelGGL(k, dim3((unsigned)((nout + GEMM_WG - 1) / GEMM_WG)), dim3(GEMM_WG), 0, s,
                       a_codes, a_scales, sg_a, bt_codes, bt_scales, sg_b, (int)M, (int)N, (int)K,
                       c);
    return hipGetLastError();
}

}  // namespace fp4dev
