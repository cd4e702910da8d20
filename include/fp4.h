/*
 * fp4.h - block-scaled FP4 (E2M1) quantization for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfp4.so.  Every tensor argument is a DEVICE pointer into memory
 * the caller owns (allocates and frees); the library allocates nothing.  Its
 * only global state is two per-device records, each filled once and never
 * changed (whether the one-pass NVFP4 kernel fits, from the CU count and
 * occupancy, and how many workgroups of the one-launch W4A4 linear kernel the
 * device holds at once).
 * Calls on different streams may run concurrently unless they share a
 * workspace (or, for fp4_quantize_nvfp4_noalloc, a GPU).  The one-pass NVFP4
 * quantize and the one-launch W4A4 linear meet at a grid barrier that does
 * not need their workgroups to be resident together: a workgroup that waits
 * too long (another kernel holding CUs) finishes by a fallback with the same
 * result, so concurrent calls give the same outputs, only slower.  All work is
 * enqueued asynchronously on `stream` (a hipStream_t passed as void*; NULL is
 * the null stream).
 *
 * Formats (one definition each, as given on the pages cited):
 *  - E2M1 element ("NVFP4 / MXFP4 format" page, charlestar.github.io, section
 *    1): 4-bit code, bit 3 = sign, bits 0-2 index {0, .5, 1, 1.5, 2, 3, 4, 6};
 *    rounding is to the nearest value with ties to the even code, magnitudes
 *    saturate at 6 and the sign bit of the quotient is kept (so -0.0 -> 8).
 *  - Packing (same page, section 1): byte j = code[2j] | code[2j+1] << 4.
 *  - MXFP4 (same page, sections 2 and 5): 32-element blocks, one E8M0 scale
 *    byte c meaning 2^(c-127); the block exponent follows the OCP floor rule
 *    e = floor(log2 amax) - 2 (a zero block takes e = 0; e >= -127).
 *  - NVFP4 (same page, section 3): 16-element blocks, an E4M3FN block scale
 *    s_b = E4M3(A_g / (6 s_g)) (nearest, ties to even, saturating at 448) and
 *    one fp32 tensor scale s_g = A / (6 * 448) (an all-zero tensor takes 1).
 *    Elements are divided by alpha = RN32(s_g * s_b) with a correctly rounded
 *    fp32 division, then rounded to E2M1.
 *
 * Layout: the input is row-major [rows, cols]; blocks run along the last
 * dimension, so cols must be a multiple of the block.  Outputs:
 *   codes  [rows, cols/2]      uint8, two codes per byte (even element low)
 *   scales [rows, cols/block]  uint8, one scale byte per block, row-major
 * Because every row holds whole blocks, the flat order of elements, codes and
 * scales is the row-major order; the library treats the tensor as flat.  The
 * *_packed entry points use the MFMA operand order instead, described at
 * fp4_pack_mxfp4_operand (MXFP4) and fp4_pack_nvfp4_operand (NVFP4).
 *
 * Errors.  Argument errors are returned synchronously, before any HIP call
 * (so they are testable without a GPU).  Data-dependent conditions are found
 * on the device and OR-ed into *status (a device int32 the caller zeroes
 * beforehand; may be NULL to ignore them) as FP4_FLAG_* bits; when
 * FP4_FLAG_NONFINITE or FP4_FLAG_SCALE_UNDERFLOW is set the outputs are
 * unspecified (FP4_FLAG_BARRIER_TIMEOUT is information only).
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are 32-bit integers on both sides of the ABI.  In C++ the
 * underlying type is fixed to int32_t, so that a value outside the named
 * constants (which a C or ctypes caller may pass) is still a value of the
 * type and is rejected by the checks below rather than being undefined. */
#ifdef __cplusplus
#define FP4_ENUM enum : int32_t
#else
#define FP4_ENUM enum
#endif

typedef FP4_ENUM {
    FP4_OK = 0,
    FP4_E_ARG = 1,       /* null pointer, wrong block size, bad candidate grid   */
    FP4_E_SHAPE = 2,     /* rows < 1, cols < 1, or cols not a multiple of block   */
    FP4_E_DTYPE = 3,     /* unknown fp4_dtype / fp4_format                        */
    FP4_E_ALIGN = 4,     /* a pointer is not aligned as documented                */
    FP4_E_WORKSPACE = 5, /* workspace missing or smaller than the *_workspace_bytes
                            call of the entry point reports                        */
    FP4_E_HIP = 6        /* a HIP runtime call (e.g. a launch) failed             */
} fp4_status;

/* Device-side condition flags OR-ed into *status. */
#define FP4_FLAG_NONFINITE 1       /* an input element is NaN or +-Inf          */
#define FP4_FLAG_SCALE_UNDERFLOW 2 /* tensor scale, block scale or alpha is 0   */
#define FP4_FLAG_BARRIER_TIMEOUT 4 /* information, not an error: a grid-barrier
                                      wait timed out and some workgroup took the
                                      fallback; the outputs are exact            */

typedef FP4_ENUM { FP4_F32 = 0, FP4_BF16 = 1 } fp4_dtype;
typedef FP4_ENUM { FP4_MXFP4 = 0, FP4_NVFP4 = 1 } fp4_format;
typedef FP4_ENUM { FP4_MX_RULE_OCP = 0, FP4_MX_RULE_CEIL = 1, FP4_MX_RULE_MSE = 2 } fp4_mx_rule;
typedef FP4_ENUM { FP4_LINEAR_ONE_LAUNCH = 0, FP4_LINEAR_TWO_LAUNCHES = 1 } fp4_linear_mode;
#undef FP4_ENUM

/*
 * MXFP4 quantize ("NVFP4 / MXFP4 format" page, sections 1, 2 and 5).
 *   x       [rows, cols] fp32 or bf16, 16-byte aligned
 *   block   must be 32
 *   codes   [rows*cols/2] bytes, 16-byte aligned
 *   scales  [rows*cols/32] E8M0 bytes
 *   status  device int32 or NULL (FP4_FLAG_NONFINITE)
 * One pass over x.  Deterministic.
 */
fp4_status fp4_quantize_mxfp4(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                              int32_t block, uint8_t *codes, uint8_t *scales,
                              int32_t *status, void *stream);

/*
 * MXFP4 quantize with another rule for the block exponent ("NVFP4 / MXFP4
 * format" page, section 5: the format fixes the set of E8M0 scales, not how a
 * block picks one).  Element rounding is the same as fp4_quantize_mxfp4.
 *   rule  FP4_MX_RULE_OCP   e = floor(log2 amax) - 2 (as fp4_quantize_mxfp4);
 *         FP4_MX_RULE_CEIL  the section's ModelOpt rule, scale
 *                           2^ceil(log2(amax / 6)): the smallest e with
 *                           6 * 2^e >= amax, so nothing saturates;
 *         FP4_MX_RULE_MSE   the squared error of the block, an fp32 sum taken
 *                           pairwise in index order, evaluated at e0 - 1, e0
 *                           and e0 + 1 around the floor rule's e0; e0 stays
 *                           unless a neighbour is strictly better, e0 - 1 is
 *                           tried first.
 *         In every rule e is clamped at -127 and a zero block takes e = 0.
 *   Other arguments, errors and status as for fp4_quantize_mxfp4 (FP4_E_ARG
 *   also for an unknown rule).  One pass over x.  Deterministic.
 */
fp4_status fp4_quantize_mxfp4_rule(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                   int32_t block, fp4_mx_rule rule, uint8_t *codes,
                                   uint8_t *scales, int32_t *status, void *stream);

/*
 * NVFP4 quantize ("NVFP4 / MXFP4 format" page, section 3, two-level scale
 * and zero/tiny contract).
 *   x, xt, rows, cols, codes as for MXFP4; block must be 16
 *   scales        [rows*cols/16] E4M3FN bytes
 *   global_scale  device float: receives s_g (dequantize direction, x ~ s_g*s_b*p)
 *   workspace     device memory of at least fp4_workspace_bytes(FP4_NVFP4, ...)
 *                 bytes, 16-byte aligned, ZERO-FILLED before its first use and
 *                 then left to the library: it keeps a barrier epoch there
 *                 between calls.  Calls that share a workspace must be ordered
 *                 (one stream, or synchronised); the same workspace may serve
 *                 fp4_scale_search too.
 *   status        FP4_FLAG_NONFINITE, FP4_FLAG_SCALE_UNDERFLOW,
 *                 FP4_FLAG_BARRIER_TIMEOUT (information only: outputs exact)
 * s_g needs the amax of the whole tensor.  A bf16 tensor that fits on chip
 * (one 512 KiB slice per CU: 8192 x 8192 on 256 CUs) is read from HBM once
 * by a single kernel whose workgroups, one per CU, meet at a grid barrier
 * after the amax; other inputs take two kernels, a tensor-amax pass and a
 * quantize pass (which reads the amax in stream order, without a host round
 * trip).  Results are identical either way.  Deterministic.
 */
fp4_status fp4_quantize_nvfp4(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                              int32_t block, uint8_t *codes, uint8_t *scales,
                              float *global_scale, void *workspace, size_t workspace_bytes,
                              int32_t *status, void *stream);

/*
 * NVFP4 quantize without allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results, errors and status as
 * fp4_quantize_nvfp4, minus the workspace: the library uses its own fixed
 * scratch instead, FP4_NOALLOC_SCRATCH_BYTES bytes per GPU in a static device
 * array, which stays allocated until the process ends.
 *   - The scratch need does not grow with the tensor: every shape
 *     fp4_quantize_nvfp4 accepts fits (a shape that did not would be rejected
 *     with FP4_E_WORKSPACE).
 *   - The first call on a device sets the scratch up: it looks up the array's
 *     device address and zero-fills it with a synchronous hipMemset waited on
 *     the null stream (FP4_E_HIP if that fails, e.g. when the first call is
 *     made while a stream is being captured; make one call outside capture
 *     first).  Later calls make no allocating or synchronising HIP call.
 *   - Every call on one GPU shares that GPU's scratch and keeps the last
 *     call's contents there (the grid barrier's epoch).  Calls that overlap
 *     in time on one GPU (different streams, or different host threads
 *     without ordering) RACE on it: their results are then unspecified.
 *     Order them on one stream, or use fp4_quantize_nvfp4 with a workspace
 *     per stream.
 */
#define FP4_NOALLOC_SCRATCH_BYTES 20480u
fp4_status fp4_quantize_nvfp4_noalloc(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                      int32_t block, uint8_t *codes, uint8_t *scales,
                                      float *global_scale, int32_t *status, void *stream);

/*
 * Quantize with stochastic element rounding (Ultralytics glossary "FP4",
 * section "Inferenza e addestramento FP4": NVFP4 pretraining rounds
 * gradients stochastically; the pages name the technique, not a rule).
 *   fmt     FP4_MXFP4 (block 32: scales as fp4_quantize_mxfp4) or FP4_NVFP4
 *           (block 16: s_g and block scales as fp4_quantize_nvfp4)
 *   seed    64-bit seed of the random bits
 *   global_scale, workspace, workspace_bytes  NVFP4 as for
 *           fp4_quantize_nvfp4; ignored (may be NULL) for MXFP4
 *   Other arguments, errors and status flags as for the deterministic
 *   quantizer of the format.
 * Element rounding: q = RN32(x / scale) as in the deterministic encoder; with
 * lo <= |q| < hi the neighbouring E2M1 magnitudes, q rounds to hi iff
 * r * (hi - lo) * 2^-24 < |q| - lo, where r is the element's 24 random bits
 * (so up with probability (|q| - lo) / (hi - lo), the expected value being
 * q); grid values stay, |q| >= 6 gives 6, the sign bit is kept.
 * Random bits of element i (flat row-major index): the (i/2 + 1)-th output of
 * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) started at state seed,
 * i.e. its finalizer applied to seed + (i/2 + 1) * 0x9E3779B97F4A7C15; even
 * i take the top 24 bits of the low 32-bit half, odd i of the high half.
 * Results depend on (x, seed) only: deterministic for a given seed.  NVFP4
 * runs two kernels (tensor amax, then quantize).
 */
fp4_status fp4_quantize_sr(fp4_format fmt, const void *x, fp4_dtype xt, int64_t rows,
                           int64_t cols, int32_t block, uint64_t seed, uint8_t *codes,
                           uint8_t *scales, float *global_scale, void *workspace,
                           size_t workspace_bytes, int32_t *status, void *stream);

/*
 * Dequantize ("FP4 / NVFP4 math summary" page, section 10: x_hat = q * alpha).
 *   fmt           FP4_MXFP4 (block 32) or FP4_NVFP4 (block 16)
 *   codes, scales as produced by the quantizers (any byte values accepted)
 *   global_scale  device float s_g for NVFP4, ignored (may be NULL) for MXFP4
 *   y             [rows, cols] fp32 or bf16 output, 16-byte aligned
 * MXFP4: y = E2M1(c) * 2^(s-127), exact in fp32 and bf16 for s <= 252.
 * NVFP4: y = RN_out(RN32(E2M1(c) * RN32(s_g * E4M3(s)))).
 * A NaN scale byte (E8M0 255, E4M3 0x7F / 0xFF) yields NaN outputs.
 */
fp4_status fp4_dequantize(fp4_format fmt, const uint8_t *codes, const uint8_t *scales,
                          const float *global_scale, int64_t rows, int64_t cols,
                          int32_t block, void *y, fp4_dtype yt, void *stream);

/*
 * MSE-optimal NVFP4 block-scale search ("FP4 / NVFP4 math summary" page,
 * section 9: minimise sum (x - s * Round_FP4(x / s))^2; "NVFP4 / MXFP4 format"
 * page, section 4: the encoded scale is what quantizes).
 *   Candidate k of n: c_k = RN32(((n-1-k) c_lo + k c_hi) / (n-1)); its block
 *   scale is E4M3(c_k * A_g / (6 s_g)) (exact real; code 0 skipped), and its
 *   loss is evaluated in fp32: q = RN32(x/alpha), x_hat = RN32(E2M1(q)*alpha),
 *   e = x - x_hat, sum of e*e as a balanced pairwise tree over the 16
 *   elements in index order.  The smallest k with the least loss wins; the
 *   block is then quantized with it.  s_g is the NVFP4 tensor scale.
 *   Requirements: block 16, n_candidates >= 2, 0 < c_lo <= c_hi <= 4 and
 *   (c_hi - c_lo) / (n_candidates - 1) <= c_lo / 24 (the candidate grid is
 *   then finer than the E4M3 grid, whose rounding intervals are at least
 *   1/15 of their value wide, so the distinct candidate scales of a block
 *   are exactly the consecutive E4M3 codes between the two ends).
 *   Other arguments as for fp4_quantize_nvfp4 (two kernels: tensor amax, then
 *   search and quantize); codes must be at least 8-byte aligned (FP4_E_ALIGN).
 *   Deterministic.
 */
fp4_status fp4_scale_search(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                            int32_t block, int32_t n_candidates, float c_lo, float c_hi,
                            uint8_t *codes, uint8_t *scales, float *global_scale,
                            void *workspace, size_t workspace_bytes, int32_t *status,
                            void *stream);

/*
 * Brute-force NVFP4 block-scale search ("NVFP4 / MXFP4 format" page, section
 * 4: every legal E4M3 scale tried on the block [0.4 x 15, 3.6], where 0.875
 * beats the max-based 0.625).  As fp4_scale_search, except that the
 * candidates of a block with amax > 0 are all E4M3 codes 1..126 whose alpha
 * is nonzero; the winner is the smallest code with the least loss.  About 14
 * times the candidate evaluations of the 64-candidate search.  Deterministic.
 */
fp4_status fp4_scale_search_exhaustive(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                       int32_t block, uint8_t *codes, uint8_t *scales,
                                       float *global_scale, void *workspace,
                                       size_t workspace_bytes, int32_t *status, void *stream);

/*
 * MXFP4 x MXFP4 block-scaled GEMM ("FP4, FP8 and INT8/INT4" page,
 * tom-jerr.github.io, section 5.1: C = sum_t sA sB sum_{k in t} qA qB with
 * fp32 accumulation; "NVFP4 / MXFP4 format" page, section 6: scales come out
 * only per K block, and storing the weight as N x K makes its last-dimension
 * blocks the K blocks).
 *   a_codes   [M, K/2], a_scales  [M, K/32]   (A quantized along K)
 *   bt_codes  [N, K/2], bt_scales [N, K/32]   (B stored transposed as Bt [N, K])
 *   c         [M, N] fp32 or bf16 (bf16 = RNE of the fp32 result)
 * K must be a multiple of 32; codes 16-byte aligned with K/2 a multiple of 16
 * (K % 32 == 0 suffices), c 4-byte aligned.  The summation order is fixed, so
 * results are deterministic.
 */
fp4_status fp4_gemm_mxfp4(const uint8_t *a_codes, const uint8_t *a_scales,
                          const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t M,
                          int64_t N, int64_t K, void *c, fp4_dtype ct, void *stream);

/*
 * The same MXFP4 x MXFP4 GEMM split over K, for short A (the operation and
 * the sources as fp4_gemm_mxfp4).  With one 128-row tile of A or two, the
 * tiling of fp4_gemm_mxfp4 makes every workgroup read all of A; here each of
 * S workgroups per 128 x 128 tile of C takes one of S equal K ranges (at most
 * 2048 K each, a multiple of 512) and writes fp32 partial sums, then a second
 * kernel adds the S partials of each output in increasing K-range order and
 * rounds once (bf16 = RNE of the fp32 sum).
 *   a_codes .. c, ct   as for fp4_gemm_mxfp4; K a multiple of 512, N a
 *                      multiple of 4; codes and scales 16-byte aligned, c 16
 *                      (fp32) or 8 (bf16) byte aligned
 *   workspace          device memory of at least
 *                      fp4_gemm_splitk_workspace_bytes(M, N, K) bytes,
 *                      16-byte aligned; its contents are scratch (S x M x N
 *                      fp32), overwritten by each call.  Calls that share a
 *                      workspace must be stream-ordered.
 * Errors: FP4_E_SHAPE for shapes this path does not take (use
 * fp4_gemm_mxfp4), FP4_E_WORKSPACE for a missing or short workspace.  The
 * summation differs from fp4_gemm_mxfp4's (fp32 partial sums per K range)
 * but is fixed, so results are deterministic.
 */
fp4_status fp4_gemm_mxfp4_splitk(const uint8_t *a_codes, const uint8_t *a_scales,
                                 const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t M,
                                 int64_t N, int64_t K, void *c, fp4_dtype ct, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* Bytes of workspace fp4_gemm_mxfp4_splitk needs for this shape: S * M * N *
 * 4 with S = the number of K ranges; 0 if the shape is not supported. */
size_t fp4_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * MFMA operand order for MXFP4 operands.  OCP leaves the physical layout of
 * elements and scales to the implementation ("NVFP4 / MXFP4 format" page,
 * section 7); this one serves the GEMM below.  An MXFP4 matrix X with rows
 * rows and K values per row (codes [rows, K/2], scales [rows, K/32], the
 * layout the quantizers write) becomes one buffer:
 *   codes, for each row tile rt of 32 rows (the last one padded with zero
 *   codes) and each K step ks of 64 values, 1024 bytes: bytes 16 l .. 16 l +
 *   15 hold the codes of row 32 rt + l % 32, K block 2 ks + l / 32
 *   (l = 0..63), as stored in that row;
 *   then scales, for each row tile and each group q of eight K steps, 512
 *   bytes: byte 8 l + i is the E8M0 byte of row 32 rt + l % 32 and K block
 *   2 (8 q + i) + l / 32 (127 on padding rows).
 * fp4_packed_operand_bytes(rows, K) is its size: 32 ceil(rows / 32) (K/2 +
 * K/32) bytes, or 0 unless rows >= 1 and K is a positive multiple of 512.
 *   codes, scales  the row-major operand (device); codes 16-byte aligned
 *   packed         device output of at least that many bytes, 16-byte aligned
 * Errors: FP4_E_SHAPE (size 0), FP4_E_WORKSPACE (packed_bytes too small),
 * FP4_E_ALIGN.  Packing moves bytes only (bit-exact).
 */
int64_t fp4_packed_operand_bytes(int64_t rows, int64_t K);
fp4_status fp4_pack_mxfp4_operand(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                  int64_t K, uint8_t *packed, size_t packed_bytes, void *stream);

/*
 * The MXFP4 x MXFP4 GEMM of fp4_gemm_mxfp4 (same operation and sources) on
 * packed operands: a_packed = A [M, K] and bt_packed = Bt [N, K], each made
 * by fp4_pack_mxfp4_operand (a weight is packed once).  Every operand load
 * is one contiguous kilobyte.  K must be a multiple of 2048, at most 16384;
 * each packed operand at most 1 GiB; operands 16-byte aligned, c 4-byte
 * aligned (FP4_E_SHAPE / FP4_E_ALIGN otherwise).  A workgroup's four waves
 * take the four quarters of K for a 128 x 32 tile of C and add their partial
 * tiles in a fixed order, so results are deterministic; the summation order
 * differs from fp4_gemm_mxfp4's.
 */
fp4_status fp4_gemm_mxfp4_packed(const uint8_t *a_packed, const uint8_t *bt_packed, int64_t M,
                                 int64_t N, int64_t K, void *c, fp4_dtype ct, void *stream);

/*
 * MXFP4 quantize of x [rows, cols] (fp32 or bf16) by the OCP floor rule, as
 * fp4_quantize_mxfp4 (same codes and scale bytes, "NVFP4 / MXFP4 format"
 * page, section 5), written directly in the packed layout of
 * fp4_pack_mxfp4_operand (padding rows come out as zero codes with scale
 * byte 127).  cols must be a multiple of 512; packed must hold
 * fp4_packed_operand_bytes(rows, cols) bytes, 16-byte aligned; x 16-byte
 * aligned.  status as for fp4_quantize_mxfp4 (FP4_FLAG_NONFINITE).
 * Errors: FP4_E_SHAPE, FP4_E_WORKSPACE (packed too small), FP4_E_ALIGN.
 */
fp4_status fp4_quantize_mxfp4_packed(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                     uint8_t *packed, size_t packed_bytes, int32_t *status,
                                     void *stream);

/*
 * W4A4 linear on a packed weight: x [M, K] (fp32 or bf16) quantized to
 * MXFP4 by the floor rule into a_packed (packed layout), then
 * fp4_gemm_mxfp4_packed with bt_packed = Bt [N, K] packed once (the
 * operation of fp4_linear_mxfp4; "FP4, FP8 and INT8/INT4" page, section
 * 5.1).  Two launches on one stream.  K a multiple of 2048, at most 16384;
 * a_packed at least fp4_packed_operand_bytes(M, K) bytes; alignment as for
 * the two calls.  status receives FP4_FLAG_NONFINITE for x.
 */
fp4_status fp4_linear_mxfp4_packed(const void *x, fp4_dtype xt, int64_t M, int64_t K,
                                   const uint8_t *bt_packed, int64_t N, uint8_t *a_packed,
                                   size_t a_packed_bytes, void *c, fp4_dtype ct, int32_t *status,
                                   void *stream);

/*
 * NVFP4 x NVFP4 GEMM ("NVFP4 / MXFP4 format" page, section 6:
 * Y = a_X a_W sum_g b^X_g b^W_g sum_{k in g} p^X_k p^W_k, 16-element groups
 * along K, E4M3 block scales b, one fp32 tensor scale a per operand).
 *   a_codes [M, K/2], a_scales [M, K/16] E4M3, a_global_scale device float
 *   bt_codes [N, K/2], bt_scales [N, K/16], bt_global_scale   (B as Bt [N, K])
 *   c       [M, N] fp32 or bf16
 * The products of FP4 values and block scales are exact (fp16 operands of
 * the fp16 MFMA), the sums fp32; the tensor scales multiply the fp32 result
 * once: c = RN(acc * RN32(a_X a_W)).  K must be a multiple of 16; a multiple
 * of 256 up to 8192 with 16-byte aligned codes and scales takes the staged
 * kernel, other shapes a slow one-output-per-thread kernel.  Scale bytes are
 * read as E4M3FN (sign bit honoured, 0x7F NaN).  Deterministic.
 */
fp4_status fp4_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales,
                          const float *a_global_scale, const uint8_t *bt_codes,
                          const uint8_t *bt_scales, const float *bt_global_scale, int64_t M,
                          int64_t N, int64_t K, void *c, fp4_dtype ct, void *stream);

/*
 * MFMA operand order for NVFP4 operands (the physical layout is the
 * implementation's choice, "NVFP4 / MXFP4 format" page, section 7).  An
 * NVFP4 matrix X with rows rows and K values per row (codes [rows, K/2],
 * E4M3 scales [rows, K/16]) becomes one buffer:
 *   codes exactly as in fp4_pack_mxfp4_operand (1024 bytes per row tile of
 *   32 rows and K step of 64 values; bytes 16 l .. 16 l + 15 hold row
 *   32 rt + l % 32, values 32 (2 ks + l / 32) .. + 31);
 *   then scales, for each row tile and each group q of eight K steps, 1024
 *   bytes: byte 16 l + 2 i + b is the E4M3 byte of row 32 rt + l % 32 and
 *   16-element block 4 (8 q + i) + 2 (l / 32) + b (0 on padding rows).
 * fp4_nv_packed_operand_bytes(rows, K) is its size: 32 ceil(rows / 32)
 * (K/2 + K/16) bytes, or 0 unless rows >= 1 and K is a positive multiple
 * of 512.  The tensor scale is not part of the buffer.
 *   codes, scales  the row-major operand (device); codes 16-byte aligned
 *   packed         device output of at least that many bytes, 16-byte aligned
 * Errors: FP4_E_SHAPE (size 0), FP4_E_WORKSPACE (packed_bytes too small),
 * FP4_E_ALIGN.  Packing moves bytes only (bit-exact).
 */
int64_t fp4_nv_packed_operand_bytes(int64_t rows, int64_t K);
fp4_status fp4_pack_nvfp4_operand(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                  int64_t K, uint8_t *packed, size_t packed_bytes, void *stream);

/*
 * The NVFP4 x NVFP4 GEMM of fp4_gemm_nvfp4 (same operation and sources) on
 * packed operands: a_packed = A [M, K] and bt_packed = Bt [N, K], each made
 * by fp4_pack_nvfp4_operand, with their tensor scales a_global_scale and
 * bt_global_scale (device floats, 4-byte aligned).  K must be a multiple of
 * 2048, at most 16384; each packed operand at most 1 GiB; operands 16-byte
 * aligned, c 4-byte aligned (FP4_E_SHAPE / FP4_E_ALIGN otherwise).  Products
 * of FP4 values and block scales are exact, sums fp32; a workgroup's four
 * waves take the four quarters of K for a 128 x 32 tile of C and add their
 * partial tiles in a fixed order, then c = RN(acc * RN32(a_X a_W)).
 * Deterministic; the summation order differs from fp4_gemm_nvfp4's.
 */
fp4_status fp4_gemm_nvfp4_packed(const uint8_t *a_packed, const float *a_global_scale,
                                 const uint8_t *bt_packed, const float *bt_global_scale,
                                 int64_t M, int64_t N, int64_t K, void *c, fp4_dtype ct,
                                 void *stream);

/*
 * NVFP4 quantize of x [rows, cols] (fp32 or bf16), as fp4_quantize_nvfp4
 * (same codes, E4M3 scale bytes and tensor scale, "NVFP4 / MXFP4 format"
 * page, section 3), written directly in the packed layout of
 * fp4_pack_nvfp4_operand (padding rows come out as zero codes and zero scale
 * bytes).  Two launches on `stream`: the tensor amax, then the encode.
 * cols must be a multiple of 512; packed must hold
 * fp4_nv_packed_operand_bytes(rows, cols) bytes, 16-byte aligned; x 16-byte
 * aligned; global_scale receives s_g; workspace as for fp4_quantize_nvfp4.
 * status as for fp4_quantize_nvfp4 (FP4_FLAG_NONFINITE,
 * FP4_FLAG_SCALE_UNDERFLOW; with either, the outputs are unspecified).
 * Errors: FP4_E_SHAPE, FP4_E_WORKSPACE (packed or workspace too small),
 * FP4_E_ALIGN.
 */
fp4_status fp4_quantize_nvfp4_packed(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                     uint8_t *packed, size_t packed_bytes, float *global_scale,
                                     void *workspace, size_t workspace_bytes, int32_t *status,
                                     void *stream);

/*
 * NVFP4 W4A4 linear on a packed weight: x [M, K] (fp32 or bf16) quantized
 * to NVFP4 into a_packed with its tensor scale in a_global_scale
 * (fp4_quantize_nvfp4_packed), then fp4_gemm_nvfp4_packed with bt_packed =
 * Bt [N, K] packed once and its tensor scale bt_global_scale (the W4A4
 * linear of the "FP4, FP8 and INT8/INT4" page, section 5.1, in the NVFP4
 * format).  Three launches on one stream.  K a multiple of 2048, at most
 * 16384; a_packed at least fp4_nv_packed_operand_bytes(M, K) bytes;
 * workspace as for fp4_quantize_nvfp4; alignment as for the two calls.
 * status receives the quantize's flags.
 */
fp4_status fp4_linear_nvfp4_packed(const void *x, fp4_dtype xt, int64_t M, int64_t K,
                                   const uint8_t *bt_packed, const float *bt_global_scale,
                                   int64_t N, uint8_t *a_packed, size_t a_packed_bytes,
                                   float *a_global_scale, void *c, fp4_dtype ct,
                                   void *workspace, size_t workspace_bytes, int32_t *status,
                                   void *stream);

/*
 * W4A4 linear layer: the activations quantized to MXFP4, then the MXFP4 GEMM
 * ("FP4, FP8 and INT8/INT4" page, tom-jerr.github.io, section 5: the cost of
 * a low-bit linear layer is the activation quantize plus the block-scaled
 * MMA; "NVFP4 / MXFP4 format" page, section 6: blocks along K).
 *   x          [M, K] fp32 or bf16 activations, 16-byte aligned
 *   bt_codes, bt_scales   the MXFP4 weight Bt [N, K] as for fp4_gemm_mxfp4
 *   a_codes    [M, K/2] bytes, a_scales [M, K/32]: receive x quantized exactly
 *              as fp4_quantize_mxfp4 does (OCP floor rule); 16-byte aligned
 *   c          [M, N] fp32 or bf16, the GEMM of a_codes with Bt
 *   workspace  as for fp4_quantize_nvfp4 (fp4_workspace_bytes(FP4_NVFP4, M, K)
 *              bytes, zero-filled before its first use, then left to the
 *              library; calls sharing it must be stream-ordered)
 *   status     FP4_FLAG_NONFINITE (x), FP4_FLAG_BARRIER_TIMEOUT (information
 *              only: the outputs are exact)
 *   mode       FP4_LINEAR_ONE_LAUNCH: when the GEMM's grid (ceil(N/32) *
 *              ceil(M/128) workgroups) fits on the device at once and K is a
 *              multiple of 512 up to 8192, one kernel quantizes x (each
 *              workgroup a share), meets at a grid barrier and multiplies;
 *              else, and under FP4_LINEAR_TWO_LAUNCHES, the two steps run as
 *              two launches on the stream.  The barrier and the cache
 *              write-back and invalidation around it cost more than a kernel
 *              boundary inside a captured graph; one launch pays where each
 *              launch is submitted on its own.
 * K must be a multiple of 32.  Results are identical in both modes and match
 * fp4_quantize_mxfp4 followed by fp4_gemm_mxfp4.  Deterministic.
 */
fp4_status fp4_linear_mxfp4(const void *x, fp4_dtype xt, int64_t M, int64_t K,
                            const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t N,
                            uint8_t *a_codes, uint8_t *a_scales, void *c, fp4_dtype ct,
                            fp4_linear_mode mode, void *workspace, size_t workspace_bytes,
                            int32_t *status, void *stream);

/*
 * Row-padded layout ("NVFP4 / MXFP4 format" page, section 8): each row of a
 * [rows, cols] matrix is padded with zeros to whole blocks (32 for MXFP4, 16
 * for NVFP4), pcols = ceil(cols / block) * block, and the padded matrix is
 * quantized: codes [rows, pcols/2] (padding codes are 0), scales
 * [rows, pcols/block]; the NVFP4 tensor scale is that of the rows*cols
 * logical values.  The logical cols is the metadata the decode needs.
 *   fp4_quantize_padded: any cols >= 1; x 2-byte (bf16) or 4-byte (fp32)
 *     aligned, codes 4-byte aligned; global_scale, workspace and
 *     workspace_bytes as for fp4_quantize_nvfp4 (NVFP4 only, ignored for
 *     MXFP4); status as for the format's quantize.  Identical to
 *     fp4_quantize_mxfp4 / _nvfp4 when cols is a multiple of the block.
 *   fp4_dequantize_padded: decodes the padded layout and writes only the
 *     logical [rows, cols] values of y (fp32 or bf16), as fp4_dequantize.
 *   fp4_padded_storage_bytes: rows * ceil(cols/block) * (block/2 + 1), plus
 *     4 for NVFP4's tensor scale (-1 for invalid arguments, and for shapes
 *     of more than 2^40 padded elements, which the entry points reject).
 * Values are moved one by one (rows need not be aligned): these are for
 * shapes the block-aligned entry points reject.  Deterministic.
 */
fp4_status fp4_quantize_padded(fp4_format fmt, const void *x, fp4_dtype xt, int64_t rows,
                               int64_t cols, uint8_t *codes, uint8_t *scales,
                               float *global_scale, void *workspace, size_t workspace_bytes,
                               int32_t *status, void *stream);
fp4_status fp4_dequantize_padded(fp4_format fmt, const uint8_t *codes, const uint8_t *scales,
                                 const float *global_scale, int64_t rows, int64_t cols, void *y,
                                 fp4_dtype yt, void *stream);
int64_t fp4_padded_storage_bytes(fp4_format fmt, int64_t rows, int64_t cols);

/*
 * For tests of the grid barrier's fallback (the one-pass NVFP4 quantize and
 * the one-launch W4A4 linear): fp4_quantize_nvfp4 and fp4_linear_mxfp4 with
 * the number of times a workgroup polls the other workgroups' slots before
 * it stops waiting, takes the fallback and raises FP4_FLAG_BARRIER_TIMEOUT
 * (0 = after the first poll) as an argument.  The entry points above use
 * FP4_BARRIER_SPIN_LIMIT_DEFAULT polls (a few milliseconds, far above the
 * barrier's usual microseconds).  Results are exact whatever the value; only
 * the time changes.  Other arguments, errors and outputs as for those two.
 */
#define FP4_BARRIER_SPIN_LIMIT_DEFAULT 2048u
fp4_status fp4_debug_quantize_nvfp4_spin(const void *x, fp4_dtype xt, int64_t rows,
                                         int64_t cols, int32_t block, uint8_t *codes,
                                         uint8_t *scales, float *global_scale, void *workspace,
                                         size_t workspace_bytes, int32_t *status, void *stream,
                                         uint32_t spin_limit);
fp4_status fp4_debug_linear_mxfp4_spin(const void *x, fp4_dtype xt, int64_t M, int64_t K,
                                       const uint8_t *bt_codes, const uint8_t *bt_scales,
                                       int64_t N, uint8_t *a_codes, uint8_t *a_scales, void *c,
                                       fp4_dtype ct, fp4_linear_mode mode, void *workspace,
                                       size_t workspace_bytes, int32_t *status, void *stream,
                                       uint32_t spin_limit);

/* Bytes of device workspace fp4_quantize_nvfp4 / fp4_scale_search need for a
 * [rows, cols] input (0 for MXFP4). */
size_t fp4_workspace_bytes(fp4_format fmt, int64_t rows, int64_t cols);

/* Static English text for a status code. */
const char *fp4_status_str(fp4_status s);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H */
