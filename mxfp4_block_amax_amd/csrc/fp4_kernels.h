// fp4_kernels.h - launchers shared by the C ABI (fp4_api.hip) and the kernel
// translation units.  Internal to libfp4.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dev {

// Largest grid of the streaming kernels (workgroups of 256 threads); waves
// loop over tiles beyond it.
constexpr int kMaxGrid = 4096;
// Workgroups (hence partial maxima) of the tensor-amax pass.
constexpr int kAmaxPartials = 2048;
// Workspace of the NVFP4 / scale-search calls: the pass-1 partial maxima,
// then (one-pass NVFP4 path) an epoch word and one 64-bit barrier slot per
// workgroup.  The epoch and slots must start zeroed and are kept between
// calls.
constexpr size_t kResidentEpochOffset = kAmaxPartials * sizeof(uint32_t);
constexpr size_t kResidentSlotsOffset = kResidentEpochOffset + 256;
constexpr int kResidentSlots = 1024;
constexpr size_t kNvWorkspaceBytes = kResidentSlotsOffset + kResidentSlots * sizeof(uint64_t);
// Size of the fixed device scratch of the no-allocation NVFP4 entry point:
// one NVFP4 workspace, rounded up to 4 KiB.
constexpr size_t kNoAllocScratchBytes = (kNvWorkspaceBytes + 4095) / 4096 * 4096;
// Polls of the grid barrier before a workgroup takes the fallback (a few
// milliseconds; a poll takes a microsecond or two).  The launchers of the
// two grid-barrier kernels take the limit as an argument; only the debug
// entry points pass another.
constexpr uint32_t kResidentSpinLimit = 2048;
constexpr int kMaxDevices = 64;

// rule: 0 the OCP floor rule, 1 the ceil rule, 2 the three-exponent search
hipError_t launch_mx_quantize(const void *x, bool bf16, int64_t n, int rule, uint8_t *codes,
                              uint8_t *scales, int32_t *status, hipStream_t s);
#ifdef FP4_PHASE_CLOCK
hipError_t read_phase_clock(uint64_t *host, size_t n);
#endif
hipError_t launch_nv_quantize(const void *x, bool bf16, int64_t n, uint8_t *codes,
                              uint8_t *scales, float *global_scale, void *workspace,
                              int32_t *status, hipStream_t s,
                              uint32_t spin_limit = kResidentSpinLimit);
// Stochastic element rounding (fmt 0 MXFP4, 1 NVFP4 in two passes); the
// random bits of element i depend on seed and i only.
hipError_t launch_quantize_sr(int fmt, const void *x, bool bf16, int64_t n, uint64_t seed,
                              uint8_t *codes, uint8_t *scales, float *global_scale,
                              void *workspace, int32_t *status, hipStream_t s);
// all: every E4M3 code is a candidate (c_lo and c_hi unused)
hipError_t launch_scale_search(const void *x, bool bf16, int64_t n, bool all, float c_lo,
                               float c_hi, uint8_t *codes, uint8_t *scales, float *global_scale,
                               void *workspace, int32_t *status, hipStream_t s);
hipError_t launch_dequantize(int fmt, const uint8_t *codes, const uint8_t *scales,
                             const float *global_scale, int64_t n, void *y, bool out_bf16,
                             hipStream_t s);
// Row-padded layout: rows of cols values padded with zeros to whole blocks
// (32 MXFP4, 16 NVFP4); codes [rows, pcols/2], scales [rows, pcols/block].
hipError_t launch_quantize_padded(int fmt, const void *x, bool bf16, int64_t rows, int64_t cols,
                                  uint8_t *codes, uint8_t *scales, float *global_scale,
                                  void *workspace, int32_t *status, hipStream_t s);
hipError_t launch_dequantize_padded(int fmt, const uint8_t *codes, const uint8_t *scales,
                                    const float *global_scale, int64_t rows, int64_t cols,
                                    void *y, bool out_bf16, hipStream_t s);
hipError_t launch_gemm_mxfp4(const uint8_t *a_codes, const uint8_t *a_scales,
                             const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t M,
                             int64_t N, int64_t K, void *c, bool out_bf16, hipStream_t s);
// MFMA operand order: bytes of a packed MXFP4 operand with rows x K values
// (0 unless K is a positive multiple of 512), the pack, and the GEMM on two
// packed operands (K a multiple of 2048, at most 16384).
int64_t packed_operand_bytes(int64_t rows, int64_t K);
hipError_t launch_pack_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                             uint8_t *packed, hipStream_t s);
hipError_t launch_gemm_mxfp4_packed(const uint8_t *a_packed, const uint8_t *bt_packed, int64_t M,
                                    int64_t N, int64_t K, void *c, bool out_bf16, hipStream_t s);
// The NVFP4 operands in fp16-MFMA operand order: bytes of a packed operand
// (0 when K is not a multiple of 512), its packing, and the GEMM on two packed
// operands (K a multiple of 2048, at most 16384).
int64_t nv_packed_operand_bytes(int64_t rows, int64_t K);
hipError_t launch_pack_nvfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                             uint8_t *packed, hipStream_t s);
hipError_t launch_gemm_nvfp4_packed(const uint8_t *a_packed, const float *sg_a,
                                    const uint8_t *bt_packed, const float *sg_b, int64_t M,
                                    int64_t N, int64_t K, void *c, bool out_bf16, hipStream_t s);
// NVFP4 quantize of x [rows, cols] (tensor amax pass, then the encode)
// written in the packed NVFP4 layout; workspace holds the amax partials.
hipError_t launch_nv_quantize_packed(const void *x, bool bf16, int64_t rows, int64_t cols,
                                     uint8_t *packed, float *global_scale, void *workspace,
                                     int32_t *status, hipStream_t s);
// MXFP4 quantize (floor rule) of x [rows, cols] written in the packed layout.
hipError_t launch_mx_quantize_packed(const void *x, bool bf16, int64_t rows, int64_t cols,
                                     uint8_t *packed, int32_t *status, hipStream_t s);
// Split-K MXFP4 GEMM: S equal K ranges (gemm_splitk_parts; 0 when the shape
// is not supported), fp32 partials in workspace [S][M][N], then a reduction
// in increasing split order.
int gemm_splitk_parts(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_mxfp4_splitk(const uint8_t *a_codes, const uint8_t *a_scales,
                                    const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t M,
                                    int64_t N, int64_t K, void *c, bool out_bf16, float *workspace,
                                    hipStream_t s);
// NVFP4 x NVFP4: C = (s_gA s_gB) * sum over 16-blocks of the E4M3 scale
// products times the FP4 dot products.
hipError_t launch_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *sg_a,
                             const uint8_t *bt_codes, const uint8_t *bt_scales, const float *sg_b,
                             int64_t M, int64_t N, int64_t K, void *c, bool out_bf16,
                             hipStream_t s);
// Activations x [M, K] quantized to MXFP4 into a_codes / a_scales, then the
// GEMM with Bt; with one_launch, one kernel (grid barrier, workspace as for
// NVFP4) when the grid fits on the device at once, else two launches.
hipError_t launch_linear_mxfp4(const void *x, bool x_bf16, const uint8_t *bt_codes,
                               const uint8_t *bt_scales, int64_t M, int64_t N, int64_t K,
                               uint8_t *a_codes, uint8_t *a_scales, void *c, bool out_bf16,
                               bool one_launch, void *workspace, int32_t *status, hipStream_t s,
                               uint32_t spin_limit = kResidentSpinLimit);

}  // namespace fp4dev
