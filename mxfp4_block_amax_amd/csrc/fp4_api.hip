// fp4_api.hip - the extern "C" entry points of libfp4.so (declared in
// include/fp4.h): argument validation on the host, then kernel launches on
// the caller's stream.  Every argument error is returned before any HIP call.
#include <stdint.h>

#include <mutex>

#include "../../include/fp4.h"
#ifdef FP4_PHASE_CLOCK
#include "../../include/fp4_phase_clock.h"
#endif
#include "fp4_kernels.h"

// Device scratch of fp4_quantize_nvfp4_noalloc, for callers that cannot
// allocate: the same workspace fp4_quantize_nvfp4 takes from its caller
// (tensor-amax partials, then the grid barrier's epoch word and slots), one
// copy per GPU, held until the process ends.  Its size does not depend on
// the tensor.  In host code the name stands for a host-side shadow, never a
// device address: host code uses the address hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[fp4dev::kNoAllocScratchBytes];
static_assert(FP4_NOALLOC_SCRATCH_BYTES == fp4dev::kNoAllocScratchBytes,
              "the header states the scratch size");
static_assert(fp4dev::kNvWorkspaceBytes <= fp4dev::kNoAllocScratchBytes,
              "the scratch holds one NVFP4 workspace");
static_assert(FP4_BARRIER_SPIN_LIMIT_DEFAULT == fp4dev::kResidentSpinLimit,
              "the header states the grid barrier's default poll limit");

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool valid_dtype(fp4_dtype t) { return t == FP4_F32 || t == FP4_BF16; }

fp4_status check_shape(int64_t rows, int64_t cols, int32_t block) {
    if (rows < 1 || cols < 1) return FP4_E_SHAPE;
    if (cols % block) return FP4_E_SHAPE;          // incomplete block / odd length
    if (rows > kMaxElems / cols) return FP4_E_SHAPE;
    return FP4_OK;
}

fp4_status from_hip(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_E_HIP; }

// The NVFP4 and scale-search tensor-amax pass needs this many bytes.
size_t nv_workspace() { return fp4dev::kNvWorkspaceBytes; }

// Per-device address of `scratch`, looked up and zero-filled once per device
// (with that device current) on the first no-allocation call there.  The
// fill is synchronous and waited for on the null stream, so it is complete
// before any kernel on any stream can use the scratch.
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[fp4dev::kMaxDevices];

hipError_t device_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= fp4dev::kMaxDevices) return hipErrorInvalidDevice;
    ScratchSlot &s = g_scratch[dev];
    std::call_once(s.once, [&s] {
        void *p = nullptr;
        hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r == hipSuccess) r = hipMemset(p, 0, fp4dev::kNoAllocScratchBytes);
        if (r == hipSuccess) r = hipStreamSynchronize(nullptr);
        s.ptr = r == hipSuccess ? p : nullptr;
        s.err = r;
    });
    *out = s.ptr;
    return s.err;
}

}  // namespace

extern "C" {

fp4_status fp4_quantize_mxfp4(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                              int32_t block, uint8_t *codes, uint8_t *scales,
                              int32_t *status, void *stream) {
    if (!x || !codes || !scales) return FP4_E_ARG;
    if (block != 32) return FP4_E_ARG;
    if (!valid_dtype(xt)) return FP4_E_DTYPE;
    fp4_status st = check_shape(rows, cols, block);
    if (st != FP4_OK) return st;
    if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(status, 4)) return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_mx_quantize(x, xt == FP4_BF16, rows * cols, 0, codes, scales,
                                               status, (hipStream_t)stream));
}

fp4_status fp4_quantize_mxfp4_rule(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                   int32_t block, fp4_mx_rule rule, uint8_t *codes,
                                   uint8_t *scales, int32_t *status, void *stream) {
    if (!x || !codes || !scales) return FP4_E_ARG;
    if (block != 32) return FP4_E_ARG;
    if (rule != FP4_MX_RULE_OCP && rule != FP4_MX_RULE_CEIL && rule != FP4_MX_RULE_MSE)
        return FP4_E_ARG;
    if (!valid_dtype(xt)) return FP4_E_DTYPE;
    fp4_status st = check_shape(rows, cols, block);
    if (st != FP4_OK) return st;
    if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(status, 4)) return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_mx_quantize(x, xt == FP4_BF16, rows * cols, (int)rule, codes,
                                               scales, status, (hipStream_t)stream));
}

// fp4_quantize_nvfp4 with the grid barrier's poll limit as an argument
static fp4_status quantize_nvfp4(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                 int32_t block, uint8_t *codes, uint8_t *scales,
                                 float *global_scale, void *workspace, size_t workspace_bytes,
                                 int32_t *status, void *stream, uint32_t spin_limit) {
    if (!x || !codes || !scales || !global_scale) return FP4_E_ARG;
    if (block != 16) return FP4_E_ARG;
    if (!valid_dtype(xt)) return FP4_E_DTYPE;
    fp4_status st = check_shape(rows, cols, block);
    if (st != FP4_OK) return st;
    if (!workspace || workspace_bytes < nv_workspace()) return FP4_E_WORKSPACE;
    if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(global_scale, 4) ||
        !aligned(workspace, 16) || !aligned(status, 4))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_nv_quantize(x, xt == FP4_BF16, rows * cols, codes, scales,
                                               global_scale, workspace, status,
                                               (hipStream_t)stream, spin_limit));
}

fp4_status fp4_quantize_nvfp4(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                              int32_t block, uint8_t *codes, uint8_t *scales,
                              float *global_scale, void *workspace, size_t workspace_bytes,
                              int32_t *status, void *stream) {
    return quantize_nvfp4(x, xt, rows, cols, block, codes, scales, global_scale, workspace,
                          workspace_bytes, status, stream, fp4dev::kResidentSpinLimit);
}

fp4_status fp4_debug_quantize_nvfp4_spin(const void *x, fp4_dtype xt, int64_t rows,
                                         int64_t cols, int32_t block, uint8_t *codes,
                                         uint8_t *scales, float *global_scale, void *workspace,
                                         size_t workspace_bytes, int32_t *status, void *stream,
                                         uint32_t spin_limit) {
    return quantize_nvfp4(x, xt, rows, cols, block, codes, scales, global_scale, workspace,
                          workspace_bytes, status, stream, spin_limit);
}

fp4_status fp4_quantize_nvfp4_noalloc(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                      int32_t block, uint8_t *codes, uint8_t *scales,
                                      float *global_scale, int32_t *status, void *stream) {
    if (!x || !codes || !scales || !global_scale) return FP4_E_ARG;
    if (block != 16) return FP4_E_ARG;
    if (!valid_dtype(xt)) return FP4_E_DTYPE;
    fp4_status st = check_shape(rows, cols, block);
    if (st != FP4_OK) return st;
    // the scratch holds the whole workspace of any accepted shape; the check
    // keeps that true if the workspace ever grows with the shape
    if (fp4_workspace_bytes(FP4_NVFP4, rows, cols) > fp4dev::kNoAllocScratchBytes)
        return FP4_E_WORKSPACE;
    if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(global_scale, 4) || !aligned(status, 4))
        return FP4_E_ALIGN;
    void *ws = nullptr;
    hipError_t e = device_scratch(&ws);
    if (e != hipSuccess) return FP4_E_HIP;
    return from_hip(fp4dev::launch_nv_quantize(x, xt == FP4_BF16, rows * cols, codes, scales,
                                               global_scale, ws, status, (hipStream_t)stream));
}

fp4_status fp4_quantize_sr(fp4_format fmt, const void *x, fp4_dtype xt, int64_t rows,
                           int64_t cols, int32_t block, uint64_t seed, uint8_t *codes,
                           uint8_t *scales, float *global_scale, void *workspace,
                           size_t workspace_bytes, int32_t *status, void *stream) {
    if (fmt != FP4_MXFP4 && fmt != FP4_NVFP4) return FP4_E_DTYPE;
    if (!valid_dtype(xt)) return FP4_E_DTYPE;
    if (!x || !codes || !scales) return FP4_E_ARG;
    if (fmt == FP4_NVFP4 && !global_scale) return FP4_E_ARG;
    if (block != (fmt == FP4_MXFP4 ? 32 : 16)) return FP4_E_ARG;
    fp4_status st = check_shape(rows, cols, block);
    if (st != FP4_OK) return st;
    if (fmt == FP4_NVFP4 && (!workspace || workspace_bytes < nv_workspace()))
        return FP4_E_WORKSPACE;
    if (!aligned(x, 16) || !aligned(codes, 4) || !aligned(status, 4)) return FP4_E_ALIGN;
    if (fmt == FP4_NVFP4 && (!aligned(global_scale, 4) || !aligned(workspace, 16)))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_quantize_sr((int)fmt, x, xt == FP4_BF16, rows * cols, seed,
                                               codes, scales, global_scale, workspace, status,
                                               (hipStream_t)stream));
}

fp4_status fp4_dequantize(fp4_format fmt, const uint8_t *codes, const uint8_t *scales,
                          const float *global_scale, int64_t rows, int64_t cols,
                          int32_t block, void *y, fp4_dtype yt, void *stream) {
    if (fmt != FP4_MXFP4 && fmt != FP4_NVFP4) return FP4_E_DTYPE;
    if (!valid_dtype(yt)) return FP4_E_DTYPE;
    if (!codes || !scales || !y) return FP4_E_ARG;
    if (fmt == FP4_NVFP4 && !global_scale) return FP4_E_ARG;
    if (block != (fmt == FP4_MXFP4 ? 32 : 16)) return FP4_E_ARG;
    fp4_status st = check_shape(rows, cols, block);
    if (st != FP4_OK) return st;
    if (!aligned(codes, 4) || !aligned(y, 16) || !aligned(global_scale, 4)) return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_dequantize((int)fmt, codes, scales, global_scale,
                                              rows * cols, y, yt == FP4_BF16,
                                              (hipStream_t)stream));
}

fp4_status fp4_scale_search(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                            int32_t block, int32_t n_candidates, float c_lo, float c_hi,
                            uint8_t *codes, uint8_t *scales, float *global_scale,
                            void *workspace, size_t workspace_bytes, int32_t *status,
                            void *stream) {
    if (!x || !codes || !scales || !global_scale) return FP4_E_ARG;
    if (block != 16) return FP4_E_ARG;
    // candidate grid: c_k = linspace(c_lo, c_hi, n); it must be finer than the
    // E4M3 grid so that the distinct encoded candidates are consecutive codes
    if (n_candidates < 2) return FP4_E_ARG;
    if (!(c_lo > 0.0f) || !(c_hi >= c_lo) || !(c_hi <= 4.0f)) return FP4_E_ARG;
    // an E4M3 rounding interval is at least 1/15 of its code's value wide, so a
    // candidate step below c_lo / 24 of the block's t cannot jump over a code
    if ((double)(c_hi - c_lo) / (double)(n_candidates - 1) > (double)c_lo / 24.0) return FP4_E_ARG;
    if (!valid_dtype(xt)) return FP4_E_DTYPE;
    fp4_status st = check_shape(rows, cols, block);
    if (st != FP4_OK) return st;
    if (!workspace || workspace_bytes < nv_workspace()) return FP4_E_WORKSPACE;
    // a block's 16 codes are stored as one 8-byte word
    if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(global_scale, 4) ||
        !aligned(workspace, 16) || !aligned(status, 4))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_scale_search(x, xt == FP4_BF16, rows * cols, false, c_lo,
                                                c_hi, codes, scales, global_scale, workspace,
                                                status, (hipStream_t)stream));
}

fp4_status fp4_scale_search_exhaustive(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                       int32_t block, uint8_t *codes, uint8_t *scales,
                                       float *global_scale, void *workspace,
                                       size_t workspace_bytes, int32_t *status, void *stream) {
    if (!x || !codes || !scales || !global_scale) return FP4_E_ARG;
    if (block != 16) return FP4_E_ARG;
    if (!valid_dtype(xt)) return FP4_E_DTYPE;
    fp4_status st = check_shape(rows, cols, block);
    if (st != FP4_OK) return st;
    if (!workspace || workspace_bytes < nv_workspace()) return FP4_E_WORKSPACE;
    // a block's 16 codes are stored as one 8-byte word
    if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(global_scale, 4) ||
        !aligned(workspace, 16) || !aligned(status, 4))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_scale_search(x, xt == FP4_BF16, rows * cols, true, 0.0f, 0.0f,
                                                codes, scales, global_scale, workspace, status,
                                                (hipStream_t)stream));
}

fp4_status fp4_gemm_mxfp4(const uint8_t *a_codes, const uint8_t *a_scales,
                          const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t M,
                          int64_t N, int64_t K, void *c, fp4_dtype ct, void *stream) {
    if (!a_codes || !a_scales || !bt_codes || !bt_scales || !c) return FP4_E_ARG;
    if (!valid_dtype(ct)) return FP4_E_DTYPE;
    if (M < 1 || N < 1 || K < 32 || K % 32) return FP4_E_SHAPE;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return FP4_E_SHAPE;
    if (!aligned(a_codes, 16) || !aligned(bt_codes, 16) || !aligned(c, 4)) return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_gemm_mxfp4(a_codes, a_scales, bt_codes, bt_scales, M, N, K,
                                              c, ct == FP4_BF16, (hipStream_t)stream));
}

int64_t fp4_packed_operand_bytes(int64_t rows, int64_t K) {
    if (rows > INT32_MAX / 2 || K > INT32_MAX / 2) return 0;
    return fp4dev::packed_operand_bytes(rows, K);
}

fp4_status fp4_pack_mxfp4_operand(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                  int64_t K, uint8_t *packed, size_t packed_bytes, void *stream) {
    if (!codes || !scales || !packed) return FP4_E_ARG;
    const int64_t need = fp4_packed_operand_bytes(rows, K);
    if (need == 0) return FP4_E_SHAPE;
    if (packed_bytes < (size_t)need) return FP4_E_WORKSPACE;
    if (!aligned(codes, 16) || !aligned(packed, 16)) return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_pack_mxfp4(codes, scales, rows, K, packed, (hipStream_t)stream));
}

fp4_status fp4_gemm_mxfp4_packed(const uint8_t *a_packed, const uint8_t *bt_packed, int64_t M,
                                 int64_t N, int64_t K, void *c, fp4_dtype ct, void *stream) {
    if (!a_packed || !bt_packed || !c) return FP4_E_ARG;
    if (!valid_dtype(ct)) return FP4_E_DTYPE;
    if (M < 1 || N < 1 || K < 2048 || K % 2048 != 0 || K > 16384) return FP4_E_SHAPE;
    if (fp4_packed_operand_bytes(M, K) > (1 << 30) || fp4_packed_operand_bytes(N, K) > (1 << 30)) return FP4_E_SHAPE;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return FP4_E_SHAPE;
    if (!aligned(a_packed, 16) || !aligned(bt_packed, 16) || !aligned(c, 4)) return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_gemm_mxfp4_packed(a_packed, bt_packed, M, N, K, c,
                                                     ct == FP4_BF16, (hipStream_t)stream));
}

int64_t fp4_nv_packed_operand_bytes(int64_t rows, int64_t K) {
    if (rows > INT32_MAX / 2 || K > INT32_MAX / 2) return 0;
    return fp4dev::nv_packed_operand_bytes(rows, K);
}

fp4_status fp4_pack_nvfp4_operand(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                  int64_t K, uint8_t *packed, size_t packed_bytes, void *stream) {
    if (!codes || !scales || !packed) return FP4_E_ARG;
    const int64_t need = fp4_nv_packed_operand_bytes(rows, K);
    if (need == 0) return FP4_E_SHAPE;
    if (packed_bytes < (size_t)need) return FP4_E_WORKSPACE;
    if (!aligned(codes, 16) || !aligned(packed, 16)) return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_pack_nvfp4(codes, scales, rows, K, packed, (hipStream_t)stream));
}

fp4_status fp4_gemm_nvfp4_packed(const uint8_t *a_packed, const float *a_global_scale,
                                 const uint8_t *bt_packed, const float *bt_global_scale,
                                 int64_t M, int64_t N, int64_t K, void *c, fp4_dtype ct,
                                 void *stream) {
    if (!a_packed || !a_global_scale || !bt_packed || !bt_global_scale || !c) return FP4_E_ARG;
    if (!valid_dtype(ct)) return FP4_E_DTYPE;
    if (M < 1 || N < 1 || K < 2048 || K % 2048 != 0 || K > 16384) return FP4_E_SHAPE;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2) return FP4_E_SHAPE;
    if (fp4_nv_packed_operand_bytes(M, K) > (1 << 30) ||
        fp4_nv_packed_operand_bytes(N, K) > (1 << 30))
        return FP4_E_SHAPE;
    if (!aligned(a_packed, 16) || !aligned(bt_packed, 16) || !aligned(c, 4) ||
        !aligned(a_global_scale, 4) || !aligned(bt_global_scale, 4))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_gemm_nvfp4_packed(a_packed, a_global_scale, bt_packed,
                                                     bt_global_scale, M, N, K, c, ct == FP4_BF16,
                                                     (hipStream_t)stream));
}

fp4_status fp4_quantize_nvfp4_packed(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                     uint8_t *packed, size_t packed_bytes, float *global_scale,
                                     void *workspace, size_t workspace_bytes, int32_t *status,
                                     void *stream) {
    if (!x || !packed || !global_scale) return FP4_E_ARG;
    if (!valid_dtype(xt)) return FP4_E_DTYPE;
    const int64_t need = fp4_nv_packed_operand_bytes(rows, cols);
    if (need == 0 || rows > kMaxElems / cols) return FP4_E_SHAPE;
    if (packed_bytes < (size_t)need) return FP4_E_WORKSPACE;
    if (!workspace || workspace_bytes < nv_workspace()) return FP4_E_WORKSPACE;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(global_scale, 4) ||
        !aligned(workspace, 16) || !aligned(status, 4))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_nv_quantize_packed(x, xt == FP4_BF16, rows, cols, packed,
                                                      global_scale, workspace, status,
                                                      (hipStream_t)stream));
}

fp4_status fp4_linear_nvfp4_packed(const void *x, fp4_dtype xt, int64_t M, int64_t K,
                                   const uint8_t *bt_packed, const float *bt_global_scale,
                                   int64_t N, uint8_t *a_packed, size_t a_packed_bytes,
                                   float *a_global_scale, void *c, fp4_dtype ct,
                                   void *workspace, size_t workspace_bytes, int32_t *status,
                                   void *stream) {
    if (!x || !bt_packed || !bt_global_scale || !a_packed || !a_global_scale || !c)
        return FP4_E_ARG;
    if (!valid_dtype(xt) || !valid_dtype(ct)) return FP4_E_DTYPE;
    if (M < 1 || N < 1 || K < 2048 || K % 2048 != 0 || K > 16384) return FP4_E_SHAPE;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || M > kMaxElems / K) return FP4_E_SHAPE;
    if (fp4_nv_packed_operand_bytes(M, K) > (1 << 30) ||
        fp4_nv_packed_operand_bytes(N, K) > (1 << 30))
        return FP4_E_SHAPE;
    if (a_packed_bytes < (size_t)fp4_nv_packed_operand_bytes(M, K)) return FP4_E_WORKSPACE;
    if (!workspace || workspace_bytes < nv_workspace()) return FP4_E_WORKSPACE;
    if (!aligned(x, 16) || !aligned(bt_packed, 16) || !aligned(a_packed, 16) || !aligned(c, 4) ||
        !aligned(bt_global_scale, 4) || !aligned(a_global_scale, 4) ||
        !aligned(workspace, 16) || !aligned(status, 4))
        return FP4_E_ALIGN;
    hipError_t e = fp4dev::launch_nv_quantize_packed(x, xt == FP4_BF16, M, K, a_packed,
                                                     a_global_scale, workspace, status,
                                                     (hipStream_t)stream);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(fp4dev::launch_gemm_nvfp4_packed(a_packed, a_global_scale, bt_packed,
                                                     bt_global_scale, M, N, K, c,
                                                     ct == FP4_BF16, (hipStream_t)stream));
}

fp4_status fp4_quantize_mxfp4_packed(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                     uint8_t *packed, size_t packed_bytes, int32_t *status,
                                     void *stream) {
    if (!x || !packed) return FP4_E_ARG;
    if (!valid_dtype(xt)) return FP4_E_DTYPE;
    const int64_t need = fp4_packed_operand_bytes(rows, cols);
    if (need == 0) return FP4_E_SHAPE;
    if (packed_bytes < (size_t)need) return FP4_E_WORKSPACE;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(status, 4)) return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_mx_quantize_packed(x, xt == FP4_BF16, rows, cols, packed, status,
                                                      (hipStream_t)stream));
}

fp4_status fp4_linear_mxfp4_packed(const void *x, fp4_dtype xt, int64_t M, int64_t K,
                                   const uint8_t *bt_packed, int64_t N, uint8_t *a_packed,
                                   size_t a_packed_bytes, void *c, fp4_dtype ct, int32_t *status,
                                   void *stream) {
    if (!x || !bt_packed || !a_packed || !c) return FP4_E_ARG;
    if (!valid_dtype(xt) || !valid_dtype(ct)) return FP4_E_DTYPE;
    if (M < 1 || N < 1 || K < 2048 || K % 2048 != 0 || K > 16384) return FP4_E_SHAPE;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2) return FP4_E_SHAPE;
    if (fp4_packed_operand_bytes(M, K) > (1 << 30) || fp4_packed_operand_bytes(N, K) > (1 << 30))
        return FP4_E_SHAPE;
    if (a_packed_bytes < (size_t)fp4_packed_operand_bytes(M, K)) return FP4_E_WORKSPACE;
    if (!aligned(x, 16) || !aligned(bt_packed, 16) || !aligned(a_packed, 16) || !aligned(c, 4) ||
        !aligned(status, 4))
        return FP4_E_ALIGN;
    hipError_t e = fp4dev::launch_mx_quantize_packed(x, xt == FP4_BF16, M, K, a_packed, status,
                                                     (hipStream_t)stream);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(fp4dev::launch_gemm_mxfp4_packed(a_packed, bt_packed, M, N, K, c,
                                                     ct == FP4_BF16, (hipStream_t)stream));
}

size_t fp4_gemm_splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return 0;
    const int S = fp4dev::gemm_splitk_parts(M, N, K);
    if (S < 1) return 0;
    // S partial products of M x N fp32; a size past size_t is no shape at all
    size_t bytes = 0;
    if (__builtin_mul_overflow((size_t)S * sizeof(float), (size_t)M, &bytes) ||
        __builtin_mul_overflow(bytes, (size_t)N, &bytes))
        return 0;
    return bytes;
}

fp4_status fp4_gemm_mxfp4_splitk(const uint8_t *a_codes, const uint8_t *a_scales,
                                 const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t M,
                                 int64_t N, int64_t K, void *c, fp4_dtype ct, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    if (!a_codes || !a_scales || !bt_codes || !bt_scales || !c) return FP4_E_ARG;
    if (!valid_dtype(ct)) return FP4_E_DTYPE;
    const size_t need = fp4_gemm_splitk_workspace_bytes(M, N, K);
    if (need == 0) return FP4_E_SHAPE;
    if (!workspace || workspace_bytes < need) return FP4_E_WORKSPACE;
    if (!aligned(a_codes, 16) || !aligned(bt_codes, 16) || !aligned(a_scales, 16) ||
        !aligned(bt_scales, 16) || !aligned(workspace, 16) ||
        !aligned(c, ct == FP4_BF16 ? 8 : 16))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_gemm_mxfp4_splitk(a_codes, a_scales, bt_codes, bt_scales, M, N,
                                                     K, c, ct == FP4_BF16, (float *)workspace,
                                                     (hipStream_t)stream));
}

fp4_status fp4_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales,
                          const float *a_global_scale, const uint8_t *bt_codes,
                          const uint8_t *bt_scales, const float *bt_global_scale, int64_t M,
                          int64_t N, int64_t K, void *c, fp4_dtype ct, void *stream) {
    if (!a_codes || !a_scales || !a_global_scale || !bt_codes || !bt_scales ||
        !bt_global_scale || !c)
        return FP4_E_ARG;
    if (!valid_dtype(ct)) return FP4_E_DTYPE;
    if (M < 1 || N < 1 || K < 16 || K % 16) return FP4_E_SHAPE;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return FP4_E_SHAPE;
    if (!aligned(c, 4) || !aligned(a_global_scale, 4) || !aligned(bt_global_scale, 4))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_gemm_nvfp4(a_codes, a_scales, a_global_scale, bt_codes,
                                              bt_scales, bt_global_scale, M, N, K, c,
                                              ct == FP4_BF16, (hipStream_t)stream));
}

// fp4_linear_mxfp4 with the grid barrier's poll limit as an argument
static fp4_status linear_mxfp4(const void *x, fp4_dtype xt, int64_t M, int64_t K,
                               const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t N,
                               uint8_t *a_codes, uint8_t *a_scales, void *c, fp4_dtype ct,
                               fp4_linear_mode mode, void *workspace, size_t workspace_bytes,
                               int32_t *status, void *stream, uint32_t spin_limit) {
    if (!x || !bt_codes || !bt_scales || !a_codes || !a_scales || !c) return FP4_E_ARG;
    if (mode != FP4_LINEAR_ONE_LAUNCH && mode != FP4_LINEAR_TWO_LAUNCHES) return FP4_E_ARG;
    if (!valid_dtype(xt) || !valid_dtype(ct)) return FP4_E_DTYPE;
    if (M < 1 || N < 1 || K < 32 || K % 32) return FP4_E_SHAPE;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return FP4_E_SHAPE;
    if (M > kMaxElems / K) return FP4_E_SHAPE;
    if (!workspace || workspace_bytes < nv_workspace()) return FP4_E_WORKSPACE;
    if (!aligned(x, 16) || !aligned(a_codes, 16) || !aligned(bt_codes, 16) || !aligned(c, 4) ||
        !aligned(workspace, 16) || !aligned(status, 4))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_linear_mxfp4(x, xt == FP4_BF16, bt_codes, bt_scales, M, N, K,
                                                a_codes, a_scales, c, ct == FP4_BF16,
                                                mode == FP4_LINEAR_ONE_LAUNCH, workspace, status,
                                                (hipStream_t)stream, spin_limit));
}

fp4_status fp4_linear_mxfp4(const void *x, fp4_dtype xt, int64_t M, int64_t K,
                            const uint8_t *bt_codes, const uint8_t *bt_scales, int64_t N,
                            uint8_t *a_codes, uint8_t *a_scales, void *c, fp4_dtype ct,
                            fp4_linear_mode mode, void *workspace, size_t workspace_bytes,
                            int32_t *status, void *stream) {
    return linear_mxfp4(x, xt, M, K, bt_codes, bt_scales, N, a_codes, a_scales, c, ct, mode,
                        workspace, workspace_bytes, status, stream, fp4dev::kResidentSpinLimit);
}

fp4_status fp4_debug_linear_mxfp4_spin(const void *x, fp4_dtype xt, int64_t M, int64_t K,
                                       const uint8_t *bt_codes, const uint8_t *bt_scales,
                                       int64_t N, uint8_t *a_codes, uint8_t *a_scales, void *c,
                                       fp4_dtype ct, fp4_linear_mode mode, void *workspace,
                                       size_t workspace_bytes, int32_t *status, void *stream,
                                       uint32_t spin_limit) {
    return linear_mxfp4(x, xt, M, K, bt_codes, bt_scales, N, a_codes, a_scales, c, ct, mode,
                        workspace, workspace_bytes, status, stream, spin_limit);
}

fp4_status fp4_quantize_padded(fp4_format fmt, const void *x, fp4_dtype xt, int64_t rows,
                               int64_t cols, uint8_t *codes, uint8_t *scales,
                               float *global_scale, void *workspace, size_t workspace_bytes,
                               int32_t *status, void *stream) {
    if (fmt != FP4_MXFP4 && fmt != FP4_NVFP4) return FP4_E_DTYPE;
    if (!valid_dtype(xt)) return FP4_E_DTYPE;
    if (!x || !codes || !scales) return FP4_E_ARG;
    if (fmt == FP4_NVFP4 && !global_scale) return FP4_E_ARG;
    const int64_t block = fmt == FP4_MXFP4 ? 32 : 16;
    if (rows < 1 || cols < 1 || cols > kMaxElems) return FP4_E_SHAPE;
    const int64_t pcols = (cols + block - 1) / block * block;
    if (rows > kMaxElems / pcols) return FP4_E_SHAPE;
    if (fmt == FP4_NVFP4 && (!workspace || workspace_bytes < nv_workspace())) return FP4_E_WORKSPACE;
    if (!aligned(x, xt == FP4_BF16 ? 2 : 4) || !aligned(codes, 4) || !aligned(status, 4) ||
        !aligned(global_scale, 4) || !aligned(workspace, 16))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_quantize_padded((int)fmt, x, xt == FP4_BF16, rows, cols, codes,
                                                   scales, global_scale, workspace, status,
                                                   (hipStream_t)stream));
}

fp4_status fp4_dequantize_padded(fp4_format fmt, const uint8_t *codes, const uint8_t *scales,
                                 const float *global_scale, int64_t rows, int64_t cols, void *y,
                                 fp4_dtype yt, void *stream) {
    if (fmt != FP4_MXFP4 && fmt != FP4_NVFP4) return FP4_E_DTYPE;
    if (!valid_dtype(yt)) return FP4_E_DTYPE;
    if (!codes || !scales || !y) return FP4_E_ARG;
    if (fmt == FP4_NVFP4 && !global_scale) return FP4_E_ARG;
    const int64_t block = fmt == FP4_MXFP4 ? 32 : 16;
    if (rows < 1 || cols < 1 || cols > kMaxElems) return FP4_E_SHAPE;
    if (rows > kMaxElems / ((cols + block - 1) / block * block)) return FP4_E_SHAPE;
    if (!aligned(codes, 4) || !aligned(y, yt == FP4_BF16 ? 2 : 4) || !aligned(global_scale, 4))
        return FP4_E_ALIGN;
    return from_hip(fp4dev::launch_dequantize_padded((int)fmt, codes, scales, global_scale, rows,
                                                     cols, y, yt == FP4_BF16,
                                                     (hipStream_t)stream));
}

int64_t fp4_padded_storage_bytes(fp4_format fmt, int64_t rows, int64_t cols) {
    if ((fmt != FP4_MXFP4 && fmt != FP4_NVFP4) || rows < 1 || cols < 1) return -1;
    const int64_t block = fmt == FP4_MXFP4 ? 32 : 16;
    // the shapes fp4_quantize_padded accepts; the products below then fit
    if (cols > kMaxElems || rows > kMaxElems / ((cols + block - 1) / block * block)) return -1;
    const int64_t blocks = rows * ((cols + block - 1) / block);
    return blocks * (block / 2 + 1) + (fmt == FP4_NVFP4 ? 4 : 0);
}

#ifdef FP4_PHASE_CLOCK
fp4_status fp4_debug_phase_clock(uint64_t *host, size_t n) {
    if (!host) return FP4_E_ARG;
    return from_hip(fp4dev::read_phase_clock(host, n));
}
#endif

size_t fp4_workspace_bytes(fp4_format fmt, int64_t rows, int64_t cols) {
    (void)rows;
    (void)cols;
    return fmt == FP4_NVFP4 ? nv_workspace() : 0;
}

const char *fp4_status_str(fp4_status s) {
    switch (s) {
        case FP4_OK: return "ok";
        case FP4_E_ARG: return "invalid argument (null pointer, block size or candidate grid)";
        case FP4_E_SHAPE: return "invalid shape (rows/cols < 1 or cols not a multiple of the block)";
        case FP4_E_DTYPE: return "invalid dtype or format";
        case FP4_E_ALIGN: return "misaligned pointer";
        case FP4_E_WORKSPACE: return "workspace missing or too small";
        case FP4_E_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

}  // extern "C"
