// capi_check.cpp - drives the host side of libfp4's C ABI (include/fp4.h)
// for a build whose host code runs under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Test infrastructure: built and run by
// tests/test_sanitize_host.py, on a machine with or without a GPU.
//
// Every compute call made here is one the header says fails validation, so
// it returns before any HIP call and no device memory is touched: the
// pointers are fake, never-dereferenced addresses.  The sizes run over the
// values that break naive size arithmetic (0, negatives, INT32 and INT64
// extremes, products past 2^63), and the size helpers are checked to
// return either their documented "invalid" value or a size that covers
// the plain product.  Exit status 0 means every call returned what the
// header states and the sanitizers reported nothing.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "../../include/fp4.h"

namespace {

int failures = 0;
long calls = 0;

#define EXPECT(call, want)                                                             \
    do {                                                                               \
        ++calls;                                                                       \
        const int got_ = (int)(call);                                                  \
        if (got_ != (int)(want)) {                                                     \
            std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, \
                         got_, (int)(want));                                           \
            ++failures;                                                                \
        }                                                                              \
    } while (0)

#define EXPECT_ERR(call)                                                            \
    do {                                                                            \
        ++calls;                                                                    \
        const int got_ = (int)(call);                                               \
        if (got_ == FP4_OK || got_ == FP4_E_HIP) {                                  \
            std::fprintf(stderr, "line %d: %s returned %d, expected an argument error\n", \
                         __LINE__, #call, got_);                                    \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

void *const A16 = reinterpret_cast<void *>(uintptr_t{0x10000});
void *const A1 = reinterpret_cast<void *>(uintptr_t{0x10001});
uint8_t *const U16 = static_cast<uint8_t *>(A16);
float *const F16 = static_cast<float *>(A16);
const fp4_dtype BF = FP4_BF16;
const size_t WS = size_t{1} << 20;

constexpr int64_t I64MAX = std::numeric_limits<int64_t>::max();
constexpr int64_t I64MIN = std::numeric_limits<int64_t>::min();
const int64_t kSizes[] = {I64MIN, -4096, -32, -1, 0, 1, 15, 17, 31, 33,
                          (int64_t)INT32_MAX, (int64_t)INT32_MAX + 1, (int64_t)1 << 40,
                          ((int64_t)1 << 40) + 32, I64MAX - 31, I64MAX};

bool positive_multiple(int64_t v, int64_t m) { return v >= m && v % m == 0; }

// Quantize-like entry points over every (rows, cols) pair that validation
// must reject as a shape (or, for sizes that are legal, skip).
void quantize_shapes() {
    for (int64_t r : kSizes)
        for (int64_t c : kSizes) {
            const bool rows_ok = r >= 1, cols32 = positive_multiple(c, 32),
                       cols16 = positive_multiple(c, 16);
            // products beyond 2^40 elements are rejected as shapes too
            const bool fits = rows_ok && c >= 1 && r <= (((int64_t)1 << 40) / c);
            if (!(rows_ok && cols32 && fits)) {
                EXPECT(fp4_quantize_mxfp4(A16, BF, r, c, 32, U16, U16, nullptr, nullptr),
                       FP4_E_SHAPE);
                EXPECT(fp4_quantize_mxfp4_rule(A16, BF, r, c, 32, FP4_MX_RULE_MSE, U16, U16,
                                               nullptr, nullptr),
                       FP4_E_SHAPE);
                EXPECT(fp4_quantize_sr(FP4_MXFP4, A16, BF, r, c, 32, 7, U16, U16, nullptr, A16,
                                       WS, nullptr, nullptr),
                       FP4_E_SHAPE);
            }
            if (!(rows_ok && cols16 && fits)) {
                EXPECT(fp4_quantize_nvfp4(A16, BF, r, c, 16, U16, U16, F16, A16, WS, nullptr,
                                          nullptr),
                       FP4_E_SHAPE);
                EXPECT(fp4_quantize_nvfp4_noalloc(A16, BF, r, c, 16, U16, U16, F16, nullptr,
                                                  nullptr),
                       FP4_E_SHAPE);
                EXPECT(fp4_scale_search(A16, BF, r, c, 16, 64, 0.5f, 1.5f, U16, U16, F16, A16, WS,
                                        nullptr, nullptr),
                       FP4_E_SHAPE);
                EXPECT(fp4_scale_search_exhaustive(A16, BF, r, c, 16, U16, U16, F16, A16, WS,
                                                   nullptr, nullptr),
                       FP4_E_SHAPE);
                EXPECT(fp4_dequantize(FP4_NVFP4, U16, U16, F16, r, c, 16, A16, BF, nullptr),
                       FP4_E_SHAPE);
            }
            // padded layouts accept any cols >= 1; reject the rest
            if (!(rows_ok && c >= 1 && c <= ((int64_t)1 << 40) &&
                  r <= ((int64_t)1 << 40) / ((c + 31) / 32 * 32))) {
                EXPECT_ERR(fp4_quantize_padded(FP4_MXFP4, A16, BF, r, c, U16, U16, nullptr,
                                               nullptr, 0, nullptr, nullptr));
                EXPECT_ERR(fp4_dequantize_padded(FP4_MXFP4, U16, U16, nullptr, r, c, A16, BF,
                                                 nullptr));
            }
            // the packed quantizers need K a multiple of 512
            if (!(rows_ok && positive_multiple(c, 512) && r <= INT32_MAX / 2 &&
                  c <= INT32_MAX / 2)) {
                EXPECT_ERR(fp4_quantize_mxfp4_packed(A16, BF, r, c, U16, WS, nullptr, nullptr));
                EXPECT_ERR(fp4_quantize_nvfp4_packed(A16, BF, r, c, U16, WS, F16, A16, WS,
                                                     nullptr, nullptr));
                EXPECT_ERR(fp4_pack_mxfp4_operand(U16, U16, r, c, U16, WS, nullptr));
                EXPECT_ERR(fp4_pack_nvfp4_operand(U16, U16, r, c, U16, WS, nullptr));
            }
        }
}

// GEMM-like entry points over every (M, N, K) triple validation must reject.
void gemm_shapes() {
    for (int64_t m : kSizes)
        for (int64_t n : kSizes)
            for (int64_t k : kSizes) {
                const bool mn_ok = m >= 1 && n >= 1 && m <= INT32_MAX / 2 && n <= INT32_MAX / 2;
                const bool k_ok = positive_multiple(k, 32) && k <= INT32_MAX / 2;
                if (!(mn_ok && k_ok)) {
                    EXPECT_ERR(fp4_gemm_mxfp4(U16, U16, U16, U16, m, n, k, A16, BF, nullptr));
                    EXPECT_ERR(fp4_gemm_mxfp4_splitk(U16, U16, U16, U16, m, n, k, A16, BF, A16,
                                                     ~size_t{0}, nullptr));
                    EXPECT_ERR(fp4_gemm_nvfp4(U16, U16, F16, U16, U16, F16, m, n, k, A16, BF,
                                              nullptr));
                    EXPECT_ERR(fp4_linear_mxfp4(A16, BF, m, k, U16, U16, n, U16, U16, A16, BF,
                                                FP4_LINEAR_TWO_LAUNCHES, A16, WS, nullptr,
                                                nullptr));
                }
                const bool k_packed = positive_multiple(k, 2048) && k <= 16384;
                if (!(mn_ok && k_packed)) {
                    EXPECT_ERR(fp4_gemm_mxfp4_packed(U16, U16, m, n, k, A16, BF, nullptr));
                    EXPECT_ERR(fp4_gemm_nvfp4_packed(U16, F16, U16, F16, m, n, k, A16, BF,
                                                     nullptr));
                    EXPECT_ERR(fp4_linear_mxfp4_packed(A16, BF, m, k, U16, n, U16, ~size_t{0},
                                                       A16, BF, nullptr, nullptr));
                    EXPECT_ERR(fp4_linear_nvfp4_packed(A16, BF, m, k, U16, F16, n, U16,
                                                       ~size_t{0}, F16, A16, BF, A16, WS,
                                                       nullptr, nullptr));
                }
            }
}

// The size helpers: an invalid shape gives the documented value, a valid
// one a size at least the plain byte count (no wrap-around).
void size_helpers() {
    for (int64_t m : kSizes)
        for (int64_t n : kSizes)
            for (int64_t k : kSizes) {
                ++calls;
                const size_t ws = fp4_gemm_splitk_workspace_bytes(m, n, k);
                if (ws != 0) {
                    const bool ok = m >= 1 && n >= 1 && k >= 1;
                    // S >= 1 whole partial products of M x N fp32 each
                    const long double plain = (long double)m * (long double)n * 4.0L;
                    if (!ok || (long double)ws < plain || fmodl((long double)ws, plain) != 0.0L) {
                        std::fprintf(stderr, "splitk workspace (%lld, %lld, %lld) = %zu\n",
                                     (long long)m, (long long)n, (long long)k, ws);
                        ++failures;
                    }
                }
            }
    for (int64_t r : kSizes)
        for (int64_t c : kSizes) {
            calls += 4;
            const int64_t pm = fp4_packed_operand_bytes(r, c);
            const int64_t pn = fp4_nv_packed_operand_bytes(r, c);
            for (int64_t p : {pm, pn})
                if (p != 0 && (p < 0 || (long double)p < (long double)r * (long double)c / 2.0L)) {
                    std::fprintf(stderr, "packed operand bytes (%lld, %lld) = %lld\n",
                                 (long long)r, (long long)c, (long long)p);
                    ++failures;
                }
            for (fp4_format f : {FP4_MXFP4, FP4_NVFP4}) {
                const int64_t s = fp4_padded_storage_bytes(f, r, c);
                const int64_t block = f == FP4_MXFP4 ? 32 : 16;
                if (s == -1) {
                    if (r >= 1 && c >= 1 && (long double)r * (long double)c < 1e12L) {
                        std::fprintf(stderr, "padded storage (%lld, %lld) rejected\n",
                                     (long long)r, (long long)c);
                        ++failures;
                    }
                    continue;
                }
                const long double blocks =
                    (long double)r * ceill((long double)c / (long double)block);
                const long double want = blocks * (long double)(block / 2 + 1) +
                                         (f == FP4_NVFP4 ? 4.0L : 0.0L);
                if (r < 1 || c < 1 || (long double)s != want) {
                    std::fprintf(stderr, "padded storage (%lld, %lld) = %lld\n", (long long)r,
                                 (long long)c, (long long)s);
                    ++failures;
                }
            }
        }
    EXPECT(fp4_padded_storage_bytes(FP4_NVFP4, 2, 17), 40);
    EXPECT(fp4_padded_storage_bytes((fp4_format)7, 2, 17), -1);
    EXPECT(fp4_workspace_bytes(FP4_MXFP4, 8192, 8192), 0);
    EXPECT(fp4_workspace_bytes(FP4_NVFP4, I64MIN, I64MAX) >= 4096, 1);
    EXPECT(fp4_workspace_bytes((fp4_format)-1, 1, 1), 0);
}

// The other argument checks: null pointers, misalignment, unknown enums,
// block sizes, workspaces, candidate grids.
void argument_checks() {
    EXPECT(fp4_quantize_mxfp4(nullptr, BF, 4, 64, 32, U16, U16, nullptr, nullptr), FP4_E_ARG);
    EXPECT(fp4_quantize_mxfp4(A16, BF, 4, 64, 16, U16, U16, nullptr, nullptr), FP4_E_ARG);
    EXPECT(fp4_quantize_mxfp4(A16, (fp4_dtype)7, 4, 64, 32, U16, U16, nullptr, nullptr),
           FP4_E_DTYPE);
    EXPECT(fp4_quantize_mxfp4(A1, BF, 4, 64, 32, U16, U16, nullptr, nullptr), FP4_E_ALIGN);
    EXPECT(fp4_quantize_mxfp4(A16, BF, 4, 64, 32, U16, U16, static_cast<int32_t *>(A1), nullptr),
           FP4_E_ALIGN);
    EXPECT(fp4_quantize_mxfp4_rule(A16, BF, 4, 64, 32, (fp4_mx_rule)3, U16, U16, nullptr,
                                   nullptr),
           FP4_E_ARG);
    EXPECT(fp4_quantize_mxfp4_rule(A16, BF, 4, 64, 32, (fp4_mx_rule)-1, U16, U16, nullptr,
                                   nullptr),
           FP4_E_ARG);
    EXPECT(fp4_quantize_nvfp4(A16, BF, 4, 64, 16, U16, U16, nullptr, A16, WS, nullptr, nullptr),
           FP4_E_ARG);
    EXPECT(fp4_quantize_nvfp4(A16, BF, 4, 64, 32, U16, U16, F16, A16, WS, nullptr, nullptr),
           FP4_E_ARG);
    EXPECT(fp4_quantize_nvfp4(A16, BF, 4, 64, 16, U16, U16, F16, nullptr, WS, nullptr, nullptr),
           FP4_E_WORKSPACE);
    EXPECT(fp4_quantize_nvfp4(A16, BF, 4, 64, 16, U16, U16, F16, A16, 16, nullptr, nullptr),
           FP4_E_WORKSPACE);
    EXPECT(fp4_quantize_nvfp4(A16, BF, 4, 64, 16, U16, U16, F16, A1, WS, nullptr, nullptr),
           FP4_E_ALIGN);
    EXPECT(fp4_quantize_nvfp4_noalloc(A16, BF, 4, 64, 16, U16, nullptr, F16, nullptr, nullptr),
           FP4_E_ARG);
    EXPECT(fp4_quantize_sr((fp4_format)2, A16, BF, 4, 64, 16, 1, U16, U16, F16, A16, WS, nullptr,
                           nullptr),
           FP4_E_DTYPE);
    EXPECT(fp4_dequantize(FP4_MXFP4, U16, U16, nullptr, 4, 64, 16, A16, BF, nullptr), FP4_E_ARG);
    EXPECT(fp4_dequantize(FP4_NVFP4, U16, U16, nullptr, 4, 64, 16, A16, BF, nullptr), FP4_E_ARG);
    EXPECT(fp4_dequantize(FP4_MXFP4, U16, U16, nullptr, 4, 64, 32, A16, (fp4_dtype)2, nullptr),
           FP4_E_DTYPE);
    // candidate grids: too few, non-positive, reversed, too wide, too coarse, NaN
    const float nan = std::numeric_limits<float>::quiet_NaN();
    const float bad[][3] = {{1, 1.0f, 1.0f},     {64, 0.0f, 1.0f},  {64, -1.0f, 1.0f},
                            {64, 1.5f, 0.5f},    {64, 0.5f, 4.5f},  {3, 0.5f, 1.5f},
                            {64, nan, 1.0f},     {64, 0.5f, nan},   {-5, 0.5f, 1.5f},
                            {64, 0.5f, 1e30f}};
    for (const auto &g : bad)
        EXPECT(fp4_scale_search(A16, BF, 4, 64, 16, (int32_t)g[0], g[1], g[2], U16, U16, F16, A16,
                                WS, nullptr, nullptr),
               FP4_E_ARG);
    EXPECT(fp4_scale_search(A16, BF, 4, 64, 16, INT32_MAX, 0.5f, 1.5f, U16, U16, F16, A16, 16,
                            nullptr, nullptr),
           FP4_E_WORKSPACE);
    EXPECT(fp4_scale_search(A16, BF, 4, 64, 16, 64, 0.5f, 1.5f, U16 + 4, U16, F16, A16, WS,
                            nullptr, nullptr),
           FP4_E_ALIGN);
    EXPECT(fp4_scale_search_exhaustive(A16, BF, 4, 64, 16, U16 + 4, U16, F16, A16, WS, nullptr,
                                       nullptr),
           FP4_E_ALIGN);
    EXPECT(fp4_gemm_mxfp4(U16, U16, U16, U16, 128, 256, 256, A16, (fp4_dtype)5, nullptr),
           FP4_E_DTYPE);
    EXPECT(fp4_gemm_mxfp4(U16 + 1, U16, U16, U16, 128, 256, 256, A16, BF, nullptr), FP4_E_ALIGN);
    EXPECT(fp4_gemm_mxfp4_splitk(U16, U16, U16, U16, 128, 256, 1024, A16, BF, A16, 16, nullptr),
           FP4_E_WORKSPACE);
    EXPECT(fp4_linear_mxfp4(A16, BF, 128, 512, U16, U16, 64, U16, U16, A16, BF,
                            (fp4_linear_mode)2, A16, WS, nullptr, nullptr),
           FP4_E_ARG);
    EXPECT(fp4_linear_mxfp4(A16, BF, 128, 512, U16, U16, 64, U16, U16, A16, BF,
                            FP4_LINEAR_ONE_LAUNCH, nullptr, WS, nullptr, nullptr),
           FP4_E_WORKSPACE);
    EXPECT(fp4_pack_mxfp4_operand(U16, U16, 64, 1024, U16, 16, nullptr), FP4_E_WORKSPACE);
    EXPECT(fp4_pack_nvfp4_operand(U16, nullptr, 64, 1024, U16, WS, nullptr), FP4_E_ARG);
    EXPECT(fp4_quantize_padded((fp4_format)3, A16, BF, 2, 17, U16, U16, F16, A16, WS, nullptr,
                               nullptr),
           FP4_E_DTYPE);
    EXPECT(fp4_quantize_padded(FP4_NVFP4, A16, BF, 2, 17, U16, U16, nullptr, A16, WS, nullptr,
                               nullptr),
           FP4_E_ARG);
    EXPECT(fp4_quantize_padded(FP4_NVFP4, A16, BF, 2, 17, U16, U16, F16, A16, 8, nullptr,
                               nullptr),
           FP4_E_WORKSPACE);
    EXPECT(fp4_dequantize_padded(FP4_NVFP4, U16, U16, F16, 2, 17, A1, BF, nullptr), FP4_E_ALIGN);
    for (int s = -2; s < 10; ++s) {
        ++calls;
        const char *msg = fp4_status_str((fp4_status)s);
        if (!msg || !msg[0]) ++failures;
    }
    // the debug entry points with a poll limit validate as the product ones
    for (uint32_t spin : {0u, 1000u, 0xFFFFFFFFu}) {
        EXPECT(fp4_debug_quantize_nvfp4_spin(A16, BF, 4, 64, 16, U16, U16, nullptr, A16, WS,
                                             nullptr, nullptr, spin),
               FP4_E_ARG);
        EXPECT(fp4_debug_quantize_nvfp4_spin(A16, BF, 4, 17, 16, U16, U16, F16, A16, WS,
                                             nullptr, nullptr, spin),
               FP4_E_SHAPE);
        EXPECT(fp4_debug_linear_mxfp4_spin(A16, BF, 128, 512, U16, U16, 64, U16, U16, A16, BF,
                                           FP4_LINEAR_ONE_LAUNCH, nullptr, WS, nullptr, nullptr,
                                           spin),
               FP4_E_WORKSPACE);
    }
}

}  // namespace

int main() {
    argument_checks();
    quantize_shapes();
    gemm_shapes();
    size_helpers();
    std::printf("C ABI sanitize check: %ld calls, %d failures\n", calls, failures);
    return failures == 0 ? 0 : 1;
}
