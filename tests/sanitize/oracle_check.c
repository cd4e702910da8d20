/*
 * oracle_check.c - drives every routine of the C oracle (oracle/fp4_oracle.c)
 * once per case on inputs that reach its edge paths, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Test infrastructure:
 * built and run by tests/test_sanitize_host.py.
 *
 * Every output buffer is a heap block of exactly the size the routine's
 * comment states, so a write one byte past it is reported.  Inputs mix
 * normal values over many binades, zero blocks, signed zeros, fp32
 * subnormals, the largest finite values, NaN and infinities, in fp32 and
 * bf16, over lengths of one block up to a few hundred blocks.  Besides the
 * sanitizers' reports, a few invariants that hold for any input are checked
 * (codes survive unpack and pack, a zero block keeps its default scale).
 * Exit status 0 means every call ran clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's routines (it has no header: Python reaches it through ctypes). */
double or_e2m1_value(int code);
int or_e2m1_round(float q);
void or_e2m1_round_array(const float *q, int64_t n, uint8_t *codes);
void or_pack(const uint8_t *codes, int64_t n, uint8_t *out);
void or_unpack(const uint8_t *bytes, int64_t nbytes, uint8_t *codes);
double or_e4m3_value(int code);
int or_e4m3_nearest(double num, double den);
uint16_t or_f32_to_bf16(float f);
int or_mx_exponent(double amax);
int or_mx_quantize(const void *x, int dt, int64_t n, uint8_t *packed, uint8_t *scales);
int or_mx_exponent_ceil(double amax);
float or_block_loss32_pow2(const float *xb, int e);
int or_mx_quantize_rule(const void *x, int dt, int64_t n, int rule, uint8_t *packed,
                        uint8_t *scales);
int or_nv_global_scale(const void *x, int dt, int64_t n, float *s_g);
int or_nv_quantize(const void *x, int dt, int64_t n, float s_g, uint8_t *packed,
                   uint8_t *scales);
void or_dequantize(int fmt, const uint8_t *packed, const uint8_t *scales, float s_g, int64_t n,
                   int out_dt, void *y);
float or_block_loss_f32(const float *xb, float alpha);
float or_candidate_c(int k, int ncand, float c_lo, float c_hi);
int or_scale_search(const void *x, int dt, int64_t n, float s_g, int ncand, float c_lo,
                    float c_hi, uint8_t *packed, uint8_t *scales, float *best_loss);
int or_scale_search_all(const void *x, int dt, int64_t n, float s_g, uint8_t *packed,
                        uint8_t *scales, float *best_loss);
void or_ideal_roundtrip(const float *x, int64_t n, int block, float *y);
int or_ideal_code(float x, float alpha);
int64_t or_storage_bytes(int64_t elements, int block, int64_t global_bytes);
int64_t or_padded_storage_bytes(int64_t rows, int64_t cols, int block, int64_t global_bytes);
int or_mx_quantize_padded(const void *x, int dt, int64_t rows, int64_t cols, uint8_t *packed,
                          uint8_t *scales);
int or_nv_quantize_padded(const void *x, int dt, int64_t rows, int64_t cols, uint8_t *packed,
                          uint8_t *scales, float *s_g);
int or_dequantize_padded(int fmt, const uint8_t *packed, const uint8_t *scales, float s_g,
                         int64_t rows, int64_t cols, int out_dt, void *y);
uint32_t or_sr_bits(uint64_t seed, int64_t i);
int or_e2m1_round_sr(float q, uint32_t r24);
int or_mx_quantize_sr(const void *x, int dt, int64_t n, uint64_t seed, uint8_t *packed,
                      uint8_t *scales);
int or_nv_quantize_sr(const void *x, int dt, int64_t n, float s_g, uint64_t seed,
                      uint8_t *packed, uint8_t *scales);

enum { F32 = 0, BF16 = 1 };

static int failures = 0;
static long calls = 0;

#define CHECK(cond, ...)                                                   \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check failed (%s:%d): ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                                  \
            fputc('\n', stderr);                                           \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

/* xorshift64*: input generation only */
static uint64_t rng_state = 0x2545F4914F6CDD1Dull;
static uint64_t next_u64(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}
static double next_unit(void) { return (double)(next_u64() >> 11) * 0x1p-53; }

static float bits_f32(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

/* One input of n values.  kind 0: finite values only; kind 1: finite plus
 * one NaN and one infinity; kind 2: all zero; kind 3: tiny values only. */
static float *make_f32(int64_t n, int kind) {
    float *x = (float *)malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) {
        double r = next_unit();
        int pick = (int)(next_u64() % 16);
        float v;
        if (kind == 2) v = 0.0f;
        else if (kind == 3) v = bits_f32((uint32_t)(next_u64() % 0x01000000u));  /* below 2^-125 */
        else if (pick == 0) v = 0.0f;
        else if (pick == 1) v = -0.0f;
        else if (pick == 2) v = bits_f32(1u + (uint32_t)(next_u64() % 0x007FFFFFu)); /* subnormal */
        else if (pick == 3) v = 3.4028234663852886e38f * (float)(r > 0.5 ? 1 : -1);
        else v = (float)((r - 0.5) * ldexp(1.0, (int)(next_u64() % 60) - 30));
        x[i] = v;
    }
    /* whole zero blocks at the start (block 16 and block 32) */
    if (kind <= 1 && n >= 64)
        for (int64_t i = 0; i < 32; ++i) x[i] = (i & 1) ? -0.0f : 0.0f;
    if (kind == 1) {
        x[n / 2] = NAN;
        x[n - 1] = -INFINITY;
    }
    return x;
}

static uint16_t *to_bf16(const float *x, int64_t n) {
    uint16_t *b = (uint16_t *)malloc((size_t)n * 2);
    for (int64_t i = 0; i < n; ++i) b[i] = or_f32_to_bf16(x[i]);
    return b;
}

static void check_nibbles(const uint8_t *packed, int64_t nbytes) {
    uint8_t *codes = (uint8_t *)malloc((size_t)nbytes * 2);
    or_unpack(packed, nbytes, codes);
    for (int64_t i = 0; i < 2 * nbytes; ++i) CHECK(codes[i] < 16, "code %d", codes[i]);
    uint8_t *again = (uint8_t *)malloc((size_t)nbytes);
    or_pack(codes, 2 * nbytes, again);
    CHECK(memcmp(again, packed, (size_t)nbytes) == 0, "pack(unpack) differs");
    free(again);
    free(codes);
}

/* Whether elements [0, len) of x are all +-0 (those blocks keep the default scale). */
static int leading_zeros(const void *x, int dt, int64_t len) {
    for (int64_t i = 0; i < len; ++i) {
        uint32_t b = dt == BF16 ? ((const uint16_t *)x)[i] & 0x7FFFu
                                : ((const uint32_t *)x)[i] & 0x7FFFFFFFu;
        if (b) return 0;
    }
    return 1;
}

static void scalar_routines(void) {
    for (int c = 0; c < 16; ++c) CHECK(isfinite(or_e2m1_value(c)), "e2m1 value %d", c);
    for (int c = 0; c < 256; ++c) (void)or_e4m3_value(c);
    const float specials[] = {0.0f, -0.0f, 0.25f, 0.75f, 5.0f, 6.0f, 7.0f, 1e30f, -1e30f,
                              1e-45f, NAN, INFINITY, -INFINITY};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
        int c = or_e2m1_round(specials[i]);
        CHECK(c >= -1 && c < 16, "round %d", c);
        (void)or_e2m1_round_sr(specials[i], 0);
        (void)or_e2m1_round_sr(specials[i], 0xFFFFFFu);
        (void)or_ideal_code(specials[i], 0.5f);
        (void)or_ideal_code(specials[i], 0.0f);
        (void)or_f32_to_bf16(specials[i]);
        calls += 6;
    }
    /* a block amax is the magnitude of an fp32 or bf16 element */
    const double amaxes[] = {0.0, 0x1p-149, 0x1p-127, 0x1p-126, 1.0, 5.99, 6.0, 448.0,
                             3.4028234663852886e38};
    for (size_t i = 0; i < sizeof amaxes / sizeof amaxes[0]; ++i) {
        int e = or_mx_exponent(amaxes[i]);
        CHECK(e >= -127 && e <= 127, "mx exponent %d", e);
        int ec = or_mx_exponent_ceil(amaxes[i]);
        CHECK(ec >= -127 && ec <= 127, "ceil exponent %d", ec);
        int n = or_e4m3_nearest(amaxes[i], 6.0 * 0x1p-20);
        CHECK(n >= 0 && n <= 126, "e4m3 nearest %d", n);
        calls += 3;
    }
    for (int k = 0; k < 64; ++k) (void)or_candidate_c(k, 64, 0.75f, 1.25f);
    for (int64_t i = 0; i < 1000; ++i) CHECK(or_sr_bits(~0ull, i) < (1u << 24), "sr bits");
    CHECK(or_storage_bytes(1024, 32, 0) == 544 && or_storage_bytes(1024, 16, 4) == 580,
          "storage bytes");
    CHECK(or_padded_storage_bytes(2, 17, 16, 4) == 40, "padded storage bytes");
    calls += 64 + 1000 + 3;
}

/* Every complete-block routine on one input of n elements (n a multiple of 32). */
static void block_routines(const void *x, int dt, int64_t n, const float *xf) {
    uint8_t *packed = (uint8_t *)malloc((size_t)n / 2);
    uint8_t *sc32 = (uint8_t *)malloc((size_t)n / 32);
    uint8_t *sc16 = (uint8_t *)malloc((size_t)n / 16);
    float *loss = (float *)malloc((size_t)n / 16 * sizeof(float));
    float *yf = (float *)malloc((size_t)n * sizeof(float));
    uint16_t *yb = (uint16_t *)malloc((size_t)n * 2);

    (void)or_mx_quantize(x, dt, n, packed, sc32);
    check_nibbles(packed, n / 2);
    if (leading_zeros(x, dt, 32)) CHECK(sc32[0] == 127, "zero MX block scale %d", sc32[0]);
    for (int fmt_out = 0; fmt_out < 2; ++fmt_out)
        or_dequantize(0, packed, sc32, 1.0f, n, fmt_out, fmt_out ? (void *)yb : (void *)yf);
    for (int rule = 0; rule < 3; ++rule) {
        (void)or_mx_quantize_rule(x, dt, n, rule, packed, sc32);
        check_nibbles(packed, n / 2);
    }
    (void)or_mx_quantize_sr(x, dt, n, 12345u, packed, sc32);
    check_nibbles(packed, n / 2);

    float s_g = 0.0f;
    (void)or_nv_global_scale(x, dt, n, &s_g);
    const float sgs[] = {s_g, 1.0f, 0x1p-140f, 3.0e38f};
    for (size_t k = 0; k < sizeof sgs / sizeof sgs[0]; ++k) {
        (void)or_nv_quantize(x, dt, n, sgs[k], packed, sc16);
        check_nibbles(packed, n / 2);
        if (leading_zeros(x, dt, 16)) CHECK(sc16[0] == 0x38, "zero NV block scale %d", sc16[0]);
        for (int fmt_out = 0; fmt_out < 2; ++fmt_out)
            or_dequantize(1, packed, sc16, sgs[k], n, fmt_out, fmt_out ? (void *)yb : (void *)yf);
        (void)or_nv_quantize_sr(x, dt, n, sgs[k], 99u, packed, sc16);
        (void)or_scale_search(x, dt, n, sgs[k], 64, 0.5f, 1.5f, packed, sc16, loss);
        (void)or_scale_search(x, dt, n, sgs[k], 2, 1.0f, 1.0f, packed, sc16, NULL);
        check_nibbles(packed, n / 2);
        calls += 5;
    }
    if (n <= 4096) {  /* 126 candidates per block: kept to the shorter inputs */
        (void)or_scale_search_all(x, dt, n, s_g, packed, sc16, loss);
        check_nibbles(packed, n / 2);
        calls += 1;
    }
    if (xf) {
        const int blocks[] = {16, 32, 4096};
        for (int k = 0; k < 3; ++k)
            if (n % blocks[k] == 0) or_ideal_roundtrip(xf, n, blocks[k], yf);
        or_e2m1_round_array(xf, n, (uint8_t *)yb);
        for (int64_t b = 0; b < n / 32; ++b) {
            (void)or_block_loss32_pow2(xf + 32 * b, -127);
            (void)or_block_loss32_pow2(xf + 32 * b, 127);
            (void)or_block_loss_f32(xf + 32 * b, 0x1p-149f);
            (void)or_block_loss_f32(xf + 32 * b + 16, 1.0f);
        }
        calls += 5;
    }
    /* a scale byte that decodes to NaN (E8M0 255, E4M3 0x7F and 0xFF) */
    memset(sc32, 255, (size_t)n / 32);
    memset(sc16, 0x7F, (size_t)n / 16);
    or_dequantize(0, packed, sc32, 1.0f, n, 0, yf);
    or_dequantize(1, packed, sc16, 1.0f, n, 1, yb);
    calls += 12;

    free(yb);
    free(yf);
    free(loss);
    free(sc16);
    free(sc32);
    free(packed);
}

/* The row-padded routines on rows x cols (cols need not be a multiple of a block). */
static void padded_routines(int64_t rows, int64_t cols, int kind) {
    const int64_t n = rows * cols;
    float *xf = make_f32(n, kind);
    uint16_t *xb = to_bf16(xf, n);
    for (int fmt = 0; fmt < 2; ++fmt) {
        const int block = fmt == 0 ? 32 : 16;
        const int64_t pc = (cols + block - 1) / block * block;
        uint8_t *packed = (uint8_t *)malloc((size_t)(rows * pc / 2));
        uint8_t *scales = (uint8_t *)malloc((size_t)(rows * pc / block));
        float *y = (float *)malloc((size_t)n * sizeof(float));
        float s_g = 1.0f;
        for (int dt = 0; dt < 2; ++dt) {
            const void *x = dt == BF16 ? (const void *)xb : (const void *)xf;
            int f = fmt == 0 ? or_mx_quantize_padded(x, dt, rows, cols, packed, scales)
                             : or_nv_quantize_padded(x, dt, rows, cols, packed, scales, &s_g);
            CHECK(f >= 0, "padded quantize ran out of memory");
            CHECK(or_dequantize_padded(fmt, packed, scales, s_g, rows, cols, dt, y) == 0,
                  "padded dequantize");
            calls += 2;
        }
        free(y);
        free(scales);
        free(packed);
    }
    free(xb);
    free(xf);
}

int main(void) {
    scalar_routines();
    const int64_t lengths[] = {32, 64, 96, 1024, 4096 + 32, 16384};
    for (size_t li = 0; li < sizeof lengths / sizeof lengths[0]; ++li) {
        for (int kind = 0; kind < 4; ++kind) {
            const int64_t n = lengths[li];
            float *xf = make_f32(n, kind);
            uint16_t *xb = to_bf16(xf, n);
            block_routines(xf, F32, n, xf);
            block_routines(xb, BF16, n, NULL);
            free(xb);
            free(xf);
        }
    }
    const int64_t shapes[][2] = {{1, 1}, {2, 17}, {3, 31}, {5, 33}, {7, 100}, {1, 4097}};
    for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; ++si)
        for (int kind = 0; kind < 3; ++kind) padded_routines(shapes[si][0], shapes[si][1], kind);
    printf("oracle sanitize check: %ld calls, %d failed checks\n", calls, failures);
    return failures == 0 ? 0 : 1;
}
