/*
 * tern_oracle.c -- the plain, slow CPU reference of the ternary-weight matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or constant with the HIP library.
 *
 * What it computes (source: the 2kiu.com article "putting a ternary embedding
 * model into vLLM", news/5082861):
 *   - each weight is one of {-1, 0, +1} stored as a 2-bit code:
 *     00 -> 0, 01 -> +1, 10 -> -1, 11 -> reserved, read as 0       (§3.1)
 *   - four codes per byte, first weight in the two lowest bits       (§3.1)
 *   - every 128 consecutive weights of a row along K share one fp16
 *     scale; blocks are cut contiguously along K                      (§1.1, §3.1)
 *   - y = x . W^T with x[M,K] fp16 activations, W[N,K] ternary,
 *     stored as packed[N,K/4] bytes plus scale[N,K/128]             (§4.2)
 *   - inside a block the signs are accumulated without multiplies
 *     (+1 adds, -1 subtracts, 0 skips) and the block sum is multiplied
 *     by its scale only at the block boundary                       (§1.1, §4.1, §4.2)
 *
 *   Y[m,n] = sum_g S[n,g] * sum_{k in block g} t(n,k) * X[m,k]
 *
 * Arithmetic is float64 throughout.  The fp16 / bf16 inputs are decoded from
 * their bit patterns by the decoders below (sign, exponent, fraction), so no
 * compiler half-precision support is involved.
 *
 * Parity pins (exhaustive byte tables, brute force, closed forms, exact
 * arithmetic, a dense numpy reduction) live in the test suite.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* ---------- floating-point formats, decoded from bits ---------- */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* zero or subnormal: f * 2^-24 */
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);    /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);              /* f * 2^-126 / 128 */
    else if (e == 255)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(128 + f), e - 134);    /* (1 + f/128) * 2^(e-127) */
    return sign ? -v : v;
}

/* IEEE binary32 decoded from bits (used to read fp32 results). */
double oracle_f32_to_f64(uint32_t u) {
    int sign = (u >> 31) & 1;
    int e = (u >> 23) & 0xFF;
    uint32_t f = u & 0x7FFFFF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -149);
    else if (e == 255)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(0x800000u + f), e - 150);
    return sign ? -v : v;
}

/* Format parameters: p = significant bits, emin = smallest normal exponent,
 * emax = largest exponent.  kind: 0 = fp16, 1 = bf16, 2 = fp32. */
static int fmt_params(int kind, int *p, int *emin, int *emax) {
    switch (kind) {
    case 0: *p = 11; *emin = -14;  *emax = 15;  return 0;
    case 1: *p = 8;  *emin = -126; *emax = 127; return 0;
    case 2: *p = 24; *emin = -126; *emax = 127; return 0;
    default: return -1;
    }
}

/* Spacing of the format's values at |v|: 2^(max(exponent of v, emin) - p + 1). */
double oracle_ulp(double v, int kind) {
    int p, emin, emax, ex;
    if (fmt_params(kind, &p, &emin, &emax)) return NAN;
    double a = fabs(v);
    if (a == 0.0 || !isfinite(a)) return ldexp(1.0, emin - p + 1);
    frexp(a, &ex);                 /* a = m * 2^ex, 0.5 <= m < 1: leading bit at ex-1 */
    int e = ex - 1;
    if (e < emin) e = emin;
    return ldexp(1.0, e - p + 1);
}

/* Round v to the nearest value of the format, ties to even; overflow gives inf. */
double oracle_round(double v, int kind) {
    int p, emin, emax;
    if (fmt_params(kind, &p, &emin, &emax)) return NAN;
    if (v == 0.0 || !isfinite(v)) return v;
    double a = fabs(v);
    if (a >= ldexp(1.0, emax + 1)) return v > 0 ? INFINITY : -INFINITY;
    double q = oracle_ulp(a, kind);
    double r = nearbyint(a / q) * q;   /* a/q is exact (q is a power of two); default mode = ties-to-even */
    if (r >= ldexp(1.0, emax + 1)) r = INFINITY;
    return v > 0 ? r : -r;
}

/* ---------- the 2-bit code ---------- */

/* Code -> weight value: 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0 (reserved). */
int oracle_code_value(unsigned code) {
    switch (code) {
    case 0: return 0;
    case 1: return 1;
    case 2: return -1;
    case 3: return 0;
    default: return 0;
    }
}

/* Weight -> code used by packing.  Values outside {-1,0,1} are written as the
 * reserved code 11, which reads back as 0. */
static unsigned value_code(int t) {
    if (t == 0) return 0;
    if (t == 1) return 1;
    if (t == -1) return 2;
    return 3;
}

/* Weight (n, k) of a packed [N, K/4] matrix: byte k/4 of row n, bits 2*(k%4)..+1. */
int oracle_weight(const uint8_t *packed, int64_t K, int64_t n, int64_t k) {
    uint8_t byte = packed[n * (K / 4) + k / 4];
    unsigned code = (byte >> (2 * (k % 4))) & 3u;
    return oracle_code_value(code);
}

/* packed[N, K/4] -> T[N, K] with values in {-1, 0, +1}. */
int oracle_unpack(const uint8_t *packed, int8_t *T, int64_t N, int64_t K) {
    if (N < 0 || K < 0 || K % 4 != 0) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            T[n * K + k] = (int8_t)oracle_weight(packed, K, n, k);
    return 0;
}

/* T[N, K] -> packed[N, K/4]: weight 4j+i of a row goes to bits 2i..2i+1 of byte j. */
int oracle_pack(const int8_t *T, uint8_t *packed, int64_t N, int64_t K) {
    if (N < 0 || K < 0 || K % 4 != 0) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 4; ++j) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i)
                byte |= value_code(T[n * K + 4 * j + i]) << (2 * i);
            packed[n * (K / 4) + j] = (uint8_t)byte;
        }
    return 0;
}

/* ---------- the matmul ---------- */

static double x_value(const uint16_t *X, int x_kind, int64_t K, int64_t m, int64_t k) {
    uint16_t bits = X[m * K + k];
    return x_kind == 1 ? oracle_bf16_to_f64(bits) : oracle_f16_to_f64(bits);
}

/* The sign-accumulated sum of one block (add for +1, subtract for -1, skip
 * for 0) of row n against activation row m, and the block's sum of |x|:
 *   block = sum_{k in [k0,k1), t=+1} x[m,k] - sum_{k in [k0,k1), t=-1} x[m,k] */
static double block_sum(const uint16_t *X, int x_kind, const uint8_t *packed, int64_t K,
                        int64_t m, int64_t n, int64_t k0, int64_t k1, double *abs_x) {
    double block = 0.0, ax = 0.0;
    for (int64_t k = k0; k < k1; ++k) {
        double x = x_value(X, x_kind, K, m, k);
        int t = oracle_weight(packed, K, n, k);
        if (t == 1) block += x;            /* +1: add      */
        else if (t == -1) block -= x;      /* -1: subtract */
                                           /*  0: skip     */
        ax += fabs(x);
    }
    *abs_x = ax;
    return block;
}

/* One output element and its error scale:
 *   y = sum_g s[n,g] * (sum_{k in g, t=+1} x[m,k] - sum_{k in g, t=-1} x[m,k])
 *   b = sum_k |x[m,k] * s[n, k/G]|
 */
static void one_output(const uint16_t *X, int x_kind, const uint8_t *packed,
                       const uint16_t *S, int64_t K, int64_t G, int64_t m, int64_t n,
                       double *y_out, double *b_out) {
    int64_t groups = K / G;
    double y = 0.0, b = 0.0;
    for (int64_t g = 0; g < groups; ++g) {
        double s = oracle_f16_to_f64(S[n * groups + g]);
        double ax;
        double block = block_sum(X, x_kind, packed, K, m, n, g * G, (g + 1) * G, &ax);
        y += s * block;                        /* scale applied at the block boundary */
        b += fabs(s) * ax;
    }
    *y_out = y;
    *b_out = b;
}

static int check_args(int64_t M, int64_t N, int64_t K, int64_t G, int x_kind) {
    if (M < 0 || N < 0 || K < 0 || G <= 0) return -1;
    if (K % 4 != 0 || K % G != 0) return -1;
    if (x_kind != 0 && x_kind != 1) return -1;
    return 0;
}

/* Y[M, N] and B[M, N] (float64) for output columns n0 <= n < n1 (all rows m).
 * x_kind: 0 = fp16 bits, 1 = bf16 bits.  S holds fp16 bits, [N, K/G]. */
int oracle_matmul_cols(const uint16_t *X, int x_kind, const uint8_t *packed,
                       const uint16_t *S, int64_t M, int64_t N, int64_t K, int64_t G,
                       int64_t n0, int64_t n1, double *Y, double *B) {
    if (check_args(M, N, K, G, x_kind)) return -1;
    if (n0 < 0 || n1 > N || n0 > n1) return -1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = n0; n < n1; ++n)
            one_output(X, x_kind, packed, S, K, G, m, n, &Y[m * N + n], &B[m * N + n]);
    return 0;
}

int oracle_matmul(const uint16_t *X, int x_kind, const uint8_t *packed, const uint16_t *S,
                  int64_t M, int64_t N, int64_t K, int64_t G, double *Y, double *B) {
    return oracle_matmul_cols(X, x_kind, packed, S, M, N, K, G, 0, N, Y, B);
}

/* Selected outputs only: (ms[i], ns[i]) for i < count -> Y[i], B[i]. */
int oracle_matmul_at(const uint16_t *X, int x_kind, const uint8_t *packed, const uint16_t *S,
                     int64_t M, int64_t N, int64_t K, int64_t G, const int64_t *ms,
                     const int64_t *ns, int64_t count, double *Y, double *B) {
    if (check_args(M, N, K, G, x_kind)) return -1;
    for (int64_t i = 0; i < count; ++i) {
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
        one_output(X, x_kind, packed, S, K, G, ms[i], ns[i], &Y[i], &B[i]);
    }
    return 0;
}

/* ---------- array helpers (bit patterns -> float64) ---------- */

void oracle_decode_array(const void *bits, int kind, int64_t count, double *out) {
    for (int64_t i = 0; i < count; ++i) {
        if (kind == 0) out[i] = oracle_f16_to_f64(((const uint16_t *)bits)[i]);
        else if (kind == 1) out[i] = oracle_bf16_to_f64(((const uint16_t *)bits)[i]);
        else out[i] = oracle_f32_to_f64(((const uint32_t *)bits)[i]);
    }
}

void oracle_round_array(const double *v, int kind, int64_t count, double *out) {
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_round(v[i], kind);
}

void oracle_ulp_array(const double *v, int kind, int64_t count, double *out) {
    for (int64_t i = 0; i < count; ++i) out[i] = oracle_ulp(v[i], kind);
}

/* ---------- the dequantised weight matrix (comparison route) ---------- */

/* W[n,k] = t(n,k) * S[n, k/G] in float64 (the dense matrix the pages' first
 * route multiplies with a library GEMM: 2kiu.com/news/5082861 §4.1). */
int oracle_dequant(const uint8_t *packed, const uint16_t *S, int64_t N, int64_t K, int64_t G,
                   double *W) {
    if (N < 0 || K < 0 || G <= 0 || K % 4 != 0 || K % G != 0) return -1;
    int64_t groups = K / G;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[n * K + k] = oracle_weight(packed, K, n, k) * oracle_f16_to_f64(S[n * groups + k / G]);
    return 0;
}

/* ---------- the all-zero block map ---------- */

/* map[n, g/32] bit (g%32) = 1 when block g of row n holds a nonzero weight
 * (a code 01 or 10); blocks of only 00 / 11 codes contribute nothing and may
 * be skipped (2kiu.com/news/5082861 §6: a sparse mask to skip zero blocks).
 * words_per_row = ceil((K/G) / 32). */
int oracle_block_map(const uint8_t *packed, int64_t N, int64_t K, int64_t G, uint32_t *map) {
    if (N < 0 || K < 0 || G <= 0 || K % 4 != 0 || K % G != 0) return -1;
    int64_t groups = K / G, words = (groups + 31) / 32;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t w = 0; w < words; ++w) map[n * words + w] = 0;
        for (int64_t g = 0; g < groups; ++g) {
            int any = 0;
            for (int64_t k = g * G; k < (g + 1) * G; ++k)
                if (oracle_weight(packed, K, n, k) != 0) any = 1;
            if (any) map[n * words + g / 32] |= (uint32_t)1 << (g % 32);
        }
    }
    return 0;
}

/* ---------- int8 scales ---------- */

/* Per-row symmetric int8 quantisation of the fp16 scales (a reading of
 * 2kiu.com/news/5082861 §6, "compress the FP16 scale further to INT8"):
 *   r[n]   = fp32( max_g |s[n,g]| / 127 )          (0 when the row's scales are all 0)
 *   q[n,g] = round-half-even( fp32( s[n,g] / r[n] ) ), within [-127, 127]
 * The integer is decided in IEEE single precision, the precision the device
 * kernel divides in, so both sides take the same decision.  The effective
 * scale is q * r.  r is returned as float32. */
int oracle_quantize_scales(const uint16_t *S, int64_t N, int64_t groups, int8_t *q, float *r) {
    if (N < 0 || groups < 0) return -1;
    for (int64_t n = 0; n < N; ++n) {
        float amax = 0.0f;
        for (int64_t g = 0; g < groups; ++g) {
            float a = (float)fabs(oracle_f16_to_f64(S[n * groups + g]));   /* exact: fp16 -> fp32 */
            if (a > amax) amax = a;
        }
        volatile float rn = amax / 127.0f;
        r[n] = rn;
        for (int64_t g = 0; g < groups; ++g) {
            float t = 0.0f;
            if (rn > 0.0f) {
                volatile float quot = (float)oracle_f16_to_f64(S[n * groups + g]) / rn;
                t = nearbyintf(quot);
            }
            if (t > 127.0f) t = 127.0f;
            if (t < -127.0f) t = -127.0f;
            q[n * groups + g] = (int8_t)t;
        }
    }
    return 0;
}

/* Y and B as oracle_matmul_cols, with the effective scale q[n,g] * r[n]
 * (r given as fp32 bits, the stored form). */
int oracle_matmul_s8_cols(const uint16_t *X, int x_kind, const uint8_t *packed, const int8_t *q,
                          const uint32_t *r_bits, int64_t M, int64_t N, int64_t K, int64_t G,
                          int64_t n0, int64_t n1, double *Y, double *B) {
    if (check_args(M, N, K, G, x_kind)) return -1;
    if (n0 < 0 || n1 > N || n0 > n1) return -1;
    int64_t groups = K / G;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = n0; n < n1; ++n) {
            double rn = oracle_f32_to_f64(r_bits[n]);
            double y = 0.0, b = 0.0;
            for (int64_t g = 0; g < groups; ++g) {
                double s = (double)q[n * groups + g] * rn;
                double ax;
                double block = block_sum(X, x_kind, packed, K, m, n, g * G, (g + 1) * G, &ax);
                y += s * block;
                b += fabs(s) * ax;
            }
            Y[m * N + n] = y;
            B[m * N + n] = b;
        }
    return 0;
}
