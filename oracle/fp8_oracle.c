/*
 * CPU oracle for the block-wise FP8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source with the HIP kernels.
 *
 * Plain scalar C, fp64 wherever the method does not fix the precision.
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fopenmp
 * (no FMA contraction, IEEE fp32 division, denormals kept).  OpenMP is used
 * only across independent rows / groups / output elements.
 *
 * What is computed, and where it is stated:
 *  - The two-step quantizer, scale S = max|X| / V_max, then Q(x) = round(x/S):
 *    "Unified FP8: Beyond Mixed Precision..." (winzheng.com), section
 *    "FP8 Quantization", Step 1 and Step 2.
 *  - E4M3 as the FP8 element format (4 exponent bits, 3 mantissa bits): same
 *    page, section "FP8 Format".  The OCP E4M3FN variant is used: bias 7,
 *    largest finite 448, no infinities, NaN = S.1111.111.  Rounding is
 *    round-to-nearest-even and out-of-range values saturate to +-448.
 *  - FP32 scales: same page, section "FP8 Scale Selection".
 *  - Granularities: per-token activations, per-block weights, per-token
 *    gradients: same page, section "FP8 Quantization" (bullet list).
 *    Block layout 128x128 with FP32 scales: "Low Precision RL"
 *    (miles.radixark.com), table "Choose a precision" and section
 *    "2. Unified block-wise FP8 (DeepSeek-style)".  Activations use 1x128
 *    groups along the contraction axis; weight-gradient operands use 128x1
 *    groups along the token axis.
 *  - Per-tensor and per-row (whole-row) groups: the "per-tensor" strategy of
 *    "Unified FP8: Beyond Mixed Precision...", section "FP8 Quantization",
 *    and the tensorwise and rowwise scalings that "Towards Full Pipeline FP8
 *    Reinforcement Learning for LLMs" (agihunt.info) compares with
 *    blockwise scaling in its accuracy and throughput results.  The same two
 *    steps, with one group per tensor or per row.
 *  - MXFP8: 32 consecutive E4M3 values share one UE8M0 (power-of-two) scale:
 *    "Low Precision RL", table "Choose a precision" and section
 *    "3. Unified MXFP8 (Blackwell)".  The exponent is the smallest e with
 *    amax <= 448 * 2^e, i.e. 2^ceil(log2(amax/448)).
 *  - The block-scaled GEMM: the dequantized operands' product, i.e.
 *    Y[m,n] = sum_k (dec(qa[m,k]) * sa) * (dec(qb[n,k]) * sb), here in fp64.
 *    The pages require the trainer and rollout forward GEMMs to consume the
 *    same quantized operands ("Low Precision RL", "Unified training recipe").
 *
 * Readings taken where the pages are silent:
 *  - an all-zero group has S = 0 and every code 0x00 (also -0 inputs);
 *  - the division x/S is one IEEE fp32 division, then one E4M3 rounding;
 *  - a group that extends past the end of a row/column covers only the
 *    elements present;
 *  - MX: an all-zero block gets exponent -127 (code 0x00) and codes 0x00;
 *    the exponent is clamped to [-127, 127].
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* bit helpers                                                          */
/* ------------------------------------------------------------------ */
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 is the upper half of an fp32 bit pattern. */
OR_EXPORT float or_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest even (NaN kept quiet). */
OR_EXPORT uint16_t or_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* fp64 -> bf16 with a single rounding (round to nearest even).  Works on the
 * fp64 bit pattern so that no intermediate fp32 rounding happens. */
OR_EXPORT uint16_t or_f64_to_bf16(double d)
{
    uint64_t u; memcpy(&u, &d, 8);
    uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    uint64_t a = u & 0x7fffffffffffffffull;
    if (a > 0x7ff0000000000000ull) return (uint16_t)(sign | 0x7fc0u);
    if (a == 0x7ff0000000000000ull) return (uint16_t)(sign | 0x7f80u);
    if (a == 0) return sign;
    int e = (int)(a >> 52) - 1023;            /* unbiased exponent */
    uint64_t m = a & 0x000fffffffffffffull;
    if ((a >> 52) == 0) {                      /* fp64 subnormal: far below bf16 range */
        return sign;
    }
    m |= 0x0010000000000000ull;                /* 53-bit significand */
    /* bf16: normal if e >= -126, 8-bit significand (7 stored).  Spacing
     * 2^(max(e,-126) - 7). */
    int se = (e < -126 ? -126 : e) - 7;        /* exponent of one bf16 ulp */
    int shift = 52 + se - e;                   /* m * 2^(e-52) / 2^se = m >> shift */
    if (shift > 60) return sign;               /* < half of the smallest subnormal */
    uint64_t q = m >> shift;
    uint64_t rem = m & ((1ull << shift) - 1ull);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1ull))) q++;
    /* q is the significand in units of 2^se; rebuild the bf16 pattern.  For a
     * normal result q is in [128, 256]; q == 256 carries into the exponent.
     * For a subnormal result (se == -133) q in [0, 128]. */
    uint32_t code;
    if (se == -133) {
        code = (uint32_t)q;                    /* subnormal (q == 128 -> min normal 0x0080) */
    } else {
        code = (uint32_t)((e + 127) << 7) + (uint32_t)q - 128u;
    }
    if (code >= 0x7f80u) return (uint16_t)(sign | 0x7f80u);   /* overflow -> inf */
    return (uint16_t)(sign | code);
}

/* ------------------------------------------------------------------ */
/* OCP E4M3FN codec                                                     */
/* ------------------------------------------------------------------ */

/* Decode one code s.eeee.mmm.  e == 0: subnormal m * 2^-9 (includes +-0);
 * 1 <= e <= 15: (1 + m/8) * 2^(e-7); e == 15 and m == 7: NaN. */
OR_EXPORT double or_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Encode an fp32 value: round to nearest, ties to even mantissa, saturate
 * to +-448 (also +-Inf), NaN -> 0x7F | sign.  Integer arithmetic on the fp32
 * bit pattern: the E4M3 grid spacing below |v| is 2^(max(floor(log2|v|),-6) - 3). */
OR_EXPORT uint8_t or_e4m3_encode(float v)
{
    uint32_t u = f32_bits(v);
    uint8_t sign = (uint8_t)((u >> 31) << 7);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint8_t)(sign | 0x7f);      /* NaN */
    if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7e);     /* |v| >= 448 (incl. Inf) */
    if ((a >> 23) == 0) return sign;                          /* fp32 zero/subnormal: < 2^-126 */
    int e = (int)(a >> 23) - 127;                             /* floor(log2|v|) */
    uint32_t m = (a & 0x7fffffu) | 0x800000u;                 /* |v| = m * 2^(e-23) */
    int eg = e < -6 ? -6 : e;                                 /* binade of the grid */
    int shift = 23 + (eg - 3) - e;                            /* m >> shift = |v| / spacing */
    if (shift > 24) return sign;                              /* |v| < spacing/2 */
    uint32_t q = m >> shift;
    uint32_t rem = m & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    /* code = (eg + 6) * 8 + q covers normal binades (q in [8,16], q == 16
     * carries into the exponent) and the subnormal range (eg = -6, q in [0,8]). */
    uint32_t code = (uint32_t)(eg + 6) * 8u + q;
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------ */
/* Quantizers with FP32 scales                                          */
/* ------------------------------------------------------------------ */

/* One group: amax over the present elements, S = amax / 448 (IEEE fp32
 * division), codes enc(x / S) (one fp32 division per element).  S == 0 gives
 * codes 0x00.  `xs` holds the group's values already widened to fp32. */
static float quant_group(const float* xs, int64_t n, uint8_t* codes)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(xs[i]);
        if (a > amax) amax = a;
    }
    float s = amax / 448.0f;
    for (int64_t i = 0; i < n; ++i)
        codes[i] = (s == 0.0f) ? (uint8_t)0 : or_e4m3_encode(xs[i] / s);
    return s;
}

/* 1x128 groups along the contiguous axis (per-token activations).
 * x: [rows][ld_x] bf16; q: [rows][cols]; s: [rows][ceil(cols/128)]. */
OR_EXPORT void or_quant_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              uint8_t* q, float* s)
{
    int64_t ng = (cols + 127) / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float buf[128];
        for (int64_t g = 0; g < ng; ++g) {
            int64_t c0 = g * 128, n = cols - c0 < 128 ? cols - c0 : 128;
            for (int64_t i = 0; i < n; ++i) buf[i] = or_bf16_to_f32(x[r * ld_x + c0 + i]);
            s[r * ng + g] = quant_group(buf, n, q + r * cols + c0);
        }
    }
}

/* 128x1 groups along the row (token) axis, output transposed so that the
 * token axis is contiguous: qt: [cols][rows]; s: [cols][ceil(rows/128)].
 * Equal, by definition, to 1x128 quantization of the transposed matrix. */
OR_EXPORT void or_quant_128x1_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                uint8_t* qt, float* s)
{
    int64_t ng = (rows + 127) / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        float buf[128];
        for (int64_t g = 0; g < ng; ++g) {
            int64_t r0 = g * 128, n = rows - r0 < 128 ? rows - r0 : 128;
            for (int64_t i = 0; i < n; ++i) buf[i] = or_bf16_to_f32(x[(r0 + i) * ld_x + c]);
            s[c * ng + g] = quant_group(buf, n, qt + c * rows + r0);
        }
    }
}

/* 128x128 blocks (weights).  q: [rows][cols]; s: [ceil(rows/128)][ceil(cols/128)]. */
OR_EXPORT void or_quant_128x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                uint8_t* q, float* s)
{
    int64_t nbr = (rows + 127) / 128, nbc = (cols + 127) / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nbr * nbc; ++b) {
        int64_t br = b / nbc, bc = b % nbc;
        int64_t r0 = br * 128, c0 = bc * 128;
        int64_t nr = rows - r0 < 128 ? rows - r0 : 128;
        int64_t nc = cols - c0 < 128 ? cols - c0 : 128;
        float amax = 0.0f;
        for (int64_t i = 0; i < nr; ++i)
            for (int64_t j = 0; j < nc; ++j) {
                float a = fabsf(or_bf16_to_f32(x[(r0 + i) * ld_x + c0 + j]));
                if (a > amax) amax = a;
            }
        float sc = amax / 448.0f;
        s[br * nbc + bc] = sc;
        for (int64_t i = 0; i < nr; ++i)
            for (int64_t j = 0; j < nc; ++j) {
                float v = or_bf16_to_f32(x[(r0 + i) * ld_x + c0 + j]);
                q[(r0 + i) * cols + c0 + j] = (sc == 0.0f) ? (uint8_t)0 : or_e4m3_encode(v / sc);
            }
    }
}

/* One group per row (rowwise scaling): q: [rows][cols]; s: [rows]. */
OR_EXPORT void or_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                uint8_t* q, float* s)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float amax = 0.0f;
        for (int64_t c = 0; c < cols; ++c) {
            float a = fabsf(or_bf16_to_f32(x[r * ld_x + c]));
            if (a > amax) amax = a;
        }
        float sc = amax / 448.0f;
        s[r] = sc;
        for (int64_t c = 0; c < cols; ++c) {
            float v = or_bf16_to_f32(x[r * ld_x + c]);
            q[r * cols + c] = (sc == 0.0f) ? (uint8_t)0 : or_e4m3_encode(v / sc);
        }
    }
}

/* One group for the whole tensor (tensorwise scaling): q: [rows][cols];
 * s: one float. */
OR_EXPORT void or_quant_tensorwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   uint8_t* q, float* s)
{
    float amax = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float a = fabsf(or_bf16_to_f32(x[r * ld_x + c]));
            if (a > amax) amax = a;
        }
    float sc = amax / 448.0f;
    *s = sc;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float v = or_bf16_to_f32(x[r * ld_x + c]);
            q[r * cols + c] = (sc == 0.0f) ? (uint8_t)0 : or_e4m3_encode(v / sc);
        }
}

/* ------------------------------------------------------------------ */
/* MXFP8 quantizer (1x32 blocks, UE8M0 scales)                          */
/* ------------------------------------------------------------------ */

/* Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127];
 * amax == 0 gives -127.  Exact: works on the fp32 exponent and mantissa. */
OR_EXPORT int or_mx_exponent(float amax)
{
    uint32_t a = f32_bits(amax) & 0x7fffffffu;
    if (a == 0) return -127;
    int ea;
    uint32_t frac;                              /* 23-bit fraction of the normalized significand */
    if ((a >> 23) == 0) {                       /* fp32 subnormal: normalize */
        uint32_t m = a;
        ea = -126;
        while (!(m & 0x800000u)) { m <<= 1; ea -= 1; }
        frac = m & 0x7fffffu;
    } else {
        ea = (int)(a >> 23) - 127;
        frac = a & 0x7fffffu;
    }
    /* amax = (1+f) 2^ea, 448 = 1.75 * 2^8.  (1+f) <= 1.75  <=>  frac <= 0x600000. */
    int e = (frac <= 0x600000u) ? ea - 8 : ea - 7;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* x: [rows][ld_x] bf16 -> q: [rows][cols], s: [rows][ceil(cols/32)] UE8M0
 * codes (e + 127).  Codes are enc(x * 2^-e); the power-of-two scaling is exact
 * in fp32 for every finite bf16 input of such a block. */
OR_EXPORT void or_mx_quant_1x32(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                uint8_t* q, uint8_t* s)
{
    int64_t ng = (cols + 31) / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            int64_t c0 = g * 32, n = cols - c0 < 32 ? cols - c0 : 32;
            float amax = 0.0f;
            for (int64_t i = 0; i < n; ++i) {
                float a = fabsf(or_bf16_to_f32(x[r * ld_x + c0 + i]));
                if (a > amax) amax = a;
            }
            int e = or_mx_exponent(amax);
            s[r * ng + g] = (uint8_t)(e + 127);
            double inv = ldexp(1.0, -e);       /* exact power of two */
            for (int64_t i = 0; i < n; ++i) {
                float v = or_bf16_to_f32(x[r * ld_x + c0 + i]);
                float scaled = (float)((double)v * inv);   /* exact unless far below E4M3 range */
                q[r * cols + c0 + i] = (amax == 0.0f) ? (uint8_t)0 : or_e4m3_encode(scaled);
            }
        }
    }
}

/* Block-wise groups with power-of-two scales: 1x128 groups along a row
 * (block_rows == 1) or 128x128 blocks (block_rows == 128).  Each group takes
 * the MX exponent rule on its own amax (e = or_mx_exponent(amax), the
 * smallest e with amax <= 448 * 2^e), stores the UE8M0 byte e + 127 and
 * encodes enc(x * 2^-e).  q: [rows][cols]; s: scale byte of (row group i,
 * column group g) at s[i * ld_s + g]. */
OR_EXPORT void or_quant_pow2(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int64_t block_rows,
                             uint8_t* q, uint8_t* s, int64_t ld_s)
{
    int64_t ngr = (rows + block_rows - 1) / block_rows, ngc = (cols + 127) / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < ngr; ++i) {
        int64_t r0 = i * block_rows, r1 = r0 + block_rows < rows ? r0 + block_rows : rows;
        for (int64_t g = 0; g < ngc; ++g) {
            int64_t c0 = g * 128, c1 = c0 + 128 < cols ? c0 + 128 : cols;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float a = fabsf(or_bf16_to_f32(x[r * ld_x + c]));
                    if (a > amax) amax = a;
                }
            int e = or_mx_exponent(amax);
            s[i * ld_s + g] = (uint8_t)(e + 127);
            double inv = ldexp(1.0, -e);
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float v = or_bf16_to_f32(x[r * ld_x + c]);
                    float scaled = (float)((double)v * inv);
                    q[r * cols + c] = (amax == 0.0f) ? (uint8_t)0 : or_e4m3_encode(scaled);
                }
        }
    }
}

/* UE8M0 decode: 2^(c-127); 0xFF is NaN. */
OR_EXPORT double or_ue8m0_decode(uint8_t c)
{
    if (c == 0xff) return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* ------------------------------------------------------------------ */
/* Reference GEMMs (fp64 on dequantized operands)                        */
/* ------------------------------------------------------------------ */

/* Scale of B element (n, k) for the two B-scale granularities:
 *   mode 0: 128x128 blocks, sb[(n/128) * stride_n + (k/128) * stride_k]
 *   mode 1: 1x128 rows,     sb[n * stride_n + (k/128) * stride_k]
 * A's scale of element (m, k) is sa[m * sa_sm + (k/128) * sa_sk]. */
static double b_scale(const float* sb, int mode, int64_t n, int64_t k,
                      int64_t stride_n, int64_t stride_k)
{
    int64_t rn = mode == 0 ? n / 128 : n;
    return (double)sb[rn * stride_n + (k / 128) * stride_k];
}

/* One output element: y = sum_k Atilde[m,k] * Btilde[n,k], and the absolute
 * sum sum_k |Atilde * Btilde| used by the error bound.  B is stored [N][K]. */
static void dot_fp32scale(int64_t m, int64_t n, int64_t K,
                          const uint8_t* qa, int64_t lda, const float* sa, int64_t sa_sm, int64_t sa_sk,
                          const uint8_t* qb, int64_t ldb, const float* sb, int64_t sb_sn, int64_t sb_sk, int mode,
                          double* y, double* yabs)
{
    double acc = 0.0, accabs = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double a = or_e4m3_decode(qa[m * lda + k]) * (double)sa[m * sa_sm + (k / 128) * sa_sk];
        double b = or_e4m3_decode(qb[n * ldb + k]) * b_scale(sb, mode, n, k, sb_sn, sb_sk);
        acc += a * b;
        accabs += fabs(a * b);
    }
    *y = acc;
    if (yabs) *yabs = accabs;
}

/* Full reference GEMM: Y[M][N] (fp64) and Babs[M][N] (nullable). */
OR_EXPORT void or_gemm_blockscaled(int64_t M, int64_t N, int64_t K,
                                   const uint8_t* qa, int64_t lda, const float* sa, int64_t sa_sm, int64_t sa_sk,
                                   const uint8_t* qb, int64_t ldb, const float* sb, int64_t sb_sn, int64_t sb_sk,
                                   int mode, double* y, double* yabs)
{
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            dot_fp32scale(m, n, K, qa, lda, sa, sa_sm, sa_sk, qb, ldb, sb, sb_sn, sb_sk, mode,
                          &y[m * N + n], yabs ? &yabs[m * N + n] : 0);
}

/* Sampled reference GEMM: only the `count` outputs (mi[i], ni[i]). */
OR_EXPORT void or_gemm_blockscaled_sampled(int64_t K,
                                           const uint8_t* qa, int64_t lda, const float* sa, int64_t sa_sm, int64_t sa_sk,
                                           const uint8_t* qb, int64_t ldb, const float* sb, int64_t sb_sn, int64_t sb_sk,
                                           int mode, const int64_t* mi, const int64_t* ni, int64_t count,
                                           double* y, double* yabs)
{
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i)
        dot_fp32scale(mi[i], ni[i], K, qa, lda, sa, sa_sm, sa_sk, qb, ldb, sb, sb_sn, sb_sk, mode,
                      &y[i], yabs ? &yabs[i] : 0);
}

/* MXFP8 reference GEMM: scales are UE8M0 codes, sa: [M][K/32], sb: [N][K/32]
 * (row strides lds_a, lds_b).  `mi`/`ni` select outputs (count of them). */
OR_EXPORT void or_gemm_mx_sampled(int64_t K,
                                  const uint8_t* qa, int64_t lda, const uint8_t* sa, int64_t lds_a,
                                  const uint8_t* qb, int64_t ldb, const uint8_t* sb, int64_t lds_b,
                                  const int64_t* mi, const int64_t* ni, int64_t count,
                                  double* y, double* yabs)
{
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = mi[i], n = ni[i];
        double acc = 0.0, accabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = or_e4m3_decode(qa[m * lda + k]) * or_ue8m0_decode(sa[m * lds_a + k / 32]);
            double b = or_e4m3_decode(qb[n * ldb + k]) * or_ue8m0_decode(sb[n * lds_b + k / 32]);
            acc += a * b;
            accabs += fabs(a * b);
        }
        y[i] = acc;
        if (yabs) yabs[i] = accabs;
    }
}

/* ------------------------------------------------------------------ */
/* SiLU(gate) * up between the MoE projections                          */
/* ------------------------------------------------------------------ */

/* gu: [rows][ld] bf16 holding gate in columns [0, I) and up in [I, 2I).
 * h[r][j] = bf16( silu(g) * u ), silu(g) = g / (1 + exp(-g)), evaluated in
 * fp64 and rounded once to bf16. */
OR_EXPORT void or_silu_mul(const uint16_t* gu, int64_t rows, int64_t I, int64_t ld, uint16_t* h)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < I; ++j) {
            double g = (double)or_bf16_to_f32(gu[r * ld + j]);
            double u = (double)or_bf16_to_f32(gu[r * ld + I + j]);
            h[r * I + j] = or_f64_to_bf16(g / (1.0 + exp(-g)) * u);
        }
}

/* ------------------------------------------------------------------ */
/* MoE combine after the down projection                                */
/* ------------------------------------------------------------------ */

/* Each token's output is the sum of its experts' outputs weighted by its
 * routing weights: out[t][n] = sum_j w[t][j] * y[pos[t][j]][n] over the
 * token's k slots, j = 0..k-1, in fp64.  y: [rows][ld_y] bf16 expert
 * outputs in grouped (expert-sorted) order; pos[t][j]: the grouped row of
 * token t's j-th assignment; w: [T][k] fp32.  out: [T][H] fp64. */
OR_EXPORT void or_moe_combine(const uint16_t* y, int64_t H, int64_t ld_y, const int32_t* pos,
                              const float* w, int64_t T, int64_t k, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < H; ++n) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j)
                acc += (double)w[t * k + j] * (double)or_bf16_to_f32(y[(int64_t)pos[t * k + j] * ld_y + n]);
            out[t * H + n] = acc;
        }
}

/* Number of OpenMP threads the parallel loops above use. */
OR_EXPORT int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the number of OpenMP threads of the parallel loops above (timing of
 * the oracle at one thread and at every core; the results do not depend on
 * it: every loop only splits independent rows or groups). */
OR_EXPORT void or_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
