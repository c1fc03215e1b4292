// Device helpers shared by the HIP kernels of libfp8bs (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

// bf16 halves of a 32-bit word -> fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round to nearest even, two values per instruction
// (v_cvt_pk_bf16_f32; `lo` lands in bits 0-15).  Checked over all 2^32 fp32
// bit patterns: identical to integer round-to-nearest-even of the bits for
// every non-NaN input (denormals and infinities included); NaN inputs give a
// quiet NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// Streaming global accesses (the "nt" cache policy) for data read or written
// once and not consumed right after: the quantizers' bf16 inputs and the
// SiLU kernel's bf16 h.  Measured on MI355X with a 1 GiB stream: 7.2 TB/s
// read and 6.0 TB/s copy with nt, against 6.3 and 5.5 TB/s with the default
// policy.  FP8 codes keep the default policy: the GEMM that follows reads
// them, and with nt stores it fetched them from HBM instead of the last-level
// cache (down projection 137 -> 122 us in the MLP step).
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
    const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
    __builtin_nontemporal_store(nt_u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u32x4*>(p));
}
__device__ __forceinline__ void store_nt8(void* p, uint32_t lo, uint32_t hi) {
    __builtin_nontemporal_store(nt_u32x2{lo, hi}, reinterpret_cast<nt_u32x2*>(p));
}

// Largest finite OCP E4M3FN value.
constexpr float kE4M3Max = 448.0f;

// gfx950's v_cvt_pk_fp8_f32 produces OCP E4M3FN codes with round-to-nearest-
// even, but maps |v| >= 464 to NaN instead of saturating.  Clamping to +-448
// first gives the saturating encoding for every finite input (clamping
// leaves values inside the range untouched and sends the rest to +-448,
// which is what saturating rounding returns for them).
__device__ __forceinline__ float sat448(float v) { return __builtin_amdgcn_fmed3f(v, -kE4M3Max, kE4M3Max); }

// Encode 4 fp32 values into one 32-bit word of E4M3 codes (byte i = value i).
__device__ __forceinline__ uint32_t enc4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
    return (uint32_t)w;
}

// Quotient x / s rounded to nearest fp32, given y = RN(1 / s) and s >= 2^-80:
// q0 = RN(x y), r = RN(x - s q0) (one FMA), q = RN(q0 + r y) (one FMA) --
// Markstein's correction step for a quotient from a correctly rounded
// reciprocal.  For
// binary32 operands whose significands are those of bf16 values (x) and of
// RN(bf16 / 448) (s), this sequence returns exactly RN(x / s): the rounding
// depends only on the two significands when nothing under- or overflows,
// and all 128 x 128 significand pairs were checked against the exact
// quotient.  Quotients small enough for intermediates to underflow lie far
// below the smallest E4M3 subnormal and encode to a signed zero either way;
// copysign keeps the sign of x (and of -0).
__device__ __forceinline__ float div_by_scale(float x, float s, float y) {
    float q0 = x * y;
    float r = __builtin_fmaf(-q0, s, x);
    float q1 = __builtin_fmaf(r, y, q0);
    return __builtin_copysignf(q1, x);
}

// Scale threshold above which div_by_scale is exact (see above).
constexpr float kFastDivMinScale = 0x1p-80f;

// Max of |v| over the 16 lanes of an aligned lane group (xor butterfly inside
// a DPP row).
__device__ __forceinline__ float group16_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 1, 16));
    v = fmaxf(v, __shfl_xor(v, 2, 16));
    v = fmaxf(v, __shfl_xor(v, 4, 16));
    v = fmaxf(v, __shfl_xor(v, 8, 16));
    return v;
}
__device__ __forceinline__ float group4_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 1, 4));
    v = fmaxf(v, __shfl_xor(v, 2, 4));
    return v;
}

// MX block exponent: smallest e with amax <= 448 * 2^e, clamped to
// [-127, 127]; -127 for amax == 0.  Exact, on the fp32 bit pattern.
__device__ __forceinline__ int mx_exponent(float amax) {
    uint32_t a = __float_as_uint(amax) & 0x7fffffffu;
    if (a == 0) return -127;
    int ea;
    uint32_t frac;
    if ((a >> 23) == 0) {                       // subnormal: normalize
        int p = 31 - __clz((int)a);             // highest set bit, value = 2^(p - 149) * 1.f
        ea = p - 149;
        frac = (a << (23 - p)) & 0x7fffffu;
    } else {
        ea = (int)(a >> 23) - 127;
        frac = a & 0x7fffffu;
    }
    int e = (frac <= 0x600000u) ? ea - 8 : ea - 7;   // 448 = 1.75 * 2^8
    e = e < -127 ? -127 : e;
    e = e > 127 ? 127 : e;
    return e;
}

// 2^-e as an fp32 (e in [-127, 127]; 2^-127 is an fp32 subnormal).
__device__ __forceinline__ float pow2_neg(int e) {
    int be = 127 - e;
    return be >= 1 ? __uint_as_float((uint32_t)be << 23) : __uint_as_float(1u << (22 + be));
}

// Codes of 8 values of one group given its scale s (S == 0 -> all 0x00).
__device__ __forceinline__ void encode8(const float v[8], float s, uint32_t& w0, uint32_t& w1) {
    float qv[8];
    if (s >= kFastDivMinScale) {
        const float y = 1.0f / s;                 // IEEE division: y = RN(1/s)
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = div_by_scale(v[i], s, y);
    } else if (s > 0.0f) {                        // subnormal-range scales: plain IEEE division
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = v[i] / s;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = 0.0f;
    }
    w0 = enc4(qv[0], qv[1], qv[2], qv[3]);
    w1 = enc4(qv[4], qv[5], qv[6], qv[7]);
}

// The same codes as encode8 with the group's reciprocal y = RN(1 / s)
// supplied by the caller (read only when s >= kFastDivMinScale), for kernels
// that compute each scale once and share it between lanes.
__device__ __forceinline__ void encode8_y(const float v[8], float s, float y, uint32_t& w0, uint32_t& w1) {
    float qv[8];
    if (s >= kFastDivMinScale) {
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = div_by_scale(v[i], s, y);
    } else if (s > 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = v[i] / s;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = 0.0f;
    }
    w0 = enc4(qv[0], qv[1], qv[2], qv[3]);
    w1 = enc4(qv[4], qv[5], qv[6], qv[7]);
}

__device__ __forceinline__ void unpack8(const uint4 raw, float v[8]) {
    v[0] = bf16_lo(raw.x); v[1] = bf16_hi(raw.x);
    v[2] = bf16_lo(raw.y); v[3] = bf16_hi(raw.y);
    v[4] = bf16_lo(raw.z); v[5] = bf16_hi(raw.z);
    v[6] = bf16_lo(raw.w); v[7] = bf16_hi(raw.w);
}

__device__ __forceinline__ float absmax8(const float v[8]) {
    float m = fabsf(v[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    return m;
}

// silu(g) * u in fp32, before rounding to bf16, for g >= -44.
// silu(g) = g * sigmoid(g), with sigmoid(g) = 1 / (1 + t) for g >= 0 and
// t / (1 + t) for g < 0, t = exp(-|g|) in (0, 1]: no overflow, and 1 + t in
// [1, 2] for the hardware reciprocal; t stays an fp32 normal over the range.
// t = 2^a with a = -|g| log2(e): the hardware exp2 of the exact product of
// |g| with a 16-bit head of log2(e), times the first-order correction for the
// rest.  Measured over every bf16 g >= -44 (except 0 < |g| < 2^-124),
// g * sigmoid(g) is within 3.22 * 2^-24 of its exact value relatively, so
// h = (g * sigmoid(g)) * u is within 3.72 fp32 ulps of the exact h.
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
    // log2(e) = kLog2eHi + rest, kLog2eHi with 16 significant bits, so that
    // |g| kLog2eHi is exact for a bf16 g (8 significant bits); the rest times
    // ln 2 (kLog2eLoLn2) gives the first-order correction of the exp2
    constexpr float kLog2eHi = 0x1.7154p+0f;
    constexpr float kLog2eLoLn2 = 0x1.480fb6p-18f;
    // |g| clamped to 128 (where t is far below fp32's resolution of 1 + t)
    // so that the exponent cannot overflow
    const float ng = fmaxf(-fabsf(g), -128.0f);
    const float t0 = __builtin_amdgcn_exp2f(ng * kLog2eHi);
    const float t = __builtin_fmaf(t0, ng * kLog2eLoLn2, t0);
    const float r = __builtin_amdgcn_rcpf(1.0f + t);
    const float sig = g >= 0.0f ? r : t * r;
    return (g * sig) * u;
}

// Where silu_mul_f32 cannot decide the bf16 rounding of h (finite inputs):
// h lies within kSiluNearUlps fp32 ulps of a bf16 rounding midpoint (an fp32
// pattern whose low 16 bits are 0x8000); g < -44, where t leaves the fp32
// normal range; or 0 < |g| < 2^-124, where g * sigmoid(g) can lose precision
// to fp32 denormals.
constexpr uint32_t kSiluNearUlps = 5;
constexpr float kSiluGMin = -44.0f;
constexpr float kSiluGTiny = 0x1p-124f;
__device__ __forceinline__ uint32_t silu_mid_dist(float h) {
    // 0 .. 2 kSiluNearUlps where h is near a midpoint
    return (__float_as_uint(h) + (kSiluNearUlps - 0x8000u)) & 0xffffu;
}
__device__ __forceinline__ bool silu_needs_f64(float g, float h) {
    return silu_mid_dist(h) <= 2u * kSiluNearUlps || g < kSiluGMin ||
           (fabsf(g) < kSiluGTiny && g != 0.0f);
}

// fp64 -> bf16 pattern, round to nearest even.  bf16 has fp32's exponent
// range: 8 significant bits down to 2^-126, then a fixed spacing of 2^-133.
// The magnitude is scaled so that one bf16 spacing becomes 1 and rounded to
// an integer q; the pattern is then (exponent of the spacing + 133) * 2^7 + q,
// which also carries q = 256 into the next binade and gives 0x7f80
// (infinity) past the largest finite value.
__device__ __forceinline__ uint32_t bf16_from_f64_rne(double x) {
    const uint64_t bits = (uint64_t)__double_as_longlong(x);
    const uint32_t sign = (uint32_t)(bits >> 48) & 0x8000u;
    const uint32_t hi = (uint32_t)(bits >> 32) & 0x7fffffffu;
    if (hi >= 0x7ff00000u) return sign | ((hi > 0x7ff00000u || (uint32_t)bits != 0u) ? 0x7fc0u : 0x7f80u);
    const double ax = fabs(x);
    int e2;
    (void)frexp(ax, &e2);                       // ax in [2^(e2-1), 2^e2)
    const int se = (e2 - 1 < -126 ? -126 : e2 - 1) - 7;
    const double q = rint(ldexp(ax, -se));      // exact scaling, then ties to even
    if (q == 0.0) return sign;
    const uint32_t b = (uint32_t)((se + 133) * 128) + (uint32_t)q;
    return sign | (b >= 0x7f80u ? 0x7f80u : b);
}

// Constants of the rare fp64 path: log2(e); ln(2) as a 39-bit head (n * head
// is exact for the |n| <= 1077 used) and the rounded rest; the clamp of the
// exponential's argument to [-746, 710] (beyond it the result is 0 or
// infinite in fp64 already); then 1/k! for k = 13 .. 0, each rounded to the
// nearest double.
__device__ const double kSiluF64[19] = {
    0x1.71547652b82fep+0,  0x1.62e42fefa2000p-1,  0x1.9ef35793c7673p-41, 0x1.63p+9, -0x1.75p+9,
    0x1.6124613a86d09p-33, 0x1.1eed8eff8d898p-29, 0x1.ae64567f544e4p-26, 0x1.27e4fb7789f5cp-22,
    0x1.71de3a556c734p-19, 0x1.a01a01a01a01ap-16, 0x1.a01a01a01a01ap-13, 0x1.6c16c16c16c17p-10,
    0x1.1111111111111p-7,  0x1.5555555555555p-5,  0x1.5555555555555p-3,  0x1p-1, 0x1p+0, 0x1p+0};

// exp(x) in fp64: x = n ln 2 + r with n = rint(x log2 e) and |r| <= ln(2)/2
// (Cody-Waite reduction with the split ln 2), e^r from its Taylor series to
// degree 13 (the first dropped term is below 2^-57 relative), scaled by 2^n.
// `c` is kSiluF64.
typedef __attribute__((address_space(4))) const double* silu_cptr;     // scalar-loadable
__device__ __forceinline__ double silu_exp_f64(double x, silu_cptr c) {
    x = fmin(fmax(x, c[4]), c[3]);
    const double n = rint(x * c[0]);
    double r = fma(-n, c[1], x);
    r = fma(-n, c[2], r);
    double p = c[5];
#pragma unroll
    for (int k = 6; k < 19; ++k) p = fma(p, r, c[k]);
    return ldexp(p, (int)n);
}

// h = g / (1 + exp(-g)) * u evaluated in fp64 and rounded once to bf16: the
// definition of the bf16 h that the next GEMM consumes.  The constants are
// read through a pointer the compiler cannot see through, so that they are
// loaded here, on the rare path that needs them, instead of being hoisted out
// of the callers' loops into registers held throughout.
__device__ __forceinline__ uint32_t silu_mul_bf16_f64(float g, float u) {
    silu_cptr c = (silu_cptr)kSiluF64;
    asm volatile("" : "+s"(c));
    const double gd = g;
    return bf16_from_f64_rne(gd / (1.0 + silu_exp_f64(-gd, c)) * (double)u);
}

// The values of silu_mul_f32 for eight (g, u) as bf16 patterns, and whether
// this lane holds one that they cannot round (about 2^-12 of the values at
// GEMM-output magnitudes); one test over the eight (their minima) decides it.
__device__ __forceinline__ bool silu_mul8_bf16_fast(const float g[8], const float u[8], uint32_t hb[8], float h[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = silu_mul_f32(g[i], u[i]);
    float gmin = g[0], amin = fabsf(g[0]);
    uint32_t dmin = silu_mid_dist(h[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        gmin = fminf(gmin, g[i]);
        amin = fminf(amin, fabsf(g[i]));
        dmin = min(dmin, silu_mid_dist(h[i]));
    }
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const uint32_t w = pack_bf16x2(h[i], h[i + 1]);
        hb[i] = w & 0xffffu;
        hb[i + 1] = w >> 16;
    }
    return gmin < kSiluGMin || amin < kSiluGTiny || dmin <= 2u * kSiluNearUlps;
}

// Replaces, in hb, each value that the fp32 evaluation h cannot round by the
// fp64 evaluation (on the lanes and values that need it).
__device__ __forceinline__ void silu_fix8(const float g[8], const float u[8], const float h[8], uint32_t hb[8]) {
    uint32_t need = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) need |= (uint32_t)silu_needs_f64(g[i], h[i]) << i;
    while (need != 0) {
        const int k = __builtin_ctz(need);
        need &= need - 1;
        float gk = g[0], uk = u[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            gk = k == i ? g[i] : gk;
            uk = k == i ? u[i] : uk;
        }
        const uint32_t r = silu_mul_bf16_f64(gk, uk);
#pragma unroll
        for (int i = 0; i < 8; ++i) hb[i] = k == i ? r : hb[i];
    }
}

// h = bf16(silu(g) * u) for the eight bf16 (g, u) pairs packed in gw, uw,
// bit-exact against the fp64 evaluation: the fp32 one, and on the rare lanes
// where it cannot decide a rounding, the fp64 one for those values.
__device__ __forceinline__ void silu_mul8_bf16(const uint4 gw, const uint4 uw, uint32_t hb[8]) {
    float g[8], u[8], h[8];
    unpack8(gw, g);
    unpack8(uw, u);
    if (__builtin_expect(silu_mul8_bf16_fast(g, u, hb, h), 0)) silu_fix8(g, u, h, hb);
}

}  // namespace fp8bs
