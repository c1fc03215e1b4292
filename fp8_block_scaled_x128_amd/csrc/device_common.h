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
// q0 = RN(x y), r = RN(x - s q0) (one FMA), q = RN(q0 + r y) (one FMA).  For
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

// silu(g) * u rounded to bf16 and widened back (the value the next GEMM consumes).
// silu(g) = g * sigmoid(g), with sigmoid(g) = 1 / (1 + t) for g >= 0 and
// t / (1 + t) for g < 0, t = exp(-|g|) in (0, 1]: no overflow, and 1 + t in
// [1, 2] for the hardware reciprocal.  t = 2^a with a = -|g| log2(e) split
// into a rounded part for the hardware exp2 and its exact residual applied to
// first order, so t is good to about one fp32 ulp.  Where t would be an fp32
// denormal (a < -64, that is |g| above about 44.4) it is formed scaled by 2^64
// and the scale is removed from the final product.  The accurate expf and IEEE
// division cost about 25 more instructions per element, enough to make this
// kernel VALU bound.  The product is rounded once to bf16: the result stays
// within one bf16 ulp of the exactly rounded value, and differs from it only
// where the exact value lies a few fp32 ulp from a bf16 rounding midpoint.
__device__ __forceinline__ uint32_t silu_mul_bf16(float g, float u) {
    constexpr float kLog2e = 1.4426950216293335f;       // log2(e) rounded to fp32
    constexpr float kLog2eLo = 1.925963033500011e-08f;  // log2(e) - kLog2e
    constexpr float kLn2 = 0.6931471824645996f;
    const float ng = -fabsf(g);
    const float a_hi = ng * kLog2e;
    const float a_lo = __builtin_fmaf(ng, kLog2e, -a_hi) + ng * kLog2eLo;
    const bool tiny = a_hi < -64.0f;
    const float t = __builtin_amdgcn_exp2f(tiny ? a_hi + 64.0f : a_hi) * __builtin_fmaf(a_lo, kLn2, 1.0f);
    const float r = __builtin_amdgcn_rcpf(1.0f + (tiny ? 0.0f : t));
    const float sig = g >= 0.0f ? r : t * r;
    float h = (g * sig) * u;
    if (tiny && g < 0.0f) h *= 0x1p-64f;
    return f32_to_bf16_rne(h);
}

}  // namespace fp8bs
