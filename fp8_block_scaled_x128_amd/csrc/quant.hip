// Quantization kernels of libfp8bs (gfx950).
//
// Each group of values gets S = max|x| / 448 (IEEE fp32 division) and codes
// E4M3(x / S) with round-to-nearest-even and saturation, the two-step
// quantizer of "Unified FP8: Beyond Mixed Precision..." (section "FP8
// Quantization", Steps 1 and 2), with the groupings of "Low Precision RL"
// (table "Choose a precision"): 1x128 per-token groups, 128x1 token-axis
// groups for the weight-gradient operands, 128x128 weight blocks, and 1x32
// MXFP8 blocks with power-of-two (UE8M0) scales.
//
// All kernels are HBM-bound.  They read bf16 with 16-byte loads (8 values
// per lane), reduce the group maximum with lane shuffles inside the 16-lane
// DPP row that owns a 1x128 group, and write codes with 8- or 16-byte stores.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fp8bs {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Row-group quantizer.  A 16-lane DPP row owns one 128-wide run of a row
// (8 values per lane); it holds one 1x128 FP32-scale group, or four 1x32 MX
// blocks (4 lanes each).  SILU: the run is h = silu(gate) * up computed from
// the gate (columns [0, I)) and up (columns [I, 2I)) halves of the input row.
// ROW_FAST: consecutive runs go down a column of groups (so that M-major
// scale arrays are written contiguously); otherwise along a row.
// Each 16-lane row processes U runs per loop trip with all loads issued first.
// ---------------------------------------------------------------------------
struct RowArgs {
    const uint16_t* x; int64_t ld_x;
    int32_t rows, cols;          // cols: width of the quantized matrix (I for SILU)
    int64_t up_off;              // SILU: column offset of the up half
    uint8_t* q; int64_t ld_q;
    void* s; int64_t ssr, ssg;
    uint16_t* h; int64_t ld_h;   // SILU: optional bf16 h output
    int32_t runs_per_row, total_runs;
};

// P2: 128-element groups with power-of-two scales (the MX exponent rule on
// the group's amax, a UE8M0 byte per group, codes E4M3(x * 2^-e)).
// The body takes its workgroup index and count as arguments so that the
// fused linear-operand kernel below can run it on part of its grid.
template <bool SILU, bool MX, bool ROW_FAST, int U, bool NTQ, bool P2>
__device__ __forceinline__ void rowgroup_body(const RowArgs& p, int32_t block, int32_t nblocks) {
    const int sub = threadIdx.x & 15;
    const int32_t rid = block * (kThreads / 16) + (int32_t)(threadIdx.x >> 4);
    const int32_t nr = nblocks * (kThreads / 16);
    for (int32_t base = rid; base < p.total_runs; base += nr * U) {
        uint4 raw[U], raw_u[U];
        int32_t rr[U], gg[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t run = base + u * nr;
            int32_t r, g;
            if (ROW_FAST) { g = run / p.rows; r = run - g * p.rows; }
            else { r = run / p.runs_per_row; g = run - r * p.runs_per_row; }
            rr[u] = r; gg[u] = g;
            const int32_t c = g * 128 + sub * 8;
            raw[u] = make_uint4(0, 0, 0, 0);
            raw_u[u] = make_uint4(0, 0, 0, 0);
            if (run < p.total_runs && c < p.cols) {
                const uint16_t* src = p.x + (int64_t)r * p.ld_x + c;
                raw[u] = load_nt16(src);
                if (SILU) raw_u[u] = load_nt16(src + p.up_off);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t run = base + u * nr;
            const int32_t r = rr[u], g = gg[u];
            const int32_t c = g * 128 + sub * 8;
            const bool valid = run < p.total_runs && c < p.cols;
            float v[8];
            unpack8(raw[u], v);
            if (SILU) {
                uint32_t hb[8];
                silu_mul8_bf16(raw[u], raw_u[u], hb);
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(hb[i] << 16);
                if (p.h != nullptr && valid) {
                    uint4 hw = make_uint4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16),
                                          hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16));
                    store_nt16(p.h + (int64_t)r * p.ld_h + c, hw);
                }
            }
            uint32_t w0, w1;
            if (!MX && !P2) {
                const float amax = group16_max(absmax8(v));
                const float s = amax / kE4M3Max;
                encode8(v, s, w0, w1);
                if (valid && sub == 0)
                    static_cast<float*>(p.s)[(int64_t)r * p.ssr + (int64_t)g * p.ssg] = s;
            } else if (P2) {
                const float amax = group16_max(absmax8(v));
                const int e = mx_exponent(amax);
                const float f = pow2_neg(e);
                if (amax == 0.0f) {
                    w0 = 0u; w1 = 0u;
                } else {
                    w0 = enc4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
                    w1 = enc4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
                }
                if (valid && sub == 0)
                    static_cast<uint8_t*>(p.s)[(int64_t)r * p.ssr + (int64_t)g * p.ssg] = (uint8_t)(e + 127);
            } else {
                const float amax = group4_max(absmax8(v));
                const int e = mx_exponent(amax);
                const float f = pow2_neg(e);
                if (amax == 0.0f) {
                    w0 = 0u; w1 = 0u;
                } else {
                    w0 = enc4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
                    w1 = enc4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
                }
                if (valid && (sub & 3) == 0)
                    static_cast<uint8_t*>(p.s)[(int64_t)r * p.ssr + (int64_t)(g * 4 + (sub >> 2)) * p.ssg] =
                        (uint8_t)(e + 127);
            }
            if (valid) {
                uint8_t* dst = p.q + (int64_t)r * p.ld_q + c;
                if (NTQ) store_nt8(dst, w0, w1);
                else *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
            }
        }
    }
}

template <bool SILU, bool MX, bool ROW_FAST, int U, bool NTQ, bool P2>
__global__ void __launch_bounds__(kThreads) k_rowgroup(RowArgs p) {
    rowgroup_body<SILU, MX, ROW_FAST, U, NTQ, P2>(p, (int32_t)blockIdx.x, (int32_t)gridDim.x);
}

template <bool SILU, bool MX, bool P2 = false>
hipError_t launch_rowgroup(RowArgs p, bool row_fast, hipStream_t st) {
    // Runs per trip, measured with inputs rotated past the last-level cache:
    // SILU three (its exact path keeps 91 registers live with three, 105
    // with four: 5 against 4 waves per SIMD, 2-3% faster); 1x128 two (2-3%
    // faster than four, six and eight were slower); MX four (two: 4% slower)
    constexpr int U = SILU ? 3 : MX ? 4 : 2;
    if (p.total_runs == 0) return hipSuccess;
    const int64_t rows16 = ((int64_t)p.total_runs + U - 1) / U;            // 16-lane rows needed
    int64_t blocks = (rows16 + (kThreads / 16) - 1) / (kThreads / 16);
    // one trip per 16-lane row up to 2^16 workgroups: a grid-stride loop
    // over fewer workgroups (at most 4096) ran large tensors at 4.4 TB/s
    // against 6.1 TB/s for one trip each (MX 196608 x 2048)
    if (blocks > 256 * 256) blocks = 256 * 256;
    // codes larger than the 256 MB last-level cache (MX weight stacks) are
    // written with the streaming policy; smaller ones stay cached for the GEMM
    const bool ntq = (int64_t)p.total_runs * 128 > ((int64_t)256 << 20);
    auto go = [&](auto rf, auto nt) {
        hipLaunchKernelGGL((k_rowgroup<SILU, MX, decltype(rf)::value, U, decltype(nt)::value, P2>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, st, p);
    };
    if (row_fast) {
        if (ntq) go(std::true_type{}, std::true_type{});
        else go(std::true_type{}, std::false_type{});
    } else {
        if (ntq) go(std::false_type{}, std::true_type{});
        else go(std::false_type{}, std::false_type{});
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token-axis groups with transposed output: 128x1 with FP32 scales, or (MX)
// 32x1 with UE8M0 scales.  No LDS.  A lane holds RPL consecutive rows of 8
// columns (RPL loads of 16 bytes); the 128 / RPL lanes of a lane group hold
// the 128 rows of a row group for the same 8 columns, and the wave's 64 / (128
// / RPL) lane groups sit side by side in columns.  Column k of a lane is the
// k-th bf16 of each of its RPL words, so the lane's values of a column are RPL
// consecutive codes of the transposed row: one store, and a lane group writes
// 128 contiguous bytes.  Column maxima: 16-bit integer maxima of the |bf16|
// bit patterns (ordered as the values), two columns per instruction, then
// across the lanes of a 128-row group (FP32 scales) or of a 32-row block (MX)
// by DPP.
// ---------------------------------------------------------------------------
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pkmax_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
template <int CTRL>
__device__ __forceinline__ uint32_t pkmax_dpp(uint32_t v) {
    return pkmax_u16(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false));
}
// maximum over aligned groups of N lanes (N = 2, 4, 8 or 16) by DPP
template <int N>
__device__ __forceinline__ uint32_t pkmax_lanes(uint32_t v) {
    constexpr int kQuadXor1 = 0xb1, kQuadXor2 = 0x4e, kHalfMirror = 0x141, kRowMirror = 0x140;
    v = pkmax_dpp<kQuadXor1>(v);
    if (N >= 4) v = pkmax_dpp<kQuadXor2>(v);
    if (N >= 8) v = pkmax_dpp<kHalfMirror>(v);
    if (N >= 16) v = pkmax_dpp<kRowMirror>(v);
    return v;
}
__device__ __forceinline__ uint32_t word_at(const uint4& w, int i) {
    return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
}

constexpr int kColTRows = 16;            // rows per lane (8 lanes x 16 bytes: whole 128-byte row pieces)
constexpr int kColTWaves = 2;            // waves per workgroup
constexpr int kColTCols = 8 * 64 / (128 / kColTRows);     // columns per wave
// Below this many workgroups (4 per CU) the LDS kernel is used.  Measured with
// inputs rotated past the last-level cache: 4096 x 9728 (2432 workgroups)
// 34.1 -> 30.2 us here; 4096 x 2560 (640) 12.0 us with LDS against 14.6 here.
constexpr int64_t kColTMinBlocks = 1024;

template <bool MX>
__global__ void __launch_bounds__(64 * kColTWaves) k_quant_col_t(const uint16_t* __restrict__ x, int32_t rows, int32_t cols,
                                                                 int64_t ld_x, uint8_t* __restrict__ qt, int64_t ld_qt,
                                                                 void* __restrict__ s, int64_t ssr, int64_t ssg) {
    constexpr int R = kColTRows, LPG = 128 / R;
    const int lane = threadIdx.x & 63;
    const int gi = lane / LPG, j = lane % LPG;
    const int32_t c = ((int32_t)blockIdx.x * kColTWaves + (int32_t)(threadIdx.x >> 6)) * kColTCols + 8 * gi;
    const int32_t rl = (int32_t)blockIdx.y * 128 + R * j;
    // cols % 8 == 0 and rows % 16 == 0 (% 32 for MX): a lane's block is
    // valid or empty, and so is each 32-row MX block
    const bool valid = c < cols && rl < rows;
    uint4 raw[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        raw[i] = make_uint4(0, 0, 0, 0);
        if (valid) raw[i] = *reinterpret_cast<const uint4*>(x + (int64_t)(rl + i) * ld_x + c);
    }
    uint32_t m[4] = {0u, 0u, 0u, 0u};      // |bf16| maxima, columns 2w (low half) and 2w + 1
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) m[w] = pkmax_u16(m[w], word_at(raw[i], w) & 0x7fff7fffu);
#pragma unroll
    for (int w = 0; w < 4; ++w) m[w] = MX ? pkmax_lanes<32 / R>(m[w]) : pkmax_lanes<LPG>(m[w]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t mw = m[k >> 1];
        const float amax = __uint_as_float((k & 1) ? (mw & 0xffff0000u) : (mw << 16));
        float v[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const uint32_t wd = word_at(raw[i], k >> 1);
            v[i] = (k & 1) ? bf16_hi(wd) : bf16_lo(wd);
        }
        uint32_t q[R / 4];
        if (!MX) {
            const float sc = amax / kE4M3Max;
#pragma unroll
            for (int i = 0; i < R / 8; ++i) encode8(&v[8 * i], sc, q[2 * i], q[2 * i + 1]);
            if (valid && j == 0) static_cast<float*>(s)[(int64_t)(c + k) * ssr + (int64_t)blockIdx.y * ssg] = sc;
        } else {
            const int e = mx_exponent(amax);
            const float f = pow2_neg(e);
#pragma unroll
            for (int i = 0; i < R / 4; ++i)
                q[i] = amax == 0.0f ? 0u : enc4(v[4 * i] * f, v[4 * i + 1] * f, v[4 * i + 2] * f, v[4 * i + 3] * f);
            if (valid && (rl & 31) == 0)
                static_cast<uint8_t*>(s)[(int64_t)(c + k) * ssr + (int64_t)(rl / 32) * ssg] = (uint8_t)(e + 127);
        }
        if (valid) {
            uint8_t* dst = qt + (int64_t)(c + k) * ld_qt + rl;
            if (R == 16) *reinterpret_cast<uint4*>(dst) = make_uint4(q[0], q[1], q[2], q[R / 4 - 1]);
            else *reinterpret_cast<uint2*>(dst) = make_uint2(q[0], q[1]);
        }
    }
}

// ---------------------------------------------------------------------------
// The same through LDS, for tensors too small to fill the chip with the
// kernel below (its 16-load, 128-value lanes then leave a long serial tail).
// Tile: 128 rows x 64 cols, staged in LDS as
// [column pair][row] words (a word is a bf16 pair of one row).  Thread t then
// owns column t/4 and rows 32*(t%4) .. +32 and writes those 32 contiguous
// codes of the transposed row.  128x1: the four threads of a column reduce
// the 128-row maximum with shuffles.  MX: each thread's 32 rows are one
// block.
// ---------------------------------------------------------------------------
template <bool MX>
__global__ void __launch_bounds__(kThreads) k_quant_col_t_lds(const uint16_t* __restrict__ x, int32_t rows, int32_t cols,
                                                          int64_t ld_x, uint8_t* __restrict__ qt, int64_t ld_qt,
                                                          void* __restrict__ s, int64_t ssr, int64_t ssg) {
    __shared__ __attribute__((aligned(16))) uint32_t tile[32][132];
    const int t = threadIdx.x;
    const int32_t r0 = (int32_t)blockIdx.y * 128;
    const int32_t c0 = (int32_t)blockIdx.x * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rl = (t >> 3) + 32 * i;
        const int cc = t & 7;
        const int32_t r = r0 + rl, c = c0 + cc * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < rows && c < cols) v = *reinterpret_cast<const uint4*>(x + (int64_t)r * ld_x + c);
        tile[cc * 4 + 0][rl] = v.x;
        tile[cc * 4 + 1][rl] = v.y;
        tile[cc * 4 + 2][rl] = v.z;
        tile[cc * 4 + 3][rl] = v.w;
    }
    __syncthreads();
    const int cl = t >> 2, rq = t & 3;
    const bool hi = (cl & 1) != 0;
    float v[32];
    const uint4* src = reinterpret_cast<const uint4*>(&tile[cl >> 1][rq * 32]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 w = src[i];
        v[4 * i + 0] = hi ? bf16_hi(w.x) : bf16_lo(w.x);
        v[4 * i + 1] = hi ? bf16_hi(w.y) : bf16_lo(w.y);
        v[4 * i + 2] = hi ? bf16_hi(w.z) : bf16_lo(w.z);
        v[4 * i + 3] = hi ? bf16_hi(w.w) : bf16_lo(w.w);
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
    uint32_t w[8];
    float sc = 0.0f;
    int e = 0;
    if (!MX) {
        m = group4_max(m);
        sc = m / kE4M3Max;
#pragma unroll
        for (int i = 0; i < 4; ++i) encode8(&v[8 * i], sc, w[2 * i], w[2 * i + 1]);
    } else {
        e = mx_exponent(m);
        const float f = pow2_neg(e);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            w[i] = m == 0.0f ? 0u : enc4(v[4 * i] * f, v[4 * i + 1] * f, v[4 * i + 2] * f, v[4 * i + 3] * f);
    }
    const int32_t c = c0 + cl;
    if (c < cols) {
        const int32_t rs = r0 + rq * 32;
        uint8_t* dst = qt + (int64_t)c * ld_qt + rs;
        if (rs < rows) *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        if (rs + 16 < rows) *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
        if (!MX) {
            if (rq == 0) static_cast<float*>(s)[(int64_t)c * ssr + (int64_t)blockIdx.y * ssg] = sc;
        } else if (rs < rows) {
            static_cast<uint8_t*>(s)[(int64_t)c * ssr + (int64_t)(blockIdx.y * 4 + rq) * ssg] = (uint8_t)(e + 127);
        }
    }
}

// ---------------------------------------------------------------------------
// Both groupings of one tensor from one read of it: 1x128 groups along rows
// (codes row-major) and 128x1 groups along columns (codes transposed), or,
// with MX, 1x32 and 32x1 blocks with UE8M0 scales.  An output gradient dY
// feeds the data-gradient GEMM through its row groups and the weight-gradient
// GEMM through its column groups; quantized here in one pass, the two share
// one HBM read of the bf16 tensor (2 bytes per element instead of 4).
// One workgroup per 128 x 128 tile; thread t holds rows 8 (t / 16) .. +7 and
// columns 8 (t % 16) .. +7 of it.
//   Row groups: the 16 lanes of a DPP row hold one tile row.  MX: the 1x32
//   maxima by lane shuffles, as in the row-group quantizer.  FP32: each lane
//   leaves its part of the row maximum in LDS, and after the barrier the
//   column groups need, threads 128..255 form one row's scale and reciprocal
//   each (not all 16 lanes of the row: two IEEE divisions saved per lane and
//   row); the row codes are encoded after the second barrier.
//   Column groups: per-lane maxima of the 8 rows (bf16 magnitudes, two per
//   word, as in the transposed quantizer), then over the wave's 4 row
//   phases, which make a 32x1 MX block; for 128x1 the 4 waves' maxima meet
//   in LDS, where threads 0..127 turn them into one scale and reciprocal per
//   column.  Column codes are packed along rows, so each lane writes 8
//   consecutive bytes of a transposed row.
// ---------------------------------------------------------------------------
template <bool MX>
__global__ void __launch_bounds__(kThreads) k_quant_dual(const uint16_t* __restrict__ x, int32_t rows, int32_t cols,
                                                         int64_t ld_x, uint8_t* __restrict__ q, int64_t ld_q,
                                                         void* __restrict__ s, int64_t ssr, int64_t ssg,
                                                         uint8_t* __restrict__ qt, int64_t ld_qt,
                                                         void* __restrict__ st, int64_t sstr, int64_t sstg) {
    __shared__ __attribute__((aligned(16))) uint4 red[MX ? 1 : 4][16];
    __shared__ float csc[MX ? 1 : 128], cyr[MX ? 1 : 128];
    __shared__ float rsc[MX ? 1 : 128], ryr[MX ? 1 : 128];          // FP32: row scales and reciprocals
    __shared__ __attribute__((aligned(16))) float rpart[MX ? 1 : 128][MX ? 1 : 16];   // FP32: per-lane row maxima
    __shared__ uint32_t cexp[MX ? 128 : 1];     // MX: the 4 row blocks' scale bytes of each column
    const int t = threadIdx.x;
    const int cc = t & 15, ph = t >> 4, wv = t >> 6;
    const int32_t r0 = (int32_t)blockIdx.x * 128, c0 = (int32_t)blockIdx.y * 128;
    const int32_t c = c0 + 8 * cc, rb = r0 + 8 * ph;
    // rows % 32 == 0 (MX) or % 16 == 0, cols % 32 == 0 (MX) or % 8 == 0: a
    // lane's 8 x 8 piece, and each 1x32 and 32x1 block, is whole or empty.
    const bool valid = c < cols && rb < rows;
    // MX scale bytes leave as one 4-byte word per row (its tile's 4 column
    // blocks) and per column (its 4 row blocks) where the tile is whole, the
    // 4 bytes are adjacent and the word is aligned; otherwise byte by byte.
    // (Single bytes from different lanes and waves, each its own partial
    // write of a scale row, cost a sixth of the kernel's time on dY.)
    const bool row_words = MX && c0 + 128 <= cols && ssg == 1 && ssr % 4 == 0 &&
                           (reinterpret_cast<uintptr_t>(s) & 3) == 0;
    const bool col_words = MX && r0 + 128 <= rows && sstg == 1 && sstr % 4 == 0 &&
                           (reinterpret_cast<uintptr_t>(st) & 3) == 0;
    uint4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        raw[i] = make_uint4(0, 0, 0, 0);
        if (valid) raw[i] = load_nt16(x + (int64_t)(rb + i) * ld_x + c);
    }
    // row groups
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float v[8];
        unpack8(raw[i], v);
        const int32_t r = rb + i;
        uint32_t w0, w1;
        if (!MX) {
            // FP32: the lane's part of the row maximum; the row's scale is
            // formed once, by one thread, below
            rpart[8 * ph + i][cc] = absmax8(v);
            continue;
        } else {
            const float amax = group4_max(absmax8(v));
            const int e = mx_exponent(amax);
            const float f = pow2_neg(e);
            if (amax == 0.0f) {
                w0 = 0u; w1 = 0u;
            } else {
                w0 = enc4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
                w1 = enc4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
            }
            const uint32_t sb = (uint32_t)(e + 127);
            if (row_words) {
                // lanes 4j of the row's 16 hold column block j
                const uint32_t wd = sb | ((uint32_t)__shfl((int)sb, 4, 16) << 8) |
                                    ((uint32_t)__shfl((int)sb, 8, 16) << 16) | ((uint32_t)__shfl((int)sb, 12, 16) << 24);
                if (rb < rows && cc == 0)
                    *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(s) + (int64_t)r * ssr + c0 / 32) = wd;
            } else if (valid && (cc & 3) == 0) {
                static_cast<uint8_t*>(s)[(int64_t)r * ssr + (int64_t)(c / 32) * ssg] = (uint8_t)sb;
            }
        }
        if (valid) *reinterpret_cast<uint2*>(q + (int64_t)r * ld_q + c) = make_uint2(w0, w1);
    }
    // column groups: maxima of |bf16| over the lane's rows, then the wave's
    uint32_t m[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) m[w] = pkmax_u16(m[w], word_at(raw[i], w) & 0x7fff7fffu);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        m[w] = pkmax_u16(m[w], (uint32_t)__shfl_xor((int)m[w], 16, 64));
        m[w] = pkmax_u16(m[w], (uint32_t)__shfl_xor((int)m[w], 32, 64));
    }
    float csv[8], cyv[8];
    if (!MX) {
        if ((t & 63) < 16) red[wv][cc] = make_uint4(m[0], m[1], m[2], m[3]);
        __syncthreads();
        if (t < 128) {
            const int j = t;                     // tile column
            uint32_t mw = 0u;
#pragma unroll
            for (int w = 0; w < 4; ++w) mw = pkmax_u16(mw, word_at(red[w][j >> 3], (j & 7) >> 1));
            const float amax = __uint_as_float((j & 1) ? (mw & 0xffff0000u) : (mw << 16));
            const float sc = amax / kE4M3Max;
            csc[j] = sc;
            cyr[j] = sc >= kFastDivMinScale ? 1.0f / sc : 0.0f;
            if (c0 + j < cols) static_cast<float*>(st)[(int64_t)(c0 + j) * sstr + (int64_t)blockIdx.x * sstg] = sc;
        } else {
            const int j = t - 128;               // tile row
            const float4* pr = reinterpret_cast<const float4*>(&rpart[j][0]);
            float amax = 0.0f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float4 w4 = pr[u];
                amax = fmaxf(amax, fmaxf(fmaxf(w4.x, w4.y), fmaxf(w4.z, w4.w)));
            }
            const float sc = amax / kE4M3Max;
            rsc[j] = sc;
            ryr[j] = sc >= kFastDivMinScale ? 1.0f / sc : 0.0f;
            if (r0 + j < rows) static_cast<float*>(s)[(int64_t)(r0 + j) * ssr + (int64_t)blockIdx.y * ssg] = sc;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 8; ++k) { csv[k] = csc[8 * cc + k]; cyv[k] = cyr[8 * cc + k]; }
        // row codes
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v[8];
            unpack8(raw[i], v);
            uint32_t w0, w1;
            encode8_y(v, rsc[8 * ph + i], ryr[8 * ph + i], w0, w1);
            if (valid) *reinterpret_cast<uint2*>(q + (int64_t)(rb + i) * ld_q + c) = make_uint2(w0, w1);
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t wd = word_at(raw[i], k >> 1);
            v[i] = (k & 1) ? bf16_hi(wd) : bf16_lo(wd);
        }
        uint32_t w0, w1;
        if (!MX) {
            encode8_y(v, csv[k], cyv[k], w0, w1);
        } else {
            const uint32_t mw = m[k >> 1];
            const float amax = __uint_as_float((k & 1) ? (mw & 0xffff0000u) : (mw << 16));
            const int e = mx_exponent(amax);
            const float f = pow2_neg(e);
            if (amax == 0.0f) {
                w0 = 0u; w1 = 0u;
            } else {
                w0 = enc4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
                w1 = enc4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
            }
            if ((t & 63) < 16) {
                if (col_words) reinterpret_cast<uint8_t*>(cexp)[(8 * cc + k) * 4 + wv] = (uint8_t)(e + 127);
                else if (valid)
                    static_cast<uint8_t*>(st)[(int64_t)(c + k) * sstr + (int64_t)(rb / 32) * sstg] = (uint8_t)(e + 127);
            }
        }
        if (valid) *reinterpret_cast<uint2*>(qt + (int64_t)(c + k) * ld_qt + rb) = make_uint2(w0, w1);
    }
    if (col_words) {
        __syncthreads();
        if (t < 128 && c0 + t < cols)
            *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(st) + (int64_t)(c0 + t) * sstr + r0 / 32) = cexp[t];
    }
}

// ---------------------------------------------------------------------------
// 128x128 block quantizer, one workgroup per block, one HBM read of the
// block.  Optional transposed copy: the block's codes are staged in LDS and
// re-read as 4x4 byte squares that are transposed in registers (v_perm).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void transpose4x4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t o[4]) {
    // byte i of __builtin_amdgcn_perm(a, b, sel) is byte sel_i of {a:b}
    // (selectors 0-3 pick b's bytes, 4-7 pick a's bytes).
    const uint32_t lo01 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
    const uint32_t hi01 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
    const uint32_t lo23 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
    o[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// P2: power-of-two scale (MX exponent rule on the block's amax) stored as a
// UE8M0 byte, codes E4M3(x * 2^-e); s is then uint8 with row stride lds.
// Block (bx, by) of matrix bz; the body takes the block coordinates as
// arguments so that the fused linear-operand kernel can run it.
template <bool TRANS, bool NT, bool P2>
__device__ __forceinline__ void block2d_body(const uint16_t* __restrict__ w, int32_t rows, int32_t cols, int64_t ld_w,
                                             uint8_t* __restrict__ q, int64_t ld_q, uint8_t* __restrict__ qt,
                                             int64_t ld_qt, void* __restrict__ s, int32_t nbr, int32_t lds, int32_t bx,
                                             int32_t by, int32_t bz) {
    __shared__ float red[kThreads / 64];
    __shared__ __attribute__((aligned(16))) uint32_t ctile[TRANS ? 128 : 1][33];
    const int t = threadIdx.x;
    const bool wq = q != nullptr;         // TRANS: the row-major codes may be skipped
    w += bz * (int64_t)rows * ld_w;
    if (wq) q += bz * (int64_t)rows * ld_q;
    if (TRANS) qt += bz * (int64_t)cols * ld_qt;
    const int64_t s_idx = bz * (int64_t)nbr * lds + (int64_t)by * lds + bx;
    const int32_t r0 = by * 128, c0 = bx * 128;
    const int cc = t & 15;
    uint4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int32_t r = r0 + (t >> 4) + 16 * i, c = c0 + cc * 8;
        raw[i] = make_uint4(0, 0, 0, 0);
        if (r < rows && c < cols) {
            const uint16_t* src = w + (int64_t)r * ld_w + c;
            raw[i] = NT ? load_nt16(src) : *reinterpret_cast<const uint4*>(src);
        }
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float v[8];
        unpack8(raw[i], v);
        m = fmaxf(m, absmax8(v));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = m / kE4M3Max;
    const int e = P2 ? mx_exponent(m) : 0;
    const float f = P2 ? pow2_neg(e) : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float v[8];
        unpack8(raw[i], v);
        uint32_t w0, w1;
        if (!P2) {
            encode8(v, sc, w0, w1);
        } else if (m == 0.0f) {
            w0 = 0u; w1 = 0u;
        } else {
            w0 = enc4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
            w1 = enc4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
        }
        const int rl = (t >> 4) + 16 * i;
        const int32_t r = r0 + rl, c = c0 + cc * 8;
        if (wq && r < rows && c < cols) {
            uint8_t* dst = q + (int64_t)r * ld_q + c;
            if (NT) store_nt8(dst, w0, w1);
            else *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
        }
        if (TRANS) { ctile[rl][2 * cc] = w0; ctile[rl][2 * cc + 1] = w1; }
    }
    if (t == 0) {
        if (P2) static_cast<uint8_t*>(s)[s_idx] = (uint8_t)(e + 127);
        else static_cast<float*>(s)[s_idx] = sc;
    }
    if (TRANS) {
        __syncthreads();
        // thread -> 4 columns (cb) x 16 rows (rb); 8 consecutive lanes cover one
        // 128-byte row segment of the transposed output.
        const int rb = t & 7, cb = t >> 3;
        uint32_t col[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = rb * 16 + 4 * j;
            uint32_t o[4];
            transpose4x4(ctile[rr][cb], ctile[rr + 1][cb], ctile[rr + 2][cb], ctile[rr + 3][cb], o);
#pragma unroll
            for (int k = 0; k < 4; ++k) col[k][j] = o[k];
        }
        const int32_t rs = r0 + rb * 16;
        if (rs < rows) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int32_t c = c0 + cb * 4 + k;
                if (c < cols) {
                    uint8_t* dst = qt + (int64_t)c * ld_qt + rs;
                    const uint4 v = make_uint4(col[k][0], col[k][1], col[k][2], col[k][3]);
                    if (NT) store_nt16(dst, v);
                    else *reinterpret_cast<uint4*>(dst) = v;
                }
            }
        }
    }
}

template <bool TRANS, bool NT, bool P2>
__global__ void __launch_bounds__(kThreads) k_quant_128x128(const uint16_t* __restrict__ w, int32_t rows, int32_t cols,
                                                            int64_t ld_w, uint8_t* __restrict__ q, int64_t ld_q,
                                                            uint8_t* __restrict__ qt, int64_t ld_qt,
                                                            void* __restrict__ s, int32_t nbr, int32_t lds) {
    block2d_body<TRANS, NT, P2>(w, rows, cols, ld_w, q, ld_q, qt, ld_qt, s, nbr, lds, (int32_t)blockIdx.x,
                                (int32_t)blockIdx.y, (int32_t)blockIdx.z);
}

// ---------------------------------------------------------------------------
// Transpose of E4M3 codes, one workgroup per 128 x 128 tile of matrix bz: the
// tile's rows are staged in LDS as words and re-read as 4x4 byte squares,
// transposed in registers (as for the quantizer's transposed copy).  The
// backward pass of a layer whose weight the forward quantized in 128 x 128
// blocks gets W's transposed operand from the forward's codes this way (the
// block scales are the same, read with swapped strides), without reading
// the bf16 weight again.  rows % 16 == 0 and cols % 16 == 0: every 16-byte
// piece is whole or absent.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_transpose_codes(const uint8_t* __restrict__ q, int32_t rows,
                                                              int32_t cols, int64_t ld_q, uint8_t* __restrict__ qt,
                                                              int64_t ld_qt) {
    __shared__ __attribute__((aligned(16))) uint32_t ctile[128][33];
    const int t = threadIdx.x;
    const int64_t bz = blockIdx.z;
    q += bz * (int64_t)rows * ld_q;
    qt += bz * (int64_t)cols * ld_qt;
    const int32_t r0 = (int32_t)blockIdx.y * 128, c0 = (int32_t)blockIdx.x * 128;
    // thread t: 16-byte piece t % 8 of rows t / 8 + 32 i
    const int cp = t & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rl = (t >> 3) + 32 * i;
        const int32_t r = r0 + rl, c = c0 + 16 * cp;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < rows && c < cols) v = *reinterpret_cast<const uint4*>(q + (int64_t)r * ld_q + c);
        ctile[rl][4 * cp] = v.x;
        ctile[rl][4 * cp + 1] = v.y;
        ctile[rl][4 * cp + 2] = v.z;
        ctile[rl][4 * cp + 3] = v.w;
    }
    __syncthreads();
    // thread -> 4 columns (cb) x 16 rows (rb); 8 consecutive lanes cover one
    // 128-byte piece of a transposed row
    const int rb = t & 7, cb = t >> 3;
    uint32_t col[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int rr = rb * 16 + 4 * j;
        uint32_t o[4];
        transpose4x4(ctile[rr][cb], ctile[rr + 1][cb], ctile[rr + 2][cb], ctile[rr + 3][cb], o);
#pragma unroll
        for (int k = 0; k < 4; ++k) col[k][j] = o[k];
    }
    const int32_t rs = r0 + rb * 16;
    if (rs < rows) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int32_t c = c0 + cb * 4 + k;
            if (c < cols)
                *reinterpret_cast<uint4*>(qt + (int64_t)c * ld_qt + rs) =
                    make_uint4(col[k][0], col[k][1], col[k][2], col[k][3]);
        }
    }
}

// The two operands of one linear layer in one launch: workgroups [0, w_blocks)
// quantize 128 x 128 blocks of the weight W (row-major block order), the rest
// run the 1x128 row-group quantizer over the activation X.  Both parts are
// HBM-bound; in one grid their loads are in flight together, and the step
// saves a launch, its ramp-up and its tail.
struct LinearArgs {
    RowArgs x;
    int32_t x_blocks;
    const uint16_t* w; int32_t w_rows, cols; int64_t ld_w;
    uint8_t* qw; int64_t ld_qw; void* sw;
    int32_t nbr, nbc, lds_w, w_blocks;      // lds_w: row stride of W's block scales
};

// P2: power-of-two scales (UE8M0 bytes) for both operands, as fp8_quant_pow2.
template <bool ROW_FAST, bool P2 = false>
__global__ void __launch_bounds__(kThreads) k_quant_linear(LinearArgs a) {
    const int32_t b = (int32_t)blockIdx.x;
    // W blocks and X workgroups dealt in proportion (workgroup b is a W block
    // when floor((b + 1) W / n) > floor(b W / n)), so that the heavier W
    // blocks do not all run first: 1-2% faster than W first on the MLP
    // operand pairs
    const int64_t n = (int64_t)a.w_blocks + a.x_blocks;
    const int32_t wb = (int32_t)((int64_t)b * a.w_blocks / n);
    if ((int32_t)(((int64_t)b + 1) * a.w_blocks / n) > wb)
        block2d_body<false, false, P2>(a.w, a.w_rows, a.cols, a.ld_w, a.qw, a.ld_qw, nullptr, 0, a.sw, a.nbr, a.lds_w,
                                       wb % a.nbc, wb / a.nbc, 0);
    else
        rowgroup_body<false, false, ROW_FAST, 4, false, P2>(a.x, b - wb, a.x_blocks);
}

__global__ void __launch_bounds__(kThreads) k_e4m3_encode(const float* __restrict__ in, uint8_t* __restrict__ out,
                                                          int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (i + 4 <= n) {
        const uint32_t w = enc4(in[i], in[i + 1], in[i + 2], in[i + 3]);
        out[i] = (uint8_t)w; out[i + 1] = (uint8_t)(w >> 8); out[i + 2] = (uint8_t)(w >> 16); out[i + 3] = (uint8_t)(w >> 24);
    } else {
        for (int64_t j = i; j < n; ++j) out[j] = (uint8_t)enc4(in[j], 0.f, 0.f, 0.f);
    }
}

// ---------------------------------------------------------------------------
// Rowwise and tensorwise scaling: one group per row or per tensor (the same
// two steps).  Rowwise: one workgroup per row; the maximum is reduced over
// the row's 16-byte chunks, then the chunks are read again (from L2) and
// encoded.  Tensorwise: a fill kernel zeroes s[0], every workgroup folds its
// chunk maximum into s[0] with an atomic max on the fp32 bits (non-negative
// floats order like their bit patterns), the encode kernel reads the maximum,
// and a last one-thread kernel replaces it by the scale max / 448.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_max(float m, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, red[i]);
    return m;
}

// Rows of at most 64 R chunks of 8 values: one wave per row (4 rows per
// workgroup) and the row held in registers: R loads per lane issued
// together, the maximum by wave shuffles, then the codes from the registers.
// No LDS, no barrier, one HBM read.
template <int R>
__global__ void __launch_bounds__(kThreads) k_quant_rowwise_wave(const uint16_t* __restrict__ x, int32_t rows,
                                                                 int32_t cols, int64_t ld_x, uint8_t* __restrict__ q,
                                                                 int64_t ld_q, float* __restrict__ s) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (r >= rows) return;                  // whole waves: nothing below needs other waves
    const uint16_t* xr = x + r * ld_x;
    uint8_t* qr = q + r * ld_q;
    const int nch = cols / 8;
    uint4 raw[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int c = lane + 64 * i;
        raw[i] = make_uint4(0, 0, 0, 0);
        if (c < nch) raw[i] = *reinterpret_cast<const uint4*>(xr + 8 * c);
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        float v[8];
        unpack8(raw[i], v);
        m = fmaxf(m, absmax8(v));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float sc = m / kE4M3Max;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
            float v[8];
            unpack8(raw[i], v);
            uint32_t w0, w1;
            encode8(v, sc, w0, w1);
            *reinterpret_cast<uint2*>(qr + 8 * c) = make_uint2(w0, w1);
        }
    }
    if (lane == 0) s[r] = sc;
}

// Longer rows: one workgroup per row, two passes over the row (the second
// served by the cache).
__global__ void __launch_bounds__(kThreads) k_quant_rowwise(const uint16_t* __restrict__ x, int32_t cols, int64_t ld_x,
                                                            uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ s) {
    __shared__ float red[kThreads / 64];
    const int64_t r = blockIdx.x;
    const uint16_t* xr = x + r * ld_x;
    uint8_t* qr = q + r * ld_q;
    const int nch = cols / 8;
    float m = 0.0f;
    for (int c = threadIdx.x; c < nch; c += kThreads) {
        float v[8];
        unpack8(*reinterpret_cast<const uint4*>(xr + 8 * c), v);
        m = fmaxf(m, absmax8(v));
    }
    m = block_max(m, red);
    const float sc = m / kE4M3Max;
    for (int c = threadIdx.x; c < nch; c += kThreads) {
        float v[8];
        unpack8(*reinterpret_cast<const uint4*>(xr + 8 * c), v);
        uint32_t w0, w1;
        encode8(v, sc, w0, w1);
        *reinterpret_cast<uint2*>(qr + 8 * c) = make_uint2(w0, w1);
    }
    if (threadIdx.x == 0) s[r] = sc;
}

__global__ void k_fill_zero(float* s) { s[0] = 0.0f; }

// WIDE: chunk indices past 2^32 (64-bit division per chunk; 32-bit otherwise)
template <bool WIDE>
__global__ void __launch_bounds__(kThreads) k_tensor_amax(const uint16_t* __restrict__ x, int32_t rows, int32_t cols,
                                                          int64_t ld_x, float* s) {
    // each thread takes 8 chunks of 8 values per trip, all loads issued
    // before the maxima; few workgroups (one atomic each on the scale cell)
    constexpr int U = 8;
    __shared__ float red[kThreads / 64];
    const uint32_t nch = (uint32_t)cols / 8;
    const int64_t total = (int64_t)rows * nch;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    float m = 0.0f;
    for (int64_t base = (int64_t)blockIdx.x * kThreads + threadIdx.x; base < total; base += stride * U) {
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * stride;
            raw[u] = make_uint4(0, 0, 0, 0);
            if (i < total) {
                int64_t r, c;
                if (WIDE) { r = i / nch; c = i - r * nch; }
                else { const uint32_t i32 = (uint32_t)i, r32 = i32 / nch; r = r32; c = i32 - r32 * nch; }
                raw[u] = *reinterpret_cast<const uint4*>(x + r * ld_x + 8 * c);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v[8];
            unpack8(raw[u], v);
            m = fmaxf(m, absmax8(v));
        }
    }
    m = block_max(m, red);
    // fl(m / 448) is monotone in m, so the maximum of the blocks' scales is
    // the scale of the tensor's amax; non-negative floats order as their bits
    if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned int*>(s), __float_as_uint(m / kE4M3Max));
}
__global__ void __launch_bounds__(kThreads) k_tensor_encode(const uint16_t* __restrict__ x, int32_t rows, int32_t cols,
                                                            int64_t ld_x, uint8_t* __restrict__ q, int64_t ld_q,
                                                            const float* s) {
    const float sc = s[0];
    const int nch = cols / 8;
    const int64_t total = (int64_t)rows * nch;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
        const int64_t r = i / nch, c = i - r * nch;
        float v[8];
        unpack8(*reinterpret_cast<const uint4*>(x + r * ld_x + 8 * c), v);
        uint32_t w0, w1;
        encode8(v, sc, w0, w1);
        *reinterpret_cast<uint2*>(q + r * ld_q + 8 * c) = make_uint2(w0, w1);
    }
}


}  // namespace

hipError_t launch_quant_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                              float* s, int64_t ssr, int64_t ssg, hipStream_t st) {
    RowArgs p{};
    p.x = x; p.ld_x = ld_x; p.rows = (int32_t)rows; p.cols = (int32_t)cols; p.up_off = 0;
    p.q = q; p.ld_q = ld_q; p.s = s; p.ssr = ssr; p.ssg = ssg; p.h = nullptr; p.ld_h = 0;
    p.runs_per_row = (int32_t)((cols + 127) / 128);
    p.total_runs = (int32_t)(rows * p.runs_per_row);
    return launch_rowgroup<false, false>(p, ssr == 1 && ssg != 1, st);
}

hipError_t launch_mx_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                           uint8_t* s, int64_t ssr, int64_t ssg, hipStream_t st) {
    RowArgs p{};
    p.x = x; p.ld_x = ld_x; p.rows = (int32_t)rows; p.cols = (int32_t)cols; p.up_off = 0;
    p.q = q; p.ld_q = ld_q; p.s = s; p.ssr = ssr; p.ssg = ssg; p.h = nullptr; p.ld_h = 0;
    p.runs_per_row = (int32_t)((cols + 127) / 128);
    p.total_runs = (int32_t)(rows * p.runs_per_row);
    return launch_rowgroup<false, true>(p, ssr == 1 && ssg != 1, st);
}

hipError_t launch_silu_mul_quant(const uint16_t* gu, int64_t rows, int64_t I, int64_t ld_in, int mx, uint8_t* q,
                                 int64_t ld_q, void* s, int64_t ssr, int64_t ssg, uint16_t* h, int64_t ld_h,
                                 hipStream_t st) {
    RowArgs p{};
    p.x = gu; p.ld_x = ld_in; p.rows = (int32_t)rows; p.cols = (int32_t)I; p.up_off = I;
    p.q = q; p.ld_q = ld_q; p.s = s; p.ssr = ssr; p.ssg = ssg; p.h = h; p.ld_h = ld_h;
    p.runs_per_row = (int32_t)((I + 127) / 128);
    p.total_runs = (int32_t)(rows * p.runs_per_row);
    const bool rf = ssr == 1 && ssg != 1;
    return mx ? launch_rowgroup<true, true>(p, rf, st) : launch_rowgroup<true, false>(p, rf, st);
}

hipError_t launch_quant_128x1_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qt,
                                int64_t ld_qt, float* s, int64_t ssr, int64_t ssg, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const unsigned gy = (unsigned)((rows + 127) / 128);
    const unsigned gx = (unsigned)((cols + kColTCols * kColTWaves - 1) / (kColTCols * kColTWaves));
    if ((int64_t)gx * gy >= kColTMinBlocks)
        hipLaunchKernelGGL(k_quant_col_t<false>, dim3(gx, gy), dim3(64 * kColTWaves), 0, st, x, (int32_t)rows,
                           (int32_t)cols, ld_x, qt, ld_qt, (void*)s, ssr, ssg);
    else
        hipLaunchKernelGGL(k_quant_col_t_lds<false>, dim3((unsigned)((cols + 63) / 64), gy), dim3(kThreads), 0, st, x,
                           (int32_t)rows, (int32_t)cols, ld_x, qt, ld_qt, (void*)s, ssr, ssg);
    return hipGetLastError();
}

hipError_t launch_mx_quant_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qt, int64_t ld_qt,
                             uint8_t* s, int64_t ssr, int64_t ssg, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const unsigned gy = (unsigned)((rows + 127) / 128);
    const unsigned gx = (unsigned)((cols + kColTCols * kColTWaves - 1) / (kColTCols * kColTWaves));
    if ((int64_t)gx * gy >= kColTMinBlocks)
        hipLaunchKernelGGL(k_quant_col_t<true>, dim3(gx, gy), dim3(64 * kColTWaves), 0, st, x, (int32_t)rows,
                           (int32_t)cols, ld_x, qt, ld_qt, (void*)s, ssr, ssg);
    else
        hipLaunchKernelGGL(k_quant_col_t_lds<true>, dim3((unsigned)((cols + 63) / 64), gy), dim3(kThreads), 0, st, x,
                           (int32_t)rows, (int32_t)cols, ld_x, qt, ld_qt, (void*)s, ssr, ssg);
    return hipGetLastError();
}

hipError_t launch_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, bool mx, uint8_t* q,
                             int64_t ld_q, void* s, int64_t ssr, int64_t ssg, uint8_t* qt, int64_t ld_qt, void* st,
                             int64_t sstr, int64_t sstg, hipStream_t stream) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 127) / 128), (unsigned)((cols + 127) / 128));
    if (mx)
        hipLaunchKernelGGL(k_quant_dual<true>, grid, dim3(kThreads), 0, stream, x, (int32_t)rows, (int32_t)cols, ld_x,
                           q, ld_q, s, ssr, ssg, qt, ld_qt, st, sstr, sstg);
    else
        hipLaunchKernelGGL(k_quant_dual<false>, grid, dim3(kThreads), 0, stream, x, (int32_t)rows, (int32_t)cols, ld_x,
                           q, ld_q, s, ssr, ssg, qt, ld_qt, st, sstr, sstg);
    return hipGetLastError();
}

hipError_t launch_quant_128x128(const uint16_t* w, int64_t batch, int64_t rows, int64_t cols, int64_t ld_w,
                                uint8_t* q, int64_t ld_q, uint8_t* qt, int64_t ld_qt, float* s, hipStream_t st) {
    if (rows == 0 || cols == 0 || batch == 0) return hipSuccess;
    const int32_t nbr = (int32_t)((rows + 127) / 128), nbc = (int32_t)((cols + 127) / 128);
    dim3 grid((unsigned)nbc, (unsigned)nbr, (unsigned)batch);
    // Weights larger than the 256 MB last-level cache (the MoE expert stacks)
    // stream through it with the nt policy: their codes cannot stay cached for
    // the GEMM anyway.  Smaller weights keep the default policy (the nt loads
    // lost on them, and their codes should stay cached for the GEMM).
    const bool nt = batch * rows * cols * 2 > ((int64_t)256 << 20);
    auto go = [&](auto trans, auto ntt) {
        hipLaunchKernelGGL((k_quant_128x128<decltype(trans)::value, decltype(ntt)::value, false>), grid, dim3(kThreads),
                           0, st, w, (int32_t)rows, (int32_t)cols, ld_w, q, ld_q, qt, ld_qt, (void*)s, nbr, nbc);
    };
    if (qt) {
        if (nt) go(std::true_type{}, std::true_type{});
        else go(std::true_type{}, std::false_type{});
    } else {
        if (nt) go(std::false_type{}, std::true_type{});
        else go(std::false_type{}, std::false_type{});
    }
    return hipGetLastError();
}

hipError_t launch_transpose_codes(const uint8_t* q, int64_t batch, int64_t rows, int64_t cols, int64_t ld_q,
                                  uint8_t* qt, int64_t ld_qt, hipStream_t st) {
    if (rows == 0 || cols == 0 || batch == 0) return hipSuccess;
    const dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128), (unsigned)batch);
    hipLaunchKernelGGL(k_transpose_codes, grid, dim3(kThreads), 0, st, q, (int32_t)rows, (int32_t)cols, ld_q, qt,
                       ld_qt);
    return hipGetLastError();
}

static hipError_t launch_linear_pair(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qx,
                                     int64_t ld_qx, void* sx, int64_t ssr, int64_t ssg, const uint16_t* w,
                                     int64_t w_rows, int64_t ld_w, uint8_t* qw, int64_t ld_qw, void* sw,
                                     int64_t lds_w, bool p2, hipStream_t st) {
    LinearArgs a{};
    RowArgs& p = a.x;
    p.x = x; p.ld_x = ld_x; p.rows = (int32_t)rows; p.cols = (int32_t)cols; p.up_off = 0;
    p.q = qx; p.ld_q = ld_qx; p.s = sx; p.ssr = ssr; p.ssg = ssg; p.h = nullptr; p.ld_h = 0;
    p.runs_per_row = (int32_t)((cols + 127) / 128);
    p.total_runs = (int32_t)(rows * p.runs_per_row);
    // one trip per 16-lane row, four runs per trip: unlike the separate
    // 1x128 launch (two), here two ran the down projection's pair 40 -> 46 us
    // (more activation workgroups beside the weight blocks); six and eight
    // were 1-7% slower than four on both pairs
    constexpr int U = 4;
    const int64_t rows16 = ((int64_t)p.total_runs + U - 1) / U;
    int64_t xb = (rows16 + (kThreads / 16) - 1) / (kThreads / 16);
    if (xb > 256 * 256) xb = 256 * 256;
    a.x_blocks = (int32_t)xb;
    a.w = w; a.w_rows = (int32_t)w_rows; a.cols = (int32_t)cols; a.ld_w = ld_w;
    a.qw = qw; a.ld_qw = ld_qw; a.sw = sw;
    a.nbr = (int32_t)((w_rows + 127) / 128);
    a.nbc = (int32_t)((cols + 127) / 128);
    a.lds_w = (int32_t)lds_w;
    a.w_blocks = a.nbr * a.nbc;
    const dim3 grid((unsigned)(a.w_blocks + a.x_blocks));
    if (p2)
        hipLaunchKernelGGL((k_quant_linear<false, true>), grid, dim3(kThreads), 0, st, a);
    else if (ssr == 1 && ssg != 1)
        hipLaunchKernelGGL(k_quant_linear<true>, grid, dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_quant_linear<false>, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

// Tensors past the 256 MB last-level cache take the streaming policies of
// the separate kernels; the fused kernel serves the cached sizes.
static bool linear_pair_fits(int64_t rows, int64_t w_rows, int64_t cols) {
    const bool big = rows * cols > ((int64_t)256 << 20) || w_rows * cols * 2 > ((int64_t)256 << 20);
    return !big && rows > 0 && w_rows > 0 && cols > 0;
}

hipError_t launch_quant_linear(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qx, int64_t ld_qx,
                               float* sx, int64_t ssr, int64_t ssg, const uint16_t* w, int64_t w_rows, int64_t ld_w,
                               uint8_t* qw, int64_t ld_qw, float* sw, hipStream_t st) {
    if (!linear_pair_fits(rows, w_rows, cols)) {
        hipError_t e = launch_quant_128x128(w, 1, w_rows, cols, ld_w, qw, ld_qw, nullptr, 0, sw, st);
        if (e != hipSuccess) return e;
        return launch_quant_1x128(x, rows, cols, ld_x, qx, ld_qx, sx, ssr, ssg, st);
    }
    return launch_linear_pair(x, rows, cols, ld_x, qx, ld_qx, sx, ssr, ssg, w, w_rows, ld_w, qw, ld_qw, sw,
                              (cols + 127) / 128, false, st);
}

hipError_t launch_quant_linear_pow2(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qx,
                                    int64_t ld_qx, uint8_t* sx, int64_t ld_sx, const uint16_t* w, int64_t w_rows,
                                    int64_t ld_w, uint8_t* qw, int64_t ld_qw, uint8_t* sw, int64_t ld_sw,
                                    hipStream_t st) {
    if (!linear_pair_fits(rows, w_rows, cols)) {
        hipError_t e = launch_quant_pow2(w, w_rows, cols, ld_w, 128, qw, ld_qw, sw, ld_sw, st);
        if (e != hipSuccess) return e;
        return launch_quant_pow2(x, rows, cols, ld_x, 1, qx, ld_qx, sx, ld_sx, st);
    }
    return launch_linear_pair(x, rows, cols, ld_x, qx, ld_qx, sx, ld_sx, 1, w, w_rows, ld_w, qw, ld_qw, sw, ld_sw, true,
                              st);
}

hipError_t launch_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                                float* s, hipStream_t st) {
    if (rows == 0) return hipSuccess;                 // cols == 0: every scale 0
    const int64_t nch = cols / 8;
    const dim3 wgrid((unsigned)((rows + kThreads / 64 - 1) / (kThreads / 64)));
    auto wave = [&](auto kern) {
        hipLaunchKernelGGL(kern, wgrid, dim3(kThreads), 0, st, x, (int32_t)rows, (int32_t)cols, ld_x, q, ld_q, s);
    };
    if (nch <= 64 * 2) wave(k_quant_rowwise_wave<2>);
    else if (nch <= 64 * 4) wave(k_quant_rowwise_wave<4>);
    else if (nch <= 64 * 8) wave(k_quant_rowwise_wave<8>);
    else if (nch <= 64 * 16) wave(k_quant_rowwise_wave<16>);
    else hipLaunchKernelGGL(k_quant_rowwise, dim3((unsigned)rows), dim3(kThreads), 0, st, x, (int32_t)cols, ld_x, q, ld_q, s);
    return hipGetLastError();
}

hipError_t launch_quant_tensorwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                                   int64_t ld_q, float* s, hipStream_t st) {
    if (rows == 0 || cols == 0) {
        hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(1), 0, st, s);
        return hipGetLastError();
    }
    const int64_t chunks = rows * (cols / 8);
    int64_t blocks = (chunks + kThreads * 8 - 1) / (kThreads * 8);
    // one workgroup per CU at most, each ending in one atomic on the scale
    // cell: against 512 (and 2048) workgroups, X_up 22.8 -> 20.4 us, W_up
    // 34.0 -> 33.4 us, 4096 x 9728 unchanged; 128 lost on the larger tensors
    if (blocks > 256) blocks = 256;
    hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(1), 0, st, s);
    // 32-bit chunk indices when every index of the grid-stride loop fits
    if (chunks + (int64_t)blocks * kThreads * 8 < ((int64_t)1 << 32))
        hipLaunchKernelGGL(k_tensor_amax<false>, dim3((unsigned)blocks), dim3(kThreads), 0, st, x, (int32_t)rows,
                           (int32_t)cols, ld_x, s);
    else
        hipLaunchKernelGGL(k_tensor_amax<true>, dim3((unsigned)blocks), dim3(kThreads), 0, st, x, (int32_t)rows,
                           (int32_t)cols, ld_x, s);
    int64_t eblocks = (chunks + kThreads - 1) / kThreads;
    if (eblocks > 256 * 64) eblocks = 256 * 64;
    hipLaunchKernelGGL(k_tensor_encode, dim3((unsigned)eblocks), dim3(kThreads), 0, st, x, (int32_t)rows, (int32_t)cols,
                       ld_x, q, ld_q, (const float*)s);
    return hipGetLastError();
}

hipError_t launch_quant_pow2(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int block_rows, uint8_t* q,
                             int64_t ld_q, uint8_t* s, int64_t ld_s, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    if (block_rows == 1) {
        RowArgs p{};
        p.x = x; p.ld_x = ld_x; p.rows = (int32_t)rows; p.cols = (int32_t)cols; p.up_off = 0;
        p.q = q; p.ld_q = ld_q; p.s = s; p.ssr = ld_s; p.ssg = 1; p.h = nullptr; p.ld_h = 0;
        p.runs_per_row = (int32_t)((cols + 127) / 128);
        p.total_runs = (int32_t)(rows * p.runs_per_row);
        return launch_rowgroup<false, false, true>(p, false, st);
    }
    const int32_t nbr = (int32_t)((rows + 127) / 128), nbc = (int32_t)((cols + 127) / 128);
    hipLaunchKernelGGL((k_quant_128x128<false, false, true>), dim3((unsigned)nbc, (unsigned)nbr, 1u), dim3(kThreads), 0,
                       st, x, (int32_t)rows, (int32_t)cols, ld_x, q, ld_q, (uint8_t*)nullptr, (int64_t)0, (void*)s, nbr,
                       (int32_t)ld_s);
    return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const int64_t blocks = (n + 4 * kThreads - 1) / (4 * kThreads);
    hipLaunchKernelGGL(k_e4m3_encode, dim3((unsigned)blocks), dim3(kThreads), 0, st, in, out, n);
    return hipGetLastError();
}

}  // namespace fp8bs
