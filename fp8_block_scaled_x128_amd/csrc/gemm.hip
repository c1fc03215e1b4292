// Block-scaled FP8 GEMMs of libfp8bs (gfx950): dense, grouped (MoE experts)
// and MXFP8.
//
//   C[m, n] = sum_kb sa(m, kb) sb(n, kb) * sum_{k in kb} dec(a[m, k]) dec(b[n, k])
//
// The scale product of each 128-wide K slice multiplies the FP32 partial of
// that slice, so the two FP32 scales per slice are applied exactly as the
// block-wise recipe defines them ("Low Precision RL", section "2. Unified
// block-wise FP8 (DeepSeek-style)": 128x128 weight blocks, FP32 scales;
// per-token activation groups from "Unified FP8: Beyond Mixed Precision...",
// section "FP8 Quantization").  The MXFP8 variant ("Low Precision RL",
// section "3. Unified MXFP8 (Blackwell)") hands its power-of-two block scales
// to the scaled matrix instruction, which applies them exactly.
//
// Kernel structure: one workgroup of 4 waves (one per SIMD, so each wave has
// the full 512-entry VGPR+AGPR budget) per output tile of 256 weight rows (n)
// x 128 activation rows (m).
//  - K advances in 128-byte slices.  Each slice of the weight tile (32 KB),
//    the activation tile (16 KB) and the slice's scales is copied straight
//    from global memory into LDS with global_load_lds (no register staging),
//    three stages deep, so two slices are in flight while one is consumed.
//  - LDS rows are 128 bytes; 16-byte chunk c of row r sits in slot
//    c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1): 16 consecutive rows reading
//    the same logical chunk hit 16 distinct 16-byte bank groups.  The copy
//    realizes the swizzle by choosing which global chunk each lane fetches.
//  - Wave w owns n rows [128 * (w >> 1), +128) and m rows [64 * (w & 1), +64):
//    8 x 4 tiles of v_mfma_scale_f32_16x16x128_f8f6f4 per slice.  Weight rows
//    are the instruction's A operand and activation rows its B operand, so a
//    lane's 4 outputs share one activation row m and four consecutive n.
//  - FP32-scale modes: each MFMA produces a fresh FP32 partial for its slice
//    (zero accumulator input, unit E8M0 scales), promoted with one FMA per
//    output, acc = fma(partial, sa * sb, acc), one n-tile behind the MFMAs so
//    that the promotion overlaps the next n-tile's matrix work.
//  - MX mode: the instruction accumulates in place with the per-lane UE8M0
//    scale bytes of its row and 32-wide K block.
#include "device_common.h"
#include "internal.h"

namespace fp8bs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BN = 256, BK = 128;              // weight rows per tile, K bytes per slice
constexpr int kE8M0One = 127;                  // UE8M0 code of 1.0

// Tile configurations.  Every wave computes 128 weight rows x 64 activation
// rows; waves are arranged 2 (n) x WAVES/2 (m).
//   WAVES = 4: 256 x 128 tile, one wave per SIMD (512 registers each), three
//              LDS stages, promotion deferred by one n-tile within the wave.
//   WAVES = 8: 256 x 256 tile, two waves per SIMD (256 registers each) whose
//              matrix and vector work interleave, two LDS stages.
template <int WAVES>
struct Cfg {
    static constexpr int kWaves = WAVES;
    static constexpr int kThreads = WAVES * 64;
    static constexpr int BM = 64 * (WAVES / 2);
    static constexpr int kStages = WAVES == 4 ? 3 : 2;
    static constexpr bool kDefer = WAVES == 4;
    static constexpr int kOffB = 0;                       // weight tile: BN rows x 128 B
    static constexpr int kOffA = BN * BK;                 // activation tile: BM rows x 128 B
    static constexpr int kOffSA = kOffA + BM * BK;        // activation scales: BM x 4 B
    static constexpr int kOffSB = kOffSA + BM * 4;        // weight scales: BN x 4 B
    static constexpr int kStageBytes = kOffSB + BN * 4;
    static constexpr int kDmaB = BN / 8 / WAVES;          // 16-byte copies per wave per slice
    static constexpr int kDmaA = BM / 8 / WAVES;
    static constexpr int kTileDma = kDmaB + kDmaA;
};

enum { MODE_BLOCK128 = 0, MODE_ROW128 = 1, MODE_MX = 2 };

struct KArgs {
    int32_t M, N, K;
    const uint8_t* a; int64_t lda;
    const uint8_t* sa; int64_t sa_sm, sa_sk;   // element strides (MX: bytes, sa_sk unused)
    const uint8_t* b; int64_t ldb; int64_t b_sg;
    const uint8_t* sb; int64_t sb_sg, sb_sn, sb_sk;
    void* c; int64_t ldc;
    int32_t G; const int32_t* offsets; const int32_t* a_rows;
};

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// global -> LDS copies: lane l's bytes land at lds_wave_base + l * BYTES.
// Issued as inline assembly on purpose: the compiler cannot tell which LDS
// stage a copy writes, so for the builtin it would wait for every outstanding
// copy (vmcnt(0)) before the first LDS read of the current stage, which
// serializes the pipeline.  Ordering is explicit instead: s_waitcnt vmcnt(n)
// on the issuing wave, then s_barrier, before any wave reads a stage.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
__device__ __forceinline__ void dma16(const void* src, const uint8_t* lds_wave_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(m0), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, const uint8_t* lds_wave_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_wave_base));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(m0), "v"(src) : "memory", "m0");
}

// Read the 32-byte MFMA fragment of tile row `row` for lane quarter q.  The
// 16x16x128 FP8 instruction takes K index 64 * (byte / 16) + 16 * q + byte % 16
// from byte `byte` of a lane in quarter q (measured with one-hot probes of its
// per-32-K scale slots: slot s covers bytes 0-15 of quarters 2s and 2s+1 for
// s < 2 and bytes 16-31 of quarters 2(s-2) and 2(s-2)+1 for s >= 2, and the
// scale of slot s comes from the lanes of quarter s).  The lane's low 16 bytes
// are therefore logical chunk q of the row's 128-byte K slice and its high 16
// bytes chunk q + 4.  In this order the 32-wide K block s of the slice is
// exactly scale slot s, which the MX mode relies on; the FP32-scale modes only
// need both operands in the same order.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int q) {
    const int f = swz(row);
    const uint8_t* base = tile + row * BK;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + ((q ^ f) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + (((q + 4) ^ f) << 4));
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

__device__ __forceinline__ v4f mfma_unit(const v8i& a, const v8i& b) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, kE8M0One, 0, kE8M0One);
}

template <int MODE, bool GROUPED, bool OUTF32, int WAVES>
__global__ void __launch_bounds__(Cfg<WAVES>::kThreads, 1) k_gemm(KArgs p) {
    using C = Cfg<WAVES>;
    constexpr int BM = C::BM, kStages = C::kStages, kStageBytes = C::kStageBytes;
    constexpr int kOffA = C::kOffA, kOffB = C::kOffB, kOffSA = C::kOffSA, kOffSB = C::kOffSB;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];
    __shared__ int s_tile[2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave & 1, wm = wave >> 1;
    const int q = lane >> 4, r16 = lane & 15;

    // ---------------------------------------------------------------- tile
    int32_t m_begin, m_end, n0;
    const uint8_t* bptr = p.b;
    const uint8_t* sbp = p.sb;
    if (!GROUPED) {
        const int ntn = (p.N + BN - 1) / BN, ntm = (p.M + BM - 1) / BM;
        const int nblk = ntn * ntm;
        const int bid = blockIdx.x;
        // consecutive tile ids on one XCD (workgroups are dealt round-robin to the 8 XCDs)
        const int per = nblk / 8;
        const int tile = bid < per * 8 ? (bid % 8) * per + bid / 8 : bid;
        // groups of GM m-tiles sweep n, so co-resident tiles share operand panels in L2
        constexpr int GM = 8;
        const int gsz = GM * ntn;
        const int grp = tile / gsz;
        const int fm = grp * GM;
        const int gm = min(ntm - fm, GM);
        const int tm = fm + (tile % gsz) % gm;
        const int tn = (tile % gsz) / gm;
        m_begin = tm * BM;
        m_end = min(p.M, m_begin + BM);
        n0 = tn * BN;
    } else {
        // Work item blockIdx.y is the blockIdx.y-th BM-row tile in the list of
        // all groups' tiles; wave 0 scans the per-group tile counts.
        if (threadIdx.x == 0) s_tile[0] = -1;
        if (wave == 0) {
            const int t = blockIdx.y;
            int carry = 0;
            for (int gb = 0; gb < p.G; gb += 128) {
                const int g0 = gb + 2 * lane, g1 = g0 + 1;
                const int o0 = g0 < p.G ? p.offsets[g0] : 0, o1 = g0 < p.G ? p.offsets[g0 + 1] : 0;
                const int o2 = g1 < p.G ? p.offsets[g1 + 1] : 0;
                const int c0 = g0 < p.G ? (o1 - o0 + BM - 1) / BM : 0;
                const int c1 = g1 < p.G ? (o2 - o1 + BM - 1) / BM : 0;
                int incl = c0 + c1;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int v = __shfl_up(incl, d, 64);
                    if (lane >= d) incl += v;
                }
                const int start0 = carry + incl - (c0 + c1);
                const int start1 = start0 + c0;
                if (t >= start0 && t < start0 + c0) { s_tile[0] = g0; s_tile[1] = t - start0; }
                if (t >= start1 && t < start1 + c1) { s_tile[0] = g1; s_tile[1] = t - start1; }
                carry += __shfl(incl, 63, 64);
            }
        }
        __syncthreads();
        const int g = s_tile[0];
        if (g < 0) return;                         // uniform: no tile for this work item
        const int lt = s_tile[1];
        m_begin = p.offsets[g] + lt * BM;
        m_end = min(p.offsets[g + 1], m_begin + BM);
        n0 = blockIdx.x * BN;
        bptr += (int64_t)g * p.b_sg;
        sbp += (int64_t)g * p.sb_sg * (MODE == MODE_MX ? 1 : 4);
    }
    auto arow = [&](int m_local) {             // physical A row of tile row m_local (clamped)
        int m = min(m_begin + m_local, m_end - 1);
        if (GROUPED && p.a_rows != nullptr) m = p.a_rows[m];
        return m;
    };

    // ------------------------------------------------------- copy set-up
    // Wave w copies weight rows [8 kDmaB w, +8 kDmaB) and activation rows
    // [8 kDmaA w, +8 kDmaA), one instruction per 8 rows x 128 bytes.  Lane l
    // fetches logical chunk (l % 8) ^ f(row) of row 8 j + l / 8.
    uint32_t offB[C::kDmaB], offA[C::kDmaA];
#pragma unroll
    for (int j = 0; j < C::kDmaB; ++j) {
        const int row = (wave * C::kDmaB + j) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(row);
        offB[j] = (uint32_t)((int64_t)min(n0 + row, p.N - 1) * p.ldb + chunk * 16);
    }
#pragma unroll
    for (int j = 0; j < C::kDmaA; ++j) {
        const int row = (wave * C::kDmaA + j) * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(row);
        offA[j] = (uint32_t)((int64_t)arow(row) * p.lda + chunk * 16);
    }
    // Scale copies (4-byte lanes).  Activation scales: waves [0, BM/64) copy
    // rows [64 w, +64).  Weight scales: MODE_BLOCK128 -> wave BM/64 copies the
    // two 128-row blocks of the tile; ROW128 / MX -> waves 0..3 copy rows [64 w, +64).
    const bool has_sa = wave < BM / 64;
    const bool has_sb = (MODE == MODE_BLOCK128) ? wave == BM / 64 : wave < 4;
    int64_t sa_off = 0, sb_off = 0;             // byte offsets without the slice term
    if (has_sa) {
        const int m = arow(wave * 64 + lane);
        sa_off = (MODE == MODE_MX) ? (int64_t)m * p.sa_sm : (int64_t)m * p.sa_sm * 4;
    }
    if (MODE == MODE_BLOCK128) {
        const int nb = min(n0 / 128 + (lane & 1), (p.N - 1) / 128);
        sb_off = (int64_t)nb * p.sb_sn * 4;
    } else {
        const int n = min(n0 + (wave & 3) * 64 + lane, p.N - 1);
        sb_off = (MODE == MODE_MX) ? (int64_t)n * p.sb_sn : (int64_t)n * p.sb_sn * 4;
    }
    auto issue_copy = [&](int kb, int stage) {
        uint8_t* st = smem + stage * kStageBytes;
        if (MODE == MODE_MX) {
            if (has_sa) dma4(p.sa + sa_off + kb * 4, st + kOffSA + wave * 64 * 4);
            if (has_sb) dma4(sbp + sb_off + kb * 4, st + kOffSB + wave * 64 * 4);
        } else {
            if (has_sa) dma4(p.sa + sa_off + (int64_t)kb * p.sa_sk * 4, st + kOffSA + wave * 64 * 4);
            if (has_sb) {
                if (MODE == MODE_BLOCK128) dma4(sbp + sb_off + (int64_t)kb * p.sb_sk * 4, st + kOffSB);
                else dma4(sbp + sb_off + (int64_t)kb * p.sb_sk * 4, st + kOffSB + wave * 64 * 4);
            }
        }
        const uint32_t ko = (uint32_t)kb * BK;
#pragma unroll
        for (int j = 0; j < C::kDmaB; ++j)
            dma16(bptr + offB[j] + ko, st + kOffB + (wave * C::kDmaB + j) * 8 * BK);
#pragma unroll
        for (int j = 0; j < C::kDmaA; ++j)
            dma16(p.a + offA[j] + ko, st + kOffA + (wave * C::kDmaA + j) * 8 * BK);
    };

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nk = p.K / BK;
#pragma unroll
    for (int s0 = 0; s0 < kStages - 1; ++s0)
        if (s0 < nk) issue_copy(s0, s0);

    for (int kb = 0; kb < nk; ++kb) {
        const int stage = kb % kStages;
        // This wave's copies for slice kb have landed once at most the
        // kTileDma tile copies of slice kb+1 (issued last, three-stage
        // pipeline) are outstanding; with two stages nothing newer is in flight.
        if (kStages == 3 && kb + 1 < nk)
            __builtin_amdgcn_s_waitcnt(0x0F70 | (C::kTileDma & 15) | ((C::kTileDma >> 4) << 14));
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);
        // Every wave's copies landed and every wave finished reading the
        // stage refilled next.  A plain s_barrier (with a compiler memory
        // clobber) rather than __syncthreads(): the latter's release fence
        // would also wait for copies still in flight.
        asm volatile("s_barrier" ::: "memory");
        if (kb + kStages - 1 < nk) issue_copy(kb + kStages - 1, (kb + kStages - 1) % kStages);

        const uint8_t* st = smem + stage * kStageBytes;
        const uint8_t* tB = st + kOffB;
        const uint8_t* tA = st + kOffA;
        v8i fa[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) fa[mt] = read_frag(tA, wm * 64 + mt * 16 + r16, q);

        if (MODE == MODE_MX) {
            const uint8_t* sa8 = st + kOffSA;
            const uint8_t* sb8 = st + kOffSB;
            int mxa[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) mxa[mt] = sa8[(wm * 64 + mt * 16 + r16) * 4 + q];
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const int row = wn * 128 + nt * 16 + r16;
                const v8i fb = read_frag(tB, row, q);
                const int mxb = sb8[row * 4 + q];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    acc[nt][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb, fa[mt], acc[nt][mt], 0, 0, 0,
                                                                                  mxb, 0, mxa[mt]);
            }
        } else {
            const float* saf = reinterpret_cast<const float*>(st + kOffSA);
            const float* sbf = reinterpret_cast<const float*>(st + kOffSB);
            float sam[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) sam[mt] = saf[wm * 64 + mt * 16 + r16];
            float sc[4];
            if (MODE == MODE_BLOCK128) {
                const float sbv = sbf[wn];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) sc[mt] = sam[mt] * sbv;
            }
            v4f part[2][4];
            float4 sbr[2];
            auto promote = [&](int pt, int ps) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (MODE == MODE_BLOCK128) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[pt][mt][r] = __builtin_fmaf(part[ps][mt][r], sc[mt], acc[pt][mt][r]);
                    } else {
                        const float s4[4] = {sbr[ps].x, sbr[ps].y, sbr[ps].z, sbr[ps].w};
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[pt][mt][r] = __builtin_fmaf(part[ps][mt][r], sam[mt] * s4[r], acc[pt][mt][r]);
                    }
                }
            };
            v8i fb_next = read_frag(tB, wn * 128 + r16, q);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const int ps = C::kDefer ? (nt & 1) : 0;
                const v8i fb = fb_next;
                if (nt < 7) fb_next = read_frag(tB, wn * 128 + (nt + 1) * 16 + r16, q);
                if (MODE == MODE_ROW128)
                    sbr[ps] = *reinterpret_cast<const float4*>(sbf + wn * 128 + nt * 16 + 4 * q);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) part[ps][mt] = mfma_unit(fb, fa[mt]);
                if (!C::kDefer) promote(nt, 0);
                else if (nt > 0) promote(nt - 1, (nt - 1) & 1);
            }
            if (C::kDefer) promote(7, 1);
        }
    }

    // ---------------------------------------------------------- epilogue
    const int nw0 = n0 + wn * 128;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int m = m_begin + wm * 64 + mt * 16 + r16;
        if (m >= m_end) continue;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const int n = nw0 + nt * 16 + 4 * q;
            if (n >= p.N) continue;
            if (OUTF32) {
                float* dst = static_cast<float*>(p.c) + (int64_t)m * p.ldc + n;
                *reinterpret_cast<float4*>(dst) = make_float4(acc[nt][mt][0], acc[nt][mt][1], acc[nt][mt][2], acc[nt][mt][3]);
            } else {
                uint16_t* dst = static_cast<uint16_t*>(p.c) + (int64_t)m * p.ldc + n;
                const uint32_t lo = f32_to_bf16_rne(acc[nt][mt][0]) | (f32_to_bf16_rne(acc[nt][mt][1]) << 16);
                const uint32_t hi = f32_to_bf16_rne(acc[nt][mt][2]) | (f32_to_bf16_rne(acc[nt][mt][3]) << 16);
                *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
            }
        }
    }
}

template <int MODE, bool GROUPED, int WAVES>
hipError_t launch(const KArgs& p, bool out_f32, dim3 grid, hipStream_t st) {
    constexpr int T = Cfg<WAVES>::kThreads;
    if (out_f32)
        hipLaunchKernelGGL((k_gemm<MODE, GROUPED, true, WAVES>), grid, dim3(T), 0, st, p);
    else
        hipLaunchKernelGGL((k_gemm<MODE, GROUPED, false, WAVES>), grid, dim3(T), 0, st, p);
    return hipGetLastError();
}

template <int MODE, bool GROUPED, int WAVES>
hipError_t launch_cfg(const KArgs& p, bool out_f32, hipStream_t st) {
    constexpr int BM = Cfg<WAVES>::BM;
    dim3 grid;
    if (!GROUPED) {
        grid = dim3((unsigned)(((int64_t)(p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN)));
    } else {
        // upper bound on the number of BM-row tiles over all groups
        grid = dim3((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM + p.G));
    }
    return launch<MODE, GROUPED, WAVES>(p, out_f32, grid, st);
}

// Tile choice: 256 x 256 (8 waves) when it still gives every CU a tile,
// else 256 x 128 (4 waves).
int waves_for(int64_t rows, int64_t N) {
    const int64_t big = ((rows + 255) / 256) * ((N + BN - 1) / BN);
    return big >= 256 ? 8 : 4;
}

KArgs base_args(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const void* sa, const uint8_t* b,
                int64_t ldb, const void* sb, void* c, int64_t ldc) {
    KArgs p{};
    p.M = (int32_t)M; p.N = (int32_t)N; p.K = (int32_t)K;
    p.a = a; p.lda = lda; p.sa = static_cast<const uint8_t*>(sa);
    p.b = b; p.ldb = ldb; p.sb = static_cast<const uint8_t*>(sb);
    p.c = c; p.ldc = ldc;
    return p;
}

}  // namespace

hipError_t launch_gemm_blockscaled(const GemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    KArgs p = base_args(g.M, g.N, g.K, g.a, g.lda, g.sa, g.b, g.ldb, g.sb, g.c, g.ldc);
    p.sa_sm = g.sa_sm; p.sa_sk = g.sa_sk; p.sb_sn = g.sb_sn; p.sb_sk = g.sb_sk;
    const int w = waves_for(g.M, g.N);
    if (g.bscale_row)
        return w == 8 ? launch_cfg<MODE_ROW128, false, 8>(p, g.out_f32, st) : launch_cfg<MODE_ROW128, false, 4>(p, g.out_f32, st);
    return w == 8 ? launch_cfg<MODE_BLOCK128, false, 8>(p, g.out_f32, st) : launch_cfg<MODE_BLOCK128, false, 4>(p, g.out_f32, st);
}

hipError_t launch_gemm_grouped(const GemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    KArgs p = base_args(g.M, g.N, g.K, g.a, g.lda, g.sa, g.b, g.ldb, g.sb, g.c, g.ldc);
    p.sa_sm = g.sa_sm; p.sa_sk = g.sa_sk; p.b_sg = g.b_sg; p.sb_sg = g.sb_sg; p.sb_sn = g.sb_sn; p.sb_sk = g.sb_sk;
    p.G = g.G; p.offsets = g.offsets; p.a_rows = g.a_rows;
    return launch_cfg<MODE_BLOCK128, true, 4>(p, g.out_f32, st);
}

hipError_t launch_gemm_mx(const MxGemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    KArgs p = base_args(g.M, g.N, g.K, g.a, g.lda, g.sa, g.b, g.ldb, g.sb, g.c, g.ldc);
    p.sa_sm = g.lds_a; p.sa_sk = 1; p.b_sg = g.b_sg; p.sb_sg = g.sb_sg; p.sb_sn = g.lds_b; p.sb_sk = 1;
    p.G = g.G; p.offsets = g.offsets; p.a_rows = g.a_rows;
    if (g.G == 0)
        return waves_for(g.M, g.N) == 8 ? launch_cfg<MODE_MX, false, 8>(p, g.out_f32, st)
                                        : launch_cfg<MODE_MX, false, 4>(p, g.out_f32, st);
    return launch_cfg<MODE_MX, true, 4>(p, g.out_f32, st);
}

}  // namespace fp8bs
