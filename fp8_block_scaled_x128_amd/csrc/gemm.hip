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
// Kernel structure (one workgroup per 256x256 output tile, 8 waves):
//  - K advances in 128-byte slices.  Each slice of the 256-row A tile and of
//    the 256-row B tile (32 KB each) is copied straight from global memory
//    into LDS with global_load_lds_dwordx4 (no register staging), double
//    buffered (2 x 64 KB).
//  - LDS rows are 128 bytes; 16-byte chunk c of row r sits in slot
//    c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1), which makes the fragment
//    reads conflict-free (16 consecutive rows reading the same logical chunk
//    hit 16 distinct 16-byte bank groups).  The copy realizes the swizzle by
//    choosing which global chunk each lane fetches.
//  - Wave w owns n rows [128 * (w / 4), +128) and m rows [64 * (w % 4), +64):
//    8 x 4 tiles of v_mfma_scale_f32_16x16x128_f8f6f4 per slice.  The weight
//    rows are the instruction's A operand and the activation rows its B
//    operand, so each lane's 4 outputs share one activation row m and four
//    consecutive n; the slice scale of a lane is then sa(m, kb) * sb(n/128, kb)
//    with sb uniform over the wave.
//  - FP32-scale modes: each MFMA produces a fresh FP32 partial for its
//    slice (zero accumulator input, unit E8M0 scales), which is promoted with
//    one FMA per output: acc = fma(partial, sa * sb, acc).
//  - MX mode: the instruction accumulates in place with the per-lane UE8M0
//    scale bytes of its row and 32-wide K block.
#include "device_common.h"
#include "internal.h"

namespace fp8bs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kWaves = 8, kThreads = kWaves * 64;
constexpr int kTileBytes = 256 * BK;          // one operand tile slice
constexpr int kE8M0One = 127;                 // UE8M0 code of 1.0

enum { MODE_BLOCK128 = 0, MODE_ROW128 = 1, MODE_MX = 2 };

struct KArgs {
    int32_t M, N, K;
    const uint8_t* a; int64_t lda;
    const void* sa; int64_t sa_sm, sa_sk;      // MX: sa_sm = lds_a, sa_sk = 1 (bytes)
    const uint8_t* b; int64_t ldb; int64_t b_sg;
    const void* sb; int64_t sb_sg, sb_sn, sb_sk;
    void* c; int64_t ldc;
    int32_t G; const int32_t* offsets; const int32_t* a_rows;
};

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Read the 32-byte MFMA fragment of tile row `row` for lane quarter q.  The
// 16x16x128 FP8 instruction takes K index 64 * (byte / 16) + 16 * q + byte % 16
// from byte `byte` of a lane in quarter q (measured with one-hot probes of its
// per-32-K scale slots: slot s covers bytes 0-15 of quarters 2s and 2s+1 for
// s < 2 and bytes 16-31 of quarters 2(s-2) and 2(s-2)+1 for s >= 2, and the
// scale of slot s comes from the lanes of quarter s).  The lane's low 16 bytes
// are therefore logical chunk q of the row's 128-byte K slice and its high 16
// bytes chunk q + 4.
// In this order the 32-wide K block s of the slice is exactly scale slot s,
// which the MX mode relies on; the FP32-scale modes only need both operands
// in the same order.
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

template <int MODE, bool GROUPED, bool OUTF32>
__global__ void __launch_bounds__(kThreads, 1) k_gemm(KArgs p) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][kTileBytes];   // [stage][0: B(n) 1: A(m)]
    __shared__ int s_tile[2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave >> 2, wm = wave & 3;

    // ---------------------------------------------------------------- tile
    int32_t m_begin, m_end, n0;
    const uint8_t* bptr = p.b;
    const uint8_t* sbp = static_cast<const uint8_t*>(p.sb);
    if (!GROUPED) {
        const int ntn = (p.N + BN - 1) / BN, ntm = (p.M + BM - 1) / BM;
        const int nblk = ntn * ntm;
        int bid = blockIdx.x;
        // consecutive tile ids on one XCD (workgroups are dealt round-robin to the 8 XCDs)
        const int per = nblk / 8;
        int tile = bid < per * 8 ? (bid % 8) * per + bid / 8 : bid;
        // groups of 4 m-tiles sweep n, so co-resident tiles share A and B panels in L2
        constexpr int GM = 4;
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
        // Work item blockIdx.y is the blockIdx.y-th 256-row tile in the list of
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

    // ------------------------------------------------------- copy set-up
    // Wave w copies rows [32 w, 32 w + 32) of each operand tile: 4 x 8 rows.
    // Lane l fetches chunk (l % 8) ^ f(row) of row 8 j' + l / 8.
    uint32_t offA[4], offB[4];     // byte offsets of the lane's rows (without the K slice)
    const uint8_t* abase = p.a;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = wave * 32 + j * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ swz(row);
        int nrow = min(n0 + row, p.N - 1);
        offB[j] = (uint32_t)((int64_t)nrow * p.ldb + chunk * 16);
        int mrow = min(m_begin + row, m_end - 1);
        if (GROUPED && p.a_rows != nullptr) mrow = p.a_rows[mrow];
        offA[j] = (uint32_t)((int64_t)mrow * p.lda + chunk * 16);
    }
    auto issue_copy = [&](int kb, int stage) {
        const uint32_t ko = (uint32_t)kb * BK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint8_t* dstB = &smem[stage][0][(wave * 32 + j * 8) * BK];
            uint8_t* dstA = &smem[stage][1][(wave * 32 + j * 8) * BK];
            dma16(bptr + offB[j] + ko, dstB);
            dma16(abase + offA[j] + ko, dstA);
        }
    };

    // ------------------------------------------------------- scales set-up
    const int q = lane >> 4, r16 = lane & 15;
    uint32_t sa_row[4];           // per m-tile: element offset of the lane's activation-row scales
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        int m = min(m_begin + wm * 64 + mt * 16 + r16, m_end - 1);
        if (GROUPED && p.a_rows != nullptr) m = p.a_rows[m];
        sa_row[mt] = (uint32_t)((int64_t)m * p.sa_sm);
    }
    const int nw0 = n0 + wn * 128;                   // first n row of the wave (128-aligned)
    const int nb_w = min(nw0, p.N - 1) / 128;
    uint32_t sb_row[8];           // MX / ROW128: per n-tile
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        const int nrow = (MODE == MODE_MX) ? min(nw0 + nt * 16 + r16, p.N - 1)
                                           : min(nw0 + nt * 16 + 4 * q, p.N - 4);
        sb_row[nt] = (uint32_t)((int64_t)nrow * p.sb_sn);
    }

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nk = p.K / BK;
    issue_copy(0, 0);

    // scale registers for the current slice
    float sa_cur[4], sb_cur = 0.f;
    uint32_t mxa_cur[4], mxb_cur[8];
    auto load_scales = [&](int kb, float sa_v[4], float& sb_v, uint32_t mxa[4], uint32_t mxb[8]) {
        if (MODE == MODE_MX) {
            const uint8_t* sa8 = static_cast<const uint8_t*>(p.sa);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) mxa[mt] = sa8[sa_row[mt] + (uint32_t)(kb * 4 + q)];
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) mxb[nt] = sbp[sb_row[nt] + (uint32_t)(kb * 4 + q)];
        } else {
            const float* saf = static_cast<const float*>(p.sa);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) sa_v[mt] = saf[(int64_t)sa_row[mt] + (int64_t)kb * p.sa_sk];
            if (MODE == MODE_BLOCK128)
                sb_v = reinterpret_cast<const float*>(sbp)[(int64_t)nb_w * p.sb_sn + (int64_t)kb * p.sb_sk];
        }
    };
    load_scales(0, sa_cur, sb_cur, mxa_cur, mxb_cur);

    for (int kb = 0; kb < nk; ++kb) {
        const int stage = kb & 1;
        __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): this wave's copies and scale loads landed
        __syncthreads();                             // all waves' copies landed; stage^1 is free
        float sa_nx[4], sb_nx = 0.f;
        uint32_t mxa_nx[4], mxb_nx[8];
        if (kb + 1 < nk) {
            issue_copy(kb + 1, stage ^ 1);
            load_scales(kb + 1, sa_nx, sb_nx, mxa_nx, mxb_nx);
        }
        const uint8_t* tB = smem[stage][0];
        const uint8_t* tA = smem[stage][1];
        v8i fa[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) fa[mt] = read_frag(tA, wm * 64 + mt * 16 + r16, q);
        float sc[4];
        if (MODE == MODE_BLOCK128) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) sc[mt] = sa_cur[mt] * sb_cur;
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const v8i fb = read_frag(tB, wn * 128 + nt * 16 + r16, q);
            float sbr[4];
            if (MODE == MODE_ROW128) {
                const float* sbf = reinterpret_cast<const float*>(sbp);
#pragma unroll
                for (int r = 0; r < 4; ++r) sbr[r] = sbf[(int64_t)sb_row[nt] + (int64_t)r * p.sb_sn + (int64_t)kb * p.sb_sk];
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (MODE == MODE_MX) {
                    acc[nt][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        fb, fa[mt], acc[nt][mt], 0, 0, 0, (int)mxb_cur[nt], 0, (int)mxa_cur[mt]);
                } else {
                    const v4f zero = {0.f, 0.f, 0.f, 0.f};
                    const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        fb, fa[mt], zero, 0, 0, 0, kE8M0One, 0, kE8M0One);
                    if (MODE == MODE_BLOCK128) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[nt][mt][r] = __builtin_fmaf(part[r], sc[mt], acc[nt][mt][r]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[nt][mt][r] = __builtin_fmaf(part[r], sa_cur[mt] * sbr[r], acc[nt][mt][r]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);   // keep the n-tile steps apart (register pressure)
        }
        if (kb + 1 < nk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) { sa_cur[i] = sa_nx[i]; mxa_cur[i] = mxa_nx[i]; }
#pragma unroll
            for (int i = 0; i < 8; ++i) mxb_cur[i] = mxb_nx[i];
            sb_cur = sb_nx;
        }
    }

    // ---------------------------------------------------------- epilogue
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

template <int MODE, bool GROUPED>
hipError_t launch(const KArgs& p, bool out_f32, dim3 grid, hipStream_t st) {
    if (out_f32)
        hipLaunchKernelGGL((k_gemm<MODE, GROUPED, true>), grid, dim3(kThreads), 0, st, p);
    else
        hipLaunchKernelGGL((k_gemm<MODE, GROUPED, false>), grid, dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_blockscaled(const GemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    KArgs p{};
    p.M = (int32_t)g.M; p.N = (int32_t)g.N; p.K = (int32_t)g.K;
    p.a = g.a; p.lda = g.lda; p.sa = g.sa; p.sa_sm = g.sa_sm; p.sa_sk = g.sa_sk;
    p.b = g.b; p.ldb = g.ldb; p.b_sg = 0; p.sb = g.sb; p.sb_sg = 0; p.sb_sn = g.sb_sn; p.sb_sk = g.sb_sk;
    p.c = g.c; p.ldc = g.ldc; p.G = 0; p.offsets = nullptr; p.a_rows = nullptr;
    const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    dim3 grid((unsigned)tiles);
    return g.bscale_row ? launch<MODE_ROW128, false>(p, g.out_f32, grid, st)
                        : launch<MODE_BLOCK128, false>(p, g.out_f32, grid, st);
}

hipError_t launch_gemm_grouped(const GemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    KArgs p{};
    p.M = (int32_t)g.M; p.N = (int32_t)g.N; p.K = (int32_t)g.K;
    p.a = g.a; p.lda = g.lda; p.sa = g.sa; p.sa_sm = g.sa_sm; p.sa_sk = g.sa_sk;
    p.b = g.b; p.ldb = g.ldb; p.b_sg = g.b_sg; p.sb = g.sb; p.sb_sg = g.sb_sg; p.sb_sn = g.sb_sn; p.sb_sk = g.sb_sk;
    p.c = g.c; p.ldc = g.ldc; p.G = g.G; p.offsets = g.offsets; p.a_rows = g.a_rows;
    // upper bound on the number of 256-row tiles over all groups
    const int64_t mt = (g.M + BM - 1) / BM + g.G;
    dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)mt);
    return launch<MODE_BLOCK128, true>(p, g.out_f32, grid, st);
}

hipError_t launch_gemm_mx(const MxGemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    KArgs p{};
    p.M = (int32_t)g.M; p.N = (int32_t)g.N; p.K = (int32_t)g.K;
    p.a = g.a; p.lda = g.lda; p.sa = g.sa; p.sa_sm = g.lds_a; p.sa_sk = 1;
    p.b = g.b; p.ldb = g.ldb; p.b_sg = g.b_sg; p.sb = g.sb; p.sb_sg = g.sb_sg; p.sb_sn = g.lds_b; p.sb_sk = 1;
    p.c = g.c; p.ldc = g.ldc; p.G = g.G; p.offsets = g.offsets; p.a_rows = g.a_rows;
    if (g.G == 0) {
        const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
        return launch<MODE_MX, false>(p, g.out_f32, dim3((unsigned)tiles), st);
    }
    const int64_t mt = (g.M + BM - 1) / BM + g.G;
    return launch<MODE_MX, true>(p, g.out_f32, dim3((unsigned)((g.N + BN - 1) / BN), (unsigned)mt), st);
}

}  // namespace fp8bs
