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
// Kernel structure: one workgroup per output tile of 32 NF weight rows (n;
// NF = 8, 6 or 5) x 128 (4 waves, one per SIMD) or 256 (8 waves, two per
// SIMD) activation rows; the host picks the tiling (waves_for, plan_dense).
//  - K advances in 128-byte slices.  The slice of the weight tile (32 NF
//    rows x 128 B), of the activation tile and the slice's scales are copied
//    straight from global memory into LDS with global_load_lds (no register
//    staging), through the multi-buffer pipeline described at Cfg.
//  - LDS rows are 128 bytes; 16-byte chunk c of row r sits in slot
//    c ^ (r & 7), which makes the fragment reads free of bank conflicts
//    (measured with the LDS bank-conflict counter; the variant
//    (r & 7) ^ ((r >> 3) & 1) costs 4 conflict cycles per read).  The copy
//    realizes the swizzle by choosing which global chunk each lane fetches.
//  - Wave w owns n rows [16 NF (w & 1), +16 NF) and m rows [64 (w >> 1), +64):
//    NF x 4 tiles of v_mfma_scale_f32_16x16x128_f8f6f4 per slice.  Weight rows
//    are the instruction's A operand and activation rows its B operand, so a
//    lane's 4 outputs share one activation row m and four consecutive n.
//  - FP32-scale modes: each MFMA produces a fresh FP32 partial for its slice
//    (zero accumulator input, unit E8M0 scales), promoted with one FMA per
//    output, acc = fma(partial, sa * sb, acc), one n-tile behind the MFMAs so
//    that the promotion overlaps the next n-tile's matrix work.
//  - MX mode: the instruction accumulates in place with the per-lane UE8M0
//    scale bytes of its row and 32-wide K block.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace fp8bs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BK = 128;                         // K bytes per slice
constexpr int kE8M0One = 127;                  // UE8M0 code of 1.0
constexpr int kCUs = 256;                       // MI355X compute units

// Lane-group maxima by DPP for code where every lane of the wave is active
// (the fused SiLU*mul epilogue): each step is one VALU op reading another
// lane's register, where a shuffle through ds_bpermute is an LDS round trip.
template <int CTRL>
__device__ __forceinline__ float max_dpp(float v) {
    const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false);
    return fmaxf(v, __int_as_float(o));
}
constexpr int kDppXor1 = 0xb1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4e;          // quad_perm [2, 3, 0, 1]
constexpr int kDppRowMirror = 0x140;    // lane i <- lane 15 - i of its 16-lane row
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7 - i of its 8-lane half row
// Max over each aligned group of 4 lanes.
__device__ __forceinline__ float quad_max_dpp(float v) { return max_dpp<kDppXor2>(max_dpp<kDppXor1>(v)); }
// Max over each 16-lane row: quads, then the half-row mirror joins quads 0-1
// and 2-3, then the row mirror joins the two halves.
__device__ __forceinline__ float row16_max_dpp(float v) {
    return max_dpp<kDppRowMirror>(max_dpp<kDppHalfMirror>(quad_max_dpp(v)));
}

// Tile configurations.  Every wave computes NF 16-row weight tiles (16 NF
// weight rows) x 64 activation rows; waves are arranged 2 (n) x WAVES/2 (m),
// so a tile is 32 NF weight rows x 32 WAVES activation rows.
//   WAVES = 4: one wave per SIMD (512 registers each), promotion deferred by
//              one n-tile within the wave.
//   WAVES = 8: two waves per SIMD (256 registers each) whose matrix and
//              vector work interleave.
//   NF = 8 (256 weight rows) is the general tile; NF = 5 and 6 (160 and 192
//   rows) exist so that problems whose 256-row tiles leave a round of the 256
//   compute units mostly idle can be tiled into whole rounds.
// LDS pipeline.  The weight tile of a slice is read during the whole slice,
// the activation tile only at its start (each wave keeps its 4 activation
// fragments in registers).  Weight slices get kBStages buffers; activation
// slices two where they fit in LDS, else one with kABarrier: a second barrier
// right after the fragment reads lets the current activation buffer be
// refilled at once.  A slice's copies are issued kLeadA / kLeadB steps before
// it is consumed.
// ROWSC: the weight scales are per row (ROW128, MX), copied in 64-row pieces,
// so their LDS region is padded to whole pieces.
template <int WAVES, int NF, bool ROWSC = false, int WN = 2>
struct Cfg {
    static constexpr int kWaves = WAVES;
    static constexpr int kNF = NF;
    static constexpr int kThreads = WAVES * 64;
    static constexpr int BN = 16 * NF * WN;
    static constexpr int BM = 64 * (WAVES / WN);
    static constexpr bool kDefer = true;
    // Workgroups resident per compute unit.  The 4-wave tiles with one wave
    // column (WN = 1, 128 x 256) and the 4-wave 160 x 128 tile are sized for
    // two per CU: each SIMD then runs two waves of different workgroups, so
    // one workgroup's barriers, fragment reads, pipeline fill and output
    // writes overlap the other's matrix work (the two waves of a SIMD in an
    // 8-wave workgroup meet the same barriers).
    static constexpr int kPerCU = (WN == 1 || (WAVES == 4 && NF == 5 && WN == 2)) ? 2 : 1;
    static constexpr int kMinWavesPerEU = kPerCU * WAVES / 4;
    static constexpr int kLdsMax = 160 * 1024 / kPerCU;
    // Measured on the MLP shapes (M 4096; N 9728, K 2560 and N 2560, K 9728):
    // 256x256 tile: 3 weight stages + 1 activation buffer with the second
    // barrier beats 2 + 2 without it (equal on the first shape, 9% faster on
    // the second); 256x128 tile: 3 + 2 without the second barrier is 2-3%
    // faster than with it.  Two workgroups per CU leave each room for 2
    // weight stages and 1 activation buffer (128 x 256) or 2 (160 x 128).
    static constexpr int kBStages = kPerCU == 2 ? 2 : 3;
    static constexpr int kBStageBytes = BN * BK + (ROWSC ? (BN + 63) / 64 * 64 : BN) * 4;   // weight tile + scales
    static constexpr int kABufBytes = BM * BK + BM * 4;     // activation tile + activation scales
    static constexpr int kAStages = kBStages * kBStageBytes + 2 * kABufBytes <= kLdsMax ? 2 : 1;
    static constexpr bool kABarrier = kAStages == 1;
    static constexpr int kLdsBytes = kBStages * kBStageBytes + kAStages * kABufBytes;
    // 16-byte copies per wave per slice: a wave copy moves 8 rows.  When the
    // 4 NF weight-row copies do not divide among the waves, the surplus copy
    // slots repeat copies of wave 0 (same bytes to the same LDS location).
    static constexpr int kCopiesB = BN / 8;
    static constexpr int kDmaB = (kCopiesB + WAVES - 1) / WAVES;
    static constexpr int kDmaA = BM / 8 / WAVES;
    static constexpr int kLeadA = kABarrier ? kAStages : kAStages - 1;
    static constexpr int kLeadB = kBStages - 1;
    static constexpr int kLeadMax = kLeadA > kLeadB ? kLeadA : kLeadB;
    // Within a step the activation copies are issued before the weight
    // copies.  At the top of step kb, slice kb's copies have landed once at
    // most kNAfter tile copies (those issued after its last one) remain.
    static constexpr int kNAfter = kLeadA < kLeadB ? kDmaB + (kLeadA - 1) * (kDmaA + kDmaB)
                                                   : (kLeadB - 1) * (kDmaA + kDmaB);
    // That count assumes the steps in between issued full copies, which holds
    // for leads of 1 or 2 (a step short of copies is then the last one).
    static_assert(kLeadA >= 1 && kLeadB >= 1 && kLeadMax <= 2, "pipeline leads must be 1 or 2");
    static_assert(kLdsBytes + 64 <= kLdsMax, "LDS budget");
    static_assert(kDmaA <= NF, "one activation copy per n-tile step");
    // tile copy slots: activation copy t in n-tile step t; weight copies
    // after the activation copies when they must follow them, else in step t
    // (lead 1: as early as possible) or spread over the slice (lead 2)
    static constexpr int kBFirst = kLeadA < kLeadB ? kDmaA : 0;
    static constexpr int b_slot(int t) { return kLeadB == 1 ? t : kBFirst + t * (NF - kBFirst) / kDmaB; }
    static_assert(kLeadB != 1 || kDmaB <= NF, "one weight copy per n-tile step");
};

// MODE_KINV: scales constant along K (rowwise / tensorwise scaling); the
// matrix unit accumulates the whole contraction with unit scales and the
// epilogue multiplies each output by sa(m) * sb(n).
// MODE_P2: 1x128 / 128x128 groups with power-of-two UE8M0 scales (bytes,
// sa [M][lds_a], sb [N/128][lds_b]); the matrix instruction applies them
// exactly, one scale byte per lane for its whole 128-K slice.
enum { MODE_BLOCK128 = 0, MODE_ROW128 = 1, MODE_MX = 2, MODE_KINV = 3, MODE_P2 = 4 };

struct KArgs {
    int32_t M, N, K;
    const uint8_t* a; int64_t lda;
    const uint8_t* sa; int64_t sa_sm, sa_sk;   // element strides (MX: bytes, sa_sk unused)
    const uint8_t* b; int64_t ldb; int64_t b_sg;
    const uint8_t* sb; int64_t sb_sg, sb_sn, sb_sk;
    void* c; int64_t ldc;
    int32_t G; const int32_t* offsets; const int32_t* a_rows;
    int32_t kinv_row;                          // MODE_KINV: sb indexed by n (1) or n / 128 (0)
    // dense K split: grid row y takes its share of the K slices and writes
    // its fp32 partial tile to c + y * c_split bytes (ksplit 1: no split)
    int32_t ksplit; int64_t c_split;
    // SWIGLU (grouped gate/up GEMM with SiLU*mul and the quantization of h in
    // the epilogue): B rows [0, swi) are gate rows, [swi, 2 swi) up rows;
    // h codes hq [rows][ld_hq]; h scales hs[m * hs_sm + group * hs_sg], fp32
    // per 128 columns (BLOCK128) or UE8M0 bytes per 32 columns (MX)
    int32_t swi;
    uint8_t* hq; int64_t ld_hq;
    void* hs; int64_t hs_sm, hs_sg;
};

__device__ __forceinline__ int swz(int r) { return r & 7; }

// LDS locations are handled as 32-bit LDS byte addresses (not generic
// pointers, whose conversion back to LDS costs a null test per use).
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return (uint32_t)(uintptr_t)(const lds_u8*)p;
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((uintptr_t)addr);
}
__device__ __forceinline__ float lds_readf(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) float*>((uintptr_t)addr);
}
__device__ __forceinline__ f32x4 lds_readf4(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>((uintptr_t)addr);
}
__device__ __forceinline__ int lds_readu8(uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) uint8_t*>((uintptr_t)addr);
}

// global -> LDS copies: lane l's bytes land at LDS address lds_dst + l * BYTES
// (lds_dst wave-uniform).  Issued as inline assembly on purpose: the compiler
// cannot tell which LDS stage a copy writes, so for the builtin it would wait
// for every outstanding copy (vmcnt(0)) before the first LDS read of the
// current stage, which serializes the pipeline.  Ordering is explicit
// instead: s_waitcnt vmcnt(n) on the issuing wave, then s_barrier, before any
// wave reads a stage.  Copies use the scalar-base form: wave-uniform 64-bit
// base in SGPRs plus a per-lane 32-bit byte offset (one VGPR per copy).  The
// K slice advances the scalar base, so the per-lane offsets stay fixed and a
// copy costs no vector instruction for its address.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(m0), "v"(off), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds_dst) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(m0), "v"(off), "s"(base) : "memory", "m0");
}

// MFMA fragment of one 16-row tile for lane quarter q.  The 16x16x128 FP8
// instruction takes K index 64 * (byte / 16) + 16 * q + byte % 16 from byte
// `byte` of a lane in quarter q (measured with one-hot probes of its per-32-K
// scale slots: slot s covers bytes 0-15 of quarters 2s and 2s+1 for s < 2 and
// bytes 16-31 of quarters 2(s-2) and 2(s-2)+1 for s >= 2, and the scale of
// slot s comes from the lanes of quarter s).  The lane's low 16 bytes are
// therefore logical chunk q of its row's 128-byte K slice and its high 16
// bytes chunk q + 4.  In this order the 32-wide K block s of the slice is
// exactly scale slot s, which the MX mode relies on; the FP32-scale modes only
// need both operands in the same order.
//
// Row r of a tile lives at r * 128 and its chunk c at slot c ^ (r & 7); tile
// rows read together differ by multiples of 16, so the two per-lane chunk
// offsets below serve every 16-row tile, which is then a constant offset.
struct FragOff {
    uint32_t lo, hi;
};
__device__ __forceinline__ FragOff frag_off(int r16, int q) {
    const int f = swz(r16);
    return FragOff{(uint32_t)(r16 * BK + ((q ^ f) << 4)), (uint32_t)(r16 * BK + (((q + 4) ^ f) << 4))};
}
// Per-lane LDS addresses of the fragments of the 16-row tile at `tile_row0`;
// later tiles of the same buffer are then constant offsets (folded into the
// ds_read offset field).  The empty asm keeps the compiler from hoisting the
// sum out of the K loop and holding one address per tile in registers.
__device__ __forceinline__ FragOff frag_base(uint32_t tile_row0, const FragOff& o) {
    FragOff b{tile_row0 + o.lo, tile_row0 + o.hi};
    asm volatile("" : "+v"(b.lo), "+v"(b.hi));
    return b;
}
__device__ __forceinline__ v8i read_frag(const FragOff& b, uint32_t offset) {
    const u32x4 lo = lds_read16(b.lo + offset);
    const u32x4 hi = lds_read16(b.hi + offset);
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}
// Barrier that orders LDS only: this wave's LDS accesses complete, then all
// waves meet.  (__syncthreads would also wait for every global access in
// flight, such as the copies of the next work item.)
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// FP32 partial of one 128-K slice of a 16 x 16 tile, unscaled.  Constant
// zero scale operands make the compiler emit the plain
// v_mfma_f32_16x16x128_f8f6f4 (one 8-byte instruction, no scaling) instead of
// the scaled form, which is issued as a v_mfma_ld_scale_b32 prefix plus the
// matrix instruction (16 bytes): 2-4% faster on the MLP shapes, bit-identical
// results (the exact-operand tests compare every tiling bit for bit).
__device__ __forceinline__ v4f mfma_unit(const v8i& a, const v8i& b) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// GATHER: grouped launches whose A rows are gathered through a_rows (the MoE
// dispatch); a separate instantiation, so that the launches with and without
// the gather (gate/up and down projections) also show as separate kernels in
// profiles.
template <int MODE, bool GROUPED, bool OUTF32, int WAVES, int NF, int WN, bool SWIGLU = false, bool GATHER = false>
__global__ void __launch_bounds__((Cfg<WAVES, NF, false, WN>::kThreads), (Cfg<WAVES, NF, false, WN>::kMinWavesPerEU))
k_gemm(KArgs p) {
    static_assert(!GATHER || GROUPED, "row gather: grouped launches only");
    using C = Cfg<WAVES, NF, (MODE == MODE_ROW128 || MODE == MODE_MX), WN>;
    // SWIGLU tiles: 256 weight rows = 128 gate rows (wave column 0) and the
    // matching 128 up rows (wave column 1) for 128 columns of h
    static_assert(!SWIGLU || (GROUPED && (MODE == MODE_BLOCK128 || MODE == MODE_MX) && !OUTF32 && WAVES == 8 &&
                              NF == 8 && WN == 2),
                  "SiLU*mul epilogue: grouped BLOCK128 or MX GEMM, 256 x 256 tiles, bf16 rounding of gate and up");
    constexpr int BM = C::BM, BN = C::BN;
    // per-row weight scales are copied by waves 0 .. ceil(BN / 64) - 1 in 64-row pieces
    static_assert(MODE == MODE_BLOCK128 || MODE == MODE_KINV || MODE == MODE_P2 || (BN + 63) / 64 <= WAVES,
                  "one wave per 64 rows of per-row weight scales");
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::kLdsBytes];
    // grouped: two slots for the published work item (the next item is
    // published while the current one may still be read), the workgroup's
    // item range, and wave 0's per-lane group table (up to 128 groups)
    __shared__ int s_tile[2][5];
    __shared__ int s_range[3];
    __shared__ int s_lk[6][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = WN == 2 ? (wave & 1) : 0, wm = WN == 2 ? (wave >> 1) : wave;
    const int q = lane >> 4, r16 = lane & 15;
    const FragOff fo = frag_off(r16, q);

    // ---------------------------------------------------------------- tile
    int32_t m_begin = 0, m_end = 0, n0 = 0;
    const uint8_t* bptr = p.b;
    const uint8_t* sbp = p.sb;
    // Grouped work items are (row tile, n-tile) pairs, row-tile major, over
    // the list of all groups' BM-row tiles.  Workgroups are dealt round-robin
    // to the 8 XCDs, and each XCD takes one contiguous range of work items:
    // the n-tiles of a row tile and the row tiles of one expert then run on
    // the same XCD and share their operand panels in its L2 (dealing n-tiles
    // across XCDs fetched the grouped gate/up operands 4.8 times from HBM).
    // The grid holds at most one workgroup per CU, and each workgroup walks
    // its XCD's items in turn: the copies of its next item go out before the
    // epilogue of the current one, so the first slices' latency overlaps the
    // output stores.  Wave 0 finds an item's group and row tile with a prefix
    // scan of the per-group row-tile counts; lane l keeps groups gb + 2l and
    // gb + 2l + 1 (row bounds o0..o1, o1..o2, tile counts c0, c1).
    const int ntn = SWIGLU ? p.swi / 128 : (p.N + BN - 1) / BN;
    int lk_o0 = 0, lk_o1 = 0, lk_o2 = 0, lk_c0 = 0, lk_c1 = 0, lk_incl = 0;
    int it_item = 0, it_end = 0, it_items = 0, it_slot = 0;
    auto lk_load = [&](int gb) {
        const int g0 = gb + 2 * lane, g1 = g0 + 1;
        lk_o0 = g0 < p.G ? p.offsets[g0] : 0;
        lk_o1 = g0 < p.G ? p.offsets[g0 + 1] : 0;
        lk_o2 = g1 < p.G ? p.offsets[g1 + 1] : 0;
        lk_c0 = g0 < p.G ? (lk_o1 - lk_o0 + BM - 1) / BM : 0;
        lk_c1 = g1 < p.G ? (lk_o2 - lk_o1 + BM - 1) / BM : 0;
    };
    auto lk_scan = [&]() {
        lk_incl = lk_c0 + lk_c1;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(lk_incl, d, 64);
            if (lane >= d) lk_incl += v;
        }
    };
    // the lane whose group holds row tile t publishes the group, the tile's
    // index in it and the group's row bounds
    auto lk_place = [&](int* st, int t, int gb, int carry) {
        const int start0 = carry + lk_incl - (lk_c0 + lk_c1);
        const int start1 = start0 + lk_c0;
        if (t >= start0 && t < start0 + lk_c0) {
            st[0] = gb + 2 * lane; st[1] = t - start0; st[3] = lk_o0; st[4] = lk_o1;
        }
        if (t >= start1 && t < start1 + lk_c1) {
            st[0] = gb + 2 * lane + 1; st[1] = t - start1; st[3] = lk_o1; st[4] = lk_o2;
        }
    };
    // wave 0: publish work item `item` in slot `slot` (group -1 if item >=
    // items).  Up to 128 groups the per-lane table comes back from LDS.
    auto lookup = [&](int item, int items, int slot) {
        int* st = s_tile[slot];
        const int t = item < items ? item / ntn : -1;
        if (lane == 0) { st[0] = -1; st[2] = item - (item / ntn) * ntn; }
        if (p.G <= 128) {
            lk_o0 = s_lk[0][lane]; lk_o1 = s_lk[1][lane]; lk_o2 = s_lk[2][lane];
            lk_c0 = s_lk[3][lane]; lk_c1 = s_lk[4][lane]; lk_incl = s_lk[5][lane];
            lk_place(st, t, 0, 0);
        } else {
            int carry = 0;
            for (int gb = 0; gb < p.G; gb += 128) {
                lk_load(gb);
                lk_scan();
                lk_place(st, t, gb, carry);
                carry += __shfl(lk_incl, 63, 64);
            }
        }
    };
    // read the published item (after a barrier); false if there is none.
    // The results are workgroup-uniform: kept in scalar registers, so the
    // copies' base addresses need no per-lane arithmetic.
    auto take_tile = [&](int slot) {
        const int* st = s_tile[slot];
        const int g = __builtin_amdgcn_readfirstlane(st[0]);
        if (g < 0) return false;
        const int lt = __builtin_amdgcn_readfirstlane(st[1]);
        m_begin = __builtin_amdgcn_readfirstlane(st[3]) + lt * BM;
        m_end = min(__builtin_amdgcn_readfirstlane(st[4]), m_begin + BM);
        n0 = __builtin_amdgcn_readfirstlane(st[2]) * (SWIGLU ? 128 : BN);   // SWIGLU: first h column
        bptr = p.b + (int64_t)g * p.b_sg;
        sbp = p.sb + (int64_t)g * p.sb_sg * ((MODE == MODE_MX || MODE == MODE_P2) ? 1 : 4);
        return true;
    };
    if (!GROUPED) {
        const int ntm = (p.M + BM - 1) / BM;
        const int nblk = ntn * ntm;
        const int bid = blockIdx.x;
        // consecutive tile ids on one XCD (workgroups are dealt round-robin to the 8 XCDs)
        const int per = nblk / 8;
        const int tile = bid < per * 8 ? (bid % 8) * per + bid / 8 : bid;
        // groups of GM m-tiles sweep n, so co-resident tiles share operand
        // panels in L2.  An XCD runs 32 tiles at a time, GM m-tiles x 32/GM
        // n-tiles, and fetches GM A panels (BM rows) and 32/GM B panels (BN
        // rows) per round: GM = 4 when BN < BM (160 x 256: 4 x 256 + 8 x 160
        // rows against 8 x 256 + 4 x 160), else 8.
        constexpr int GM = BN < BM ? 4 : 8;
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
        if (wave == 0) {
            // up to 128 groups: one load of the offsets serves both the
            // total and the prefix sums (and every later lookup)
            int total = 0;
            if (p.G <= 128) {
                lk_load(0);
                lk_scan();
                total = __shfl(lk_incl, 63, 64);
                s_lk[0][lane] = lk_o0; s_lk[1][lane] = lk_o1; s_lk[2][lane] = lk_o2;
                s_lk[3][lane] = lk_c0; s_lk[4][lane] = lk_c1; s_lk[5][lane] = lk_incl;
            } else {
                for (int gb = 0; gb < p.G; gb += 128) {
                    lk_load(gb);
                    int c = lk_c0 + lk_c1;
#pragma unroll
                    for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
                    total += c;
                }
            }
            // XCD x = bid % 8 owns items [x per, x per + per); its workgroups
            // take them in turn, 8 / gridDim apart
            const int items = total * ntn;
            const int per = (items + 7) / 8;
            const int bid = blockIdx.x;
            const int first = (bid % 8) * per + bid / 8;
            const int last = min((bid % 8) * per + per, items);
            if (lane == 0) { s_range[0] = first; s_range[1] = last; s_range[2] = items; }
            lookup(first < last ? first : items, items, 0);
        }
        __syncthreads();
        it_item = __builtin_amdgcn_readfirstlane(s_range[0]);
        it_end = __builtin_amdgcn_readfirstlane(s_range[1]);
        it_items = __builtin_amdgcn_readfirstlane(s_range[2]);
        if (!take_tile(0)) return;                 // uniform: no work item for this workgroup
    }
    // K slices of this workgroup: [kbase, kbase + nk).  Dense K split: grid
    // row y takes the y-th of ksplit contiguous ranges (the first
    // nk_all % ksplit ranges one slice longer).
    const int nk_all = p.K / BK;
    int kbase = 0, nk = nk_all;
    if (!GROUPED && p.ksplit > 1) {
        const int y = (int)blockIdx.y, per = nk_all / p.ksplit, extra = nk_all % p.ksplit;
        kbase = y * per + min(y, extra);
        nk = per + (y < extra ? 1 : 0);
    }
    auto arow = [&](int m_local) {             // physical A row of tile row m_local (clamped)
        int m = min(m_begin + m_local, m_end - 1);
        if (GATHER) m = p.a_rows[m];
        return m;
    };

    // ------------------------------------------------------- copy set-up
    // Wave w copies weight rows [8 kDmaB w, +8 kDmaB) and activation rows
    // [8 kDmaA w, +8 kDmaA), one instruction per 8 rows x 128 bytes.  Lane l
    // fetches logical chunk (l % 8) ^ f(row) of row 8 j + l / 8.  Copy slots
    // past the tile's kCopiesB weight copies repeat the first ones.
    uint32_t offB[C::kDmaB], offA[C::kDmaA];
    auto bcopy = [&](int t) { const int j = wave * C::kDmaB + t; return j < C::kCopiesB ? j : j - C::kCopiesB; };
    // Scale copies (4-byte lanes).  Activation scales: waves [0, BM/64) copy
    // rows [64 w, +64).  Weight scales: BLOCK128 / P2 -> wave (BM/64) % WAVES copies the
    // two 128-row blocks of the tile; ROW128 / MX -> waves [0, ceil(BN/64))
    // copy rows [64 w, +64) (the last piece may pass the tile's rows: they
    // land in the padded scale region and read clamped rows of B's scales).
    const bool has_sa = MODE != MODE_KINV && wave < BM / 64;
    const bool has_sb = MODE != MODE_KINV &&
                        ((MODE == MODE_BLOCK128 || MODE == MODE_P2) ? wave == (BM / 64) % WAVES : wave < (BN + 63) / 64);
    uint32_t sa_off = 0, sb_off = 0;            // byte offsets without the slice term (< 4 GiB)
    // BLOCK128 weight scales: the wave's n-tiles before nb_w lie in the
    // tile's first 128-row block, the rest in the next one.  Tiles span at
    // most two blocks: 256 rows start at multiples of 256, 160 rows at
    // multiples of 160 (block offsets 0..96) and 192 rows at multiples of
    // 192 (offsets 0 or 64).
    int nb_w = NF;
    // per-lane copy offsets of the tile at (m_begin, m_end, n0, bptr, sbp)
    auto setup_tile = [&]() {
#pragma unroll
        for (int j = 0; j < C::kDmaB; ++j) {
            const int row = bcopy(j) * 8 + (lane >> 3);
            const int chunk = (lane & 7) ^ swz(row);
            const int brow = !SWIGLU ? min(n0 + row, p.N - 1) : row < 128 ? n0 + row : p.swi + n0 + row - 128;
            offB[j] = (uint32_t)((int64_t)brow * p.ldb + chunk * 16);
        }
#pragma unroll
        for (int j = 0; j < C::kDmaA; ++j) {
            const int row = (wave * C::kDmaA + j) * 8 + (lane >> 3);
            const int chunk = (lane & 7) ^ swz(row);
            offA[j] = (uint32_t)((int64_t)arow(row) * p.lda + chunk * 16);
        }
        if (has_sa) {
            const int m = arow(wave * 64 + lane);
            sa_off = (uint32_t)((MODE == MODE_MX || MODE == MODE_P2) ? (int64_t)m * p.sa_sm : (int64_t)m * p.sa_sm * 4);
        }
        if (MODE == MODE_BLOCK128 || MODE == MODE_P2) {
            const int nb = !SWIGLU ? min(n0 / 128 + (lane & 1), (p.N - 1) / 128)
                                   : ((lane & 1) ? (p.swi + n0) / 128 : n0 / 128);   // gate block, up block
            sb_off = (uint32_t)((int64_t)nb * p.sb_sn * (MODE == MODE_P2 ? 1 : 4));
        } else if (MODE != MODE_KINV) {
            const int r = (wave & 3) * 64 + lane;          // tile row
            const int n = !SWIGLU ? min(n0 + r, p.N - 1) : r < 128 ? n0 + r : p.swi + n0 + r - 128;
            sb_off = (uint32_t)((MODE == MODE_MX) ? (int64_t)n * p.sb_sn : (int64_t)n * p.sb_sn * 4);
        }
        nb_w = NF == 8 ? NF : min(max(((n0 / 128 + 1) * 128 - (n0 + wn * 16 * NF)) / 16, 0), NF);
    };
    setup_tile();
    const uint32_t lds0 = lds_addr(smem);
    auto bstage = [&](int i) { return lds0 + (uint32_t)(i * C::kBStageBytes); };                      // weights + sb
    auto abuf = [&](int i) { return lds0 + (uint32_t)(C::kBStages * C::kBStageBytes + i * C::kABufBytes); };  // acts + sa
    // Copies of slice kb: the scale copies (wave-dependent, issued outside
    // the n-tile loop), the activation tile with its scales, and weight-tile
    // copy t of this wave.
    auto copy_sb = [&](int kb, int stage) {
        if (!has_sb) return;
        const uint32_t st = bstage(stage) + BN * BK;
        const int kg = kbase + kb;
        if (MODE == MODE_MX) dma4(sbp + kg * 4, sb_off, st + wave * 64 * 4);
        else if (MODE == MODE_P2) dma4(sbp + (kg >> 2) * 4, sb_off, st);   // slices 4(kg/4) .. +3
        else if (MODE == MODE_BLOCK128) dma4(sbp + kg * p.sb_sk * 4, sb_off, st);
        else dma4(sbp + kg * p.sb_sk * 4, sb_off, st + wave * 64 * 4);
    };
    auto copy_sa = [&](int kb, int buf) {
        if (!has_sa) return;
        const uint32_t st = abuf(buf) + BM * BK + wave * 64 * 4;
        const int kg = kbase + kb;
        if (MODE == MODE_MX) dma4(p.sa + kg * 4, sa_off, st);
        else if (MODE == MODE_P2) dma4(p.sa + (kg >> 2) * 4, sa_off, st);
        else dma4(p.sa + kg * p.sa_sk * 4, sa_off, st);
    };
    auto copy_a = [&](int kb, int buf, int t) {
        dma16(p.a + (kbase + kb) * BK, offA[t], abuf(buf) + (wave * C::kDmaA + t) * 8 * BK);
    };
    auto copy_b = [&](int kb, int stage, int t) {
        dma16(bptr + (kbase + kb) * BK, offB[t], bstage(stage) + bcopy(t) * 8 * BK);
    };

    v4f acc[NF][4];

    // Issue order (the waits rely on it): step kb issues the copies of
    // activation slice kb + kLeadA (scales right after the barriers, tile in
    // the first n-tile steps) and then those of weight slice kb + kLeadB; the
    // prologue issues the same sequence for the steps -kLeadMax..-1.
    auto prologue = [&]() {
#pragma unroll
        for (int j = -C::kLeadMax; j < 0; ++j) {
            const int sa_kb = j + C::kLeadA, sb_kb = j + C::kLeadB;
            if (sa_kb >= 0 && sa_kb < nk) {
                copy_sa(sa_kb, sa_kb % C::kAStages);
#pragma unroll
                for (int t = 0; t < C::kDmaA; ++t) copy_a(sa_kb, sa_kb % C::kAStages, t);
            }
            if (sb_kb >= 0 && sb_kb < nk) {
                copy_sb(sb_kb, sb_kb % C::kBStages);
#pragma unroll
                for (int t = 0; t < C::kDmaB; ++t) copy_b(sb_kb, sb_kb % C::kBStages, t);
            }
        }
    };
    prologue();

    // One K slice.  CA / CB (compile time): this step copies activation slice
    // kb + kLeadA / weight slice kb + kLeadB.  Both hold in every step but the
    // last one or two; keeping them constants leaves each n-tile step a single basic
    // block, so the sched_barrier below really bounds the scheduler (with a
    // branch per copy the compiler sank every matrix instruction below all
    // fragment reads).
    // ACT (compile time): the wave has rows of the tile inside the matrix
    // (or its group).  A wave without any issues only its share of the
    // copies and meets the barriers: on a ragged last tile of a group the
    // waves of the empty half then leave their SIMDs' matrix units to the
    // waves that have rows.
    auto step = [&](int kb, auto ca_tag, auto cb_tag, auto act_tag) {
        constexpr bool CA = decltype(ca_tag)::value, CB = decltype(cb_tag)::value;
        constexpr bool ACT = decltype(act_tag)::value;
        // Wait for this wave's copies of slice kb (scale copies were issued
        // before the tile copies of their step, so counting tile copies only
        // is conservative).
        if (kb + 1 < nk) {
            constexpr int n = C::kNAfter;
            __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        const int a_kb = kb + C::kLeadA, b_kb = kb + C::kLeadB;
        const int a_buf = a_kb % C::kAStages, cst = b_kb % C::kBStages;
        const uint32_t tB = bstage(kb % C::kBStages);
        const uint32_t tA = abuf(kb % C::kAStages);

        v8i fa[4];
        int mxa[4];
        float sam[4];
        auto read_a = [&]() {
            const FragOff ab = frag_base(tA + wm * 64 * BK, fo);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) fa[mt] = read_frag(ab, mt * 16 * BK);
            // activation-side scales of the wave's 4 m-tiles (bytes in MX mode)
            const uint32_t sa_lds = opaque(tA + BM * BK + (wm * 64 + r16) * 4);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (MODE == MODE_MX) mxa[mt] = lds_readu8(sa_lds + mt * 64 + q);
                else if (MODE == MODE_P2) mxa[mt] = lds_readu8(sa_lds + mt * 64 + ((kbase + kb) & 3));
                else if (MODE == MODE_KINV) mxa[mt] = 0;    // constant 0: the plain (unscaled) instruction, see mfma_unit
                else sam[mt] = lds_readf(sa_lds + mt * 64);
            }
        };
        // With one wave column (WN = 1) a wave's activation rows and their
        // scales are copied, read and refilled by that wave alone.  Its own
        // wait above then makes slice kb's rows readable, so the reads go out
        // before the barrier and overlap it (up projection and wgrad ~2%
        // faster, bit-identical).
        if constexpr (ACT && WN == 1) read_a();
        // Every wave's copies landed and every wave finished step kb-1, so
        // the buffers of slice kb-1 are free.  A plain s_barrier (with a compiler memory
        // clobber) rather than __syncthreads(): the latter's release fence
        // would also wait for copies still in flight.
        asm volatile("s_barrier" ::: "memory");
        if constexpr (ACT && WN != 1) read_a();
        if (C::kABarrier) {
            // This wave's activation fragments and scales are in registers.
            // With several wave columns, waves share activation rows, and
            // all of them must have read before the buffer is refilled; with
            // one, the wave's own reads are all that its refill waits for.
            __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
            if constexpr (WN != 1) asm volatile("s_barrier" ::: "memory");
        }
        if (CA) copy_sa(a_kb, a_buf);
        if (CB) copy_sb(b_kb, cst);
        // tile copies, placed in the n-tile steps given by Cfg
        auto copy_step = [&](int nt) {
#pragma unroll
            for (int t = 0; t < C::kDmaA; ++t)
                if (CA && t == nt) copy_a(a_kb, a_buf, t);
#pragma unroll
            for (int t = 0; t < C::kDmaB; ++t)
                if (CB && C::b_slot(t) == nt) copy_b(b_kb, cst, t);
        };

        if constexpr (!ACT) {
#pragma unroll
            for (int nt = 0; nt < NF; ++nt) copy_step(nt);
        } else if (MODE == MODE_MX || MODE == MODE_KINV || MODE == MODE_P2) {
            const uint32_t sb8 = opaque(tB + BN * BK + (wn * 16 * NF + r16) * 4 + q);
            // P2: the tile's two 128-row weight blocks, byte kb % 4 of each
            // block's copied word (chosen per n-tile as in BLOCK128)
            int pb0 = kE8M0One, pb1 = kE8M0One;
            if (MODE == MODE_P2) {
                const uint32_t sbw = tB + BN * BK + ((kbase + kb) & 3);
                pb0 = lds_readu8(sbw + (NF == 8 ? wn * 4 : 0));
                pb1 = NF == 8 ? pb0 : lds_readu8(sbw + 4);
            }
            const FragOff bb = frag_base(tB + wn * 16 * NF * BK, fo);
#pragma unroll
            for (int nt = 0; nt < NF; ++nt) {
                const v8i fb = read_frag(bb, nt * 16 * BK);
                const int mxb = MODE == MODE_KINV ? 0
                                : MODE == MODE_P2 ? ((NF == 8 || nt < nb_w) ? pb0 : pb1)
                                                  : lds_readu8(sb8 + nt * 64);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    acc[nt][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb, fa[mt], acc[nt][mt], 0, 0, 0,
                                                                                  mxb, 0, mxa[mt]);
                copy_step(nt);
                // keep the scheduler from hoisting every n-tile's fragment
                // reads to the top of the slice (8 fragments = 64 registers)
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            const uint32_t sbf = tB + BN * BK;
            // BLOCK128: a 256-row tile is two aligned 128-row blocks, one per
            // wave column; other tiles hold the tile's first block for the
            // wave's n-tiles before nb_w and the next block after it.
            float sc[4], sc1[4];
            if (MODE == MODE_BLOCK128) {
                const float sbv = lds_readf(sbf + (NF == 8 ? wn * 4 : 0));
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) sc[mt] = sam[mt] * sbv;
                if (NF != 8) {
                    const float sbv1 = lds_readf(sbf + 4);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) sc1[mt] = sam[mt] * sbv1;
                }
            }
            v4f part[2][4];
            f32x4 sbr[2];
            auto promote = [&](int pt, int ps) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (MODE == MODE_BLOCK128) {
                        const float s = (NF == 8 || pt < nb_w) ? sc[mt] : sc1[mt];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[pt][mt][r] = __builtin_fmaf(part[ps][mt][r], s, acc[pt][mt][r]);
                    } else {
                        const float s4[4] = {sbr[ps][0], sbr[ps][1], sbr[ps][2], sbr[ps][3]};
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[pt][mt][r] = __builtin_fmaf(part[ps][mt][r], sam[mt] * s4[r], acc[pt][mt][r]);
                    }
                }
            };
            const FragOff bb = frag_base(tB + wn * 16 * NF * BK, fo);
            const uint32_t sbr_lds = opaque(sbf + (wn * 16 * NF + 4 * q) * 4);
            v8i fb_next = read_frag(bb, 0);
#pragma unroll
            for (int nt = 0; nt < NF; ++nt) {
                const int ps = C::kDefer ? (nt & 1) : 0;
                const v8i fb = fb_next;
                if (nt < NF - 1) fb_next = read_frag(bb, (nt + 1) * 16 * BK);
                if (MODE == MODE_ROW128) sbr[ps] = lds_readf4(sbr_lds + nt * 64);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) part[ps][mt] = mfma_unit(fb, fa[mt]);
                copy_step(nt);
                if (!C::kDefer) promote(nt, 0);
                else if (nt > 0) promote(nt - 1, (nt - 1) & 1);
                if (C::kDefer && nt > 0) {
                    // issue order: one matrix instruction, then four of the
                    // promotion FMAs, four times, so that a wave running alone
                    // on its SIMD keeps the matrix unit busy while its vector
                    // FMAs issue (a block of four matrix instructions followed
                    // by sixteen FMAs leaves the unit idle during the FMAs)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (C::kDefer) promote(NF - 1, (NF - 1) & 1);
        }
    };
    // Grouped: one work item per trip; dense: one trip.  Wave 0 publishes the
    // next item at the start of each trip, in the slot not being read.
    for (;;) {
    if constexpr (GROUPED) {
        it_item += (int)(gridDim.x / 8);
        it_slot ^= 1;
        if (wave == 0) lookup(it_item < it_end ? it_item : it_items, it_items, it_slot);
    }
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    auto kloop = [&](auto act_tag) {
        int kb = 0;
        for (; kb + C::kLeadMax < nk; ++kb) step(kb, std::true_type{}, std::true_type{}, act_tag);
        // At most kLeadMax (<= 2) steps remain.  With unequal leads the next to
        // last step still copies the side with the longer lead; the last step
        // copies nothing.
        if constexpr (C::kLeadA != C::kLeadB) {
            if (kb + 2 == nk) {
                step(kb, std::integral_constant<bool, (C::kLeadA < C::kLeadB)>{},
                     std::integral_constant<bool, (C::kLeadB < C::kLeadA)>{}, act_tag);
                ++kb;
            }
        }
        for (; kb < nk; ++kb) step(kb, std::false_type{}, std::false_type{}, act_tag);
    };
    // grouped: the last row tile of a group is ragged (wave-uniform test:
    // m_begin, m_end and wm are); dense tiles keep the one loop
    if (!GROUPED || m_begin + wm * 64 < m_end) kloop(std::true_type{});
    else kloop(std::false_type{});

    // Grouped: take the next work item; its first copies go out in the
    // middle of this item's epilogue.  The barrier (LDS only: every wave has
    // finished reading the last slice, and wave 0 has published the item)
    // frees the first stages and the activation buffer; the epilogue stages
    // its outputs in weight stage 2, which the next item's first steps do
    // not fill.
    const int32_t em_begin = m_begin, em_end = m_end, en0 = n0;
    bool more = false;
    if constexpr (GROUPED) {
        lds_barrier();
        more = take_tile(it_slot);
    }

    // ---------------------------------------------------------- epilogue
    // N % 128 == 0: with 256-row tiles each wave covers 128 aligned n, so a
    // wave's columns are all inside the matrix or all outside; other tiles
    // check each 16-column n-tile (wave-uniform).  Rows are checked per lane.
    const int nw0 = en0 + wn * 16 * NF;
    const bool wave_out = nw0 < p.N;
    if (MODE == MODE_KINV && wave_out) {
        // scales constant along K: each output times sa(m) * sb(n), once
        const float* sa = reinterpret_cast<const float*>(p.sa);
        const float* sb = reinterpret_cast<const float*>(p.sb);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int m = min(em_begin + wm * 64 + mt * 16 + r16, em_end - 1);
            const float sam = sa[(int64_t)m * p.sa_sm];
#pragma unroll
            for (int nt = 0; nt < NF; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = min(nw0 + nt * 16 + 4 * q + r, p.N - 1);
                    const float sbn = sb[(int64_t)(p.kinv_row ? n : n / 128) * p.sb_sn];
                    acc[nt][mt][r] *= sam * sbn;
                }
        }
    }
    // The outputs leave through LDS so that every store writes whole rows:
    // a lane holds 4 consecutive columns of one row per 16 x 16 block, and
    // storing those directly makes each store instruction write 32-byte
    // pieces of 16 different rows.  Each wave stages its 64 x 16 NF block in
    // passes of kRows rows (row pitch padded by 16 bytes to spread the banks)
    // and reads it back in 16-byte pieces of consecutive columns.  Dense: the
    // staging uses the operand buffers, freed by a barrier, 32 rows a pass.
    // Grouped: it uses weight stage 2 (the next item's copies are already on
    // their way to the other buffers).  With bf16 output, 16 rows a pass:
    // waves 0-3 in weight stage 2 and waves 4-7 in a second region of the
    // same size (fewer passes, and for SiLU*mul fewer barriers between the
    // staging and the cross-wave reads of gate and up); with fp32 output,
    // 8 rows a pass in weight stage 2.  Each wave then touches only its own
    // staging region, whose LDS accesses complete in program order.
    constexpr int EB = OUTF32 ? 4 : 2;                 // output bytes per element
    constexpr bool kTwoRegions = GROUPED && !OUTF32 && WAVES == 8;  // 16 rows a pass in two regions
    constexpr int kRows = kTwoRegions ? 16 : GROUPED ? 8 : 32;   // rows per pass
    constexpr int kPitch = 16 * NF * EB + 16;          // staged row, bytes
    constexpr int kChunks = 16 * NF * EB / 16;         // 16-byte pieces per row
    constexpr int kStageWaves = kTwoRegions ? 4 : WAVES;    // waves per staging region
    static_assert(GROUPED ? (C::kBStages == 3 && kStageWaves * kRows * kPitch <= C::kBStageBytes)
                          : WAVES * kRows * kPitch <= C::kLdsBytes,
                  "epilogue staging fits its region");
    static_assert((kRows * kChunks) % 64 == 0, "whole store instructions per pass");
    if constexpr (!GROUPED) {
        __syncthreads();
        if (!wave_out) return;
    }
    const uint32_t ebase = GROUPED ? bstage(2) : lds0;
    uint32_t ebase2 = ebase;
    if constexpr (kTwoRegions) {
        // staging of waves 4-7 (wave rows 2 and 3); the other kernels do not
        // allocate it
        __shared__ __attribute__((aligned(16))) uint8_t s_stage2[kStageWaves * kRows * kPitch];
        ebase2 = lds_addr(s_stage2);
    }
    const uint32_t wst = (kTwoRegions && wave >= 4 ? ebase2 : ebase) + (uint32_t)((wave % kStageWaves) * kRows * kPitch);
    uint8_t* cbase = static_cast<uint8_t*>(p.c) + (int64_t)nw0 * EB + (GROUPED ? 0 : (int64_t)blockIdx.y * p.c_split);
    // SWIGLU tiles never leave the matrix (wave_out holds), so its barriers
    // are met by every wave
#pragma unroll
    for (int pass = 0; pass < 64 / kRows; ++pass) {
        if (GROUPED && pass == 64 / kRows / 2 && more) {
            // half of the accumulators are staged (and free): the next
            // item's copy offsets and first copies fit beside the rest
            setup_tile();
            prologue();
        }
        if (wave_out) {
#pragma unroll
            for (int h = 0; h < (kRows + 15) / 16; ++h) {
                const int mt = (pass * kRows) / 16 + h;
                const int ro = (pass * kRows) % 16;        // first m-tile row of the pass (kRows < 16)
                const uint32_t rowa = wst + (uint32_t)((h * 16 + r16 - ro) * kPitch + 4 * q * EB);
                if (kRows >= 16 || (r16 >= ro && r16 < ro + kRows)) {
#pragma unroll
                    for (int nt = 0; nt < NF; ++nt) {
                        const uint32_t a = rowa + nt * 16 * EB;
                        if (OUTF32) {
                            *reinterpret_cast<__attribute__((address_space(3))) f32x4*>((uintptr_t)a) =
                                f32x4{acc[nt][mt][0], acc[nt][mt][1], acc[nt][mt][2], acc[nt][mt][3]};
                        } else {
                            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>((uintptr_t)a) =
                                u32x2{pack_bf16x2(acc[nt][mt][0], acc[nt][mt][1]),
                                      pack_bf16x2(acc[nt][mt][2], acc[nt][mt][3])};
                        }
                    }
                }
            }
        }
        if constexpr (SWIGLU) {
            // h = bf16(silu(gate) * up) for the pass's rows of all four wave
            // rows, then each row's 128 h values form one 1x128 group.  The
            // gate half of wave row wr is staged by wave 2 wr, its up half by
            // wave 2 wr + 1, so every wave must have staged first.  Gate and
            // up are the bf16-rounded GEMM outputs and h uses the SiLU of the
            // separate SiLU*mul kernel, so codes and scales equal those of
            // the bf16 GEMM followed by fp8_silu_mul_quant.
            lds_barrier();
            const int sub = lane & 15;
            constexpr int kPerWave = 4 * kRows / WAVES;     // h rows per wave and pass
#pragma unroll
            for (int it = 0; it < kPerWave / 4; ++it) {
                const int R = wave * kPerWave + it * 4 + (lane >> 4);    // row of the pass, 0 .. 4 kRows - 1
                const int wr = R / kRows, rr = R % kRows;
                // waves 2 wr and 2 wr + 1 share a staging region
                const uint32_t ga = (wr < 2 ? ebase : ebase2) +
                                    (uint32_t)(2 * (wr & 1) * kRows * kPitch + rr * kPitch + sub * 16);
                const u32x4 gv = lds_read16(ga);
                const u32x4 uv = lds_read16(ga + kRows * kPitch);
                float v[8];
                uint32_t hb[8];
                silu_mul8_bf16(make_uint4(gv.x, gv.y, gv.z, gv.w), make_uint4(uv.x, uv.y, uv.z, uv.w), hb);
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(hb[i] << 16);
                const int m = em_begin + wr * 64 + pass * kRows + rr;
                uint32_t w0, w1;
                if (MODE == MODE_MX) {
                    // four 1x32 blocks per row: 4 lanes each, UE8M0 scales
                    // (the rule of the MX quantizer)
                    const float amax = quad_max_dpp(absmax8(v));
                    const int e = mx_exponent(amax);
                    const float f = pow2_neg(e);
                    if (amax == 0.0f) {
                        w0 = 0u; w1 = 0u;
                    } else {
                        w0 = enc4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
                        w1 = enc4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
                    }
                    if (m < em_end && (sub & 3) == 0)
                        static_cast<uint8_t*>(p.hs)[(int64_t)m * p.hs_sm + (int64_t)(en0 / 32 + (sub >> 2)) * p.hs_sg] =
                            (uint8_t)(e + 127);
                } else {
                    const float amax = row16_max_dpp(absmax8(v));
                    const float sc = amax / kE4M3Max;
                    encode8(v, sc, w0, w1);
                    if (m < em_end && sub == 0)
                        static_cast<float*>(p.hs)[(int64_t)m * p.hs_sm + (int64_t)(en0 / 128) * p.hs_sg] = sc;
                }
                if (m < em_end)
                    *reinterpret_cast<uint2*>(p.hq + (int64_t)m * p.ld_hq + en0 + sub * 8) = make_uint2(w0, w1);
            }
            lds_barrier();     // the next pass overwrites the staging regions
        } else if (wave_out) {
#pragma unroll
            for (int it = 0; it < kRows * kChunks / 64; ++it) {
                const int sidx = it * 64 + lane;
                const int row = sidx / kChunks, ch = sidx % kChunks;
                const u32x4 v = lds_read16(wst + (uint32_t)(row * kPitch + ch * 16));
                const int m = em_begin + wm * 64 + pass * kRows + row;
                const int col = ch * (16 / EB);
                if (m < em_end && (NF == 8 || nw0 + col < p.N)) {
                    // grouped outputs (the MoE layer's 400-540 MB) are larger
                    // than the last-level cache: streaming stores keep it for
                    // the operand panels still being reused (down GEMM 323 ->
                    // 310 us); dense outputs stay cached for the next layer
                    u32x4* dst = reinterpret_cast<u32x4*>(cbase + ((int64_t)m * p.ldc) * EB + col * EB);
                    if (GROUPED) __builtin_nontemporal_store(v, dst);
                    else *dst = v;
                }
            }
        }
    }
    if (!more) break;
    }
}

template <int MODE, bool GROUPED, int WAVES, int NF, int WN = 2>
hipError_t launch(const KArgs& p, bool out_f32, hipStream_t st) {
    using C = Cfg<WAVES, NF, false, WN>;
    dim3 grid;
    if (!GROUPED) {
        grid = dim3((unsigned)(((int64_t)(p.M + C::BM - 1) / C::BM) * ((p.N + C::BN - 1) / C::BN)),
                    (unsigned)(p.ksplit > 1 ? p.ksplit : 1));
    } else {
        // upper bound on the work items (row tiles over all groups x n-tiles),
        // rounded up to a multiple of the 8 XCDs
        const int64_t items = ((int64_t)(p.M + C::BM - 1) / C::BM + p.G) * ((p.N + C::BN - 1) / C::BN);
        grid = dim3((unsigned)std::min<int64_t>((items + 7) / 8 * 8, kCUs));
    }
    if (GROUPED && p.a_rows != nullptr) {
        if (out_f32)
            hipLaunchKernelGGL((k_gemm<MODE, GROUPED, true, WAVES, NF, WN, false, GROUPED>), grid, dim3(C::kThreads), 0,
                               st, p);
        else
            hipLaunchKernelGGL((k_gemm<MODE, GROUPED, false, WAVES, NF, WN, false, GROUPED>), grid, dim3(C::kThreads), 0,
                               st, p);
    } else if (out_f32) {
        hipLaunchKernelGGL((k_gemm<MODE, GROUPED, true, WAVES, NF, WN>), grid, dim3(C::kThreads), 0, st, p);
    } else {
        hipLaunchKernelGGL((k_gemm<MODE, GROUPED, false, WAVES, NF, WN>), grid, dim3(C::kThreads), 0, st, p);
    }
    return hipGetLastError();
}

// Tile choice by rounds of tiles over the 256 CUs: a 256 x 256 tile (8 waves)
// does twice the work of a 256 x 128 tile (4 waves) in about 4/3 of its time,
// so it wins unless it saves no round (small problems, where the smaller tile
// finishes first).  `extra_tiles` counts partial tiles of grouped problems.
int waves_for(int64_t rows, int64_t N, int64_t extra_tiles = 0) {
    const int64_t ntn = (N + 255) / 256;
    const int64_t r8 = (((rows + 255) / 256 + extra_tiles) * ntn + 255) / 256;
    const int64_t r4 = (((rows + 127) / 128 + extra_tiles) * ntn + 255) / 256;
    return 4 * r8 <= 3 * r4 ? 8 : 4;
}

// Dense BLOCK128 plans.  The output columns (weight rows) are cut into at
// most two regions, each tiled with one configuration, so that the tiles
// fill whole rounds over the compute units where a single tiling would
// leave most of a round idle (N 2560 at M 4096: 320 tiles of 128 x 256 or
// 160 of 256 x 256 for 256 CUs, against 256 tiles of 160 x 256).  The
// estimate per region is rounds x (K slices x cycles per slice + cycles per
// tile), with the cycle figures fitted to the MLP shapes (M 4096; N 9728,
// K 2560; N 2560, K 9728; and M 9728, N 2560, K 4096).  For the tiles sized
// two per CU a round is two tiles per CU; a last round of at most one tile
// per CU runs each tile at its lone speed (128 x 256: only about 12% faster
// per slice, as a lone 4-wave workgroup leaves each SIMD one wave).  The
// 160 x 128 pair is ~8% faster per slice than one 160 x 256 tile but costs
// ~4.7 us more per tile (K 9728 against K 4096, M 4096, N 2560): it wins
// with long K and full rounds (the down projection and dgrad), and its lone
// figure is the 192 x 128 tile's scaled by their measured ratio.
struct TileCfg {
    int waves, nf, wn, per_cu;
    double slice_cycles, tile_cycles;   // per round of tiles (per_cu = 2: two tiles per CU)
    double lone_slice_cycles;           // per_cu = 2: one tile on the CU
};
constexpr TileCfg kDenseCfgs[] = {
    {8, 8, 2, 1, 3300, 9000, 0},       // 256 x 256
    {4, 8, 2, 1, 2450, 7000, 0},       // 256 x 128
    {8, 5, 2, 1, 2520, 8000, 0},       // 160 x 256
    {4, 6, 2, 1, 2400, 6000, 0},       // 192 x 128
    {4, 8, 1, 2, 3100, 8000, 2700},    // 128 x 256, two per CU
    {4, 5, 2, 2, 2324, 18400, 2750},   // 160 x 128, two per CU
};
// A second launch on the stream: its ramp-up and the first region's tail.
constexpr double kLaunchCycles = 15000;

int64_t cfg_bn(const TileCfg& c) { return 16 * c.nf * c.wn; }
int64_t cfg_bm(const TileCfg& c) { return 64 * c.waves / c.wn; }

int64_t cfg_tiles(const TileCfg& c, int64_t M, int64_t N) {
    return ((M + cfg_bm(c) - 1) / cfg_bm(c)) * ((N + cfg_bn(c) - 1) / cfg_bn(c));
}

// `tiles` workgroups of nk slices each over the CUs
double units_cycles(const TileCfg& c, int64_t tiles, int64_t nk) {
    const double round = (double)nk * c.slice_cycles + c.tile_cycles;
    if (c.per_cu != 2) return (double)((tiles + kCUs - 1) / kCUs) * round;
    const int64_t full = tiles / (2 * kCUs), rest = tiles % (2 * kCUs);
    const double last = rest == 0 ? 0.0 : rest <= kCUs ? (double)nk * c.lone_slice_cycles + c.tile_cycles : round;
    return (double)full * round + last;
}

double region_cycles(const TileCfg& c, int64_t M, int64_t N, int64_t nk) {
    return units_cycles(c, cfg_tiles(c, M, N), nk);
}

struct DensePlan {
    int c1, c2;          // indices into kDenseCfgs; c2 < 0: one region
    int64_t split;       // first column of the second region (multiple of 128)
    double cycles;       // the estimate it was chosen by
};

DensePlan plan_dense(int64_t M, int64_t N, int64_t K) {
    const int64_t nk = K / BK;
    DensePlan best{0, -1, N, 0.0};
    double best_t = region_cycles(kDenseCfgs[0], M, N, nk);
    const int nc = (int)(sizeof(kDenseCfgs) / sizeof(kDenseCfgs[0]));
    for (int i = 0; i < nc; ++i) {
        const double t = region_cycles(kDenseCfgs[i], M, N, nk);
        if (t < best_t) { best_t = t; best = DensePlan{i, -1, N, 0.0}; }
        // region 1 in whole tiles of configuration i, on a 128-column boundary
        const int64_t bn = cfg_bn(kDenseCfgs[i]);
        for (int64_t split = bn; split < N; split += bn) {
            if (split % 128) continue;
            const double t1 = region_cycles(kDenseCfgs[i], M, split, nk);
            for (int j = 0; j < nc; ++j) {
                if (j == i) continue;
                const double tt = t1 + region_cycles(kDenseCfgs[j], M, N - split, nk) + kLaunchCycles;
                if (tt < best_t) { best_t = tt; best = DensePlan{i, j, split, 0.0}; }
            }
        }
    }
    best.cycles = best_t;
    return best;
}

// Dense K split.  With few output tiles and a long K (the decode-sized
// GEMMs of the rollout side: M of a few hundred tokens, K 9728), most CUs
// would idle while each tile walks every K slice.  The slices are divided
// into `splits` contiguous ranges, one per grid row; each writes its fp32
// partial tile to a workspace, and k_splitk_sum adds the partials in split
// order.  Priced as the tiles times `splits` workgroups of ceil(nk / splits)
// slices, plus the sum's traffic (read splits x M x N fp32, write M x N) at
// ~4 TB/s and a second launch.
constexpr double kSumBytesPerCycle = 2000.0;
constexpr int kMaxSplits = 32;

struct SplitPlan {
    int ci;              // configuration index (-1: no split, plan_dense)
    int splits;
    double cycles;
};

SplitPlan plan_split_cfg(int64_t M, int64_t N, int64_t nk, int splits, int out_bytes) {
    SplitPlan best{-1, splits, 1e300};
    const int nc = (int)(sizeof(kDenseCfgs) / sizeof(kDenseCfgs[0]));
    const int64_t nks = (nk + splits - 1) / splits;
    const double sum = ((double)splits * 4.0 + out_bytes) * (double)M * (double)N / kSumBytesPerCycle;
    for (int i = 0; i < nc; ++i) {
        const double t = units_cycles(kDenseCfgs[i], cfg_tiles(kDenseCfgs[i], M, N) * splits, nks) + sum + kLaunchCycles;
        if (t < best.cycles) best = SplitPlan{i, splits, t};
    }
    return best;
}

SplitPlan plan_splitk(int64_t M, int64_t N, int64_t K, int out_bytes) {
    const int64_t nk = K / BK;
    SplitPlan best{-1, 1, plan_dense(M, N, K).cycles};
    for (int s = 2; s <= kMaxSplits && s <= nk; ++s) {
        const SplitPlan t = plan_split_cfg(M, N, nk, s, out_bytes);
        if (t.cycles < best.cycles) best = t;
    }
    return best;
}

// c[m][n] = sum over splits s (in order) of ws[s][m][n]; one thread per 8
// consecutive outputs of a row (N % 128 == 0), rounded to bf16 or kept fp32.
template <bool OUTF32>
__global__ void __launch_bounds__(256) k_splitk_sum(const float* __restrict__ ws, int64_t split_elems, int32_t splits,
                                                    int64_t chunks, int32_t cpr, void* __restrict__ c, int64_t ldc) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= chunks) return;
    const int64_t m = i / cpr;
    const int64_t n = (i - m * cpr) * 8;
    const float* src = ws + m * ((int64_t)cpr * 8) + n;
    f32x4 a0 = *reinterpret_cast<const f32x4*>(src);
    f32x4 a1 = *reinterpret_cast<const f32x4*>(src + 4);
    for (int32_t sp = 1; sp < splits; ++sp) {
        const float* q = src + (int64_t)sp * split_elems;
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(q);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(q + 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) { a0[r] = a0[r] + b0[r]; a1[r] = a1[r] + b1[r]; }
    }
    if (OUTF32) {
        float* dst = static_cast<float*>(c) + m * ldc + n;
        *reinterpret_cast<f32x4*>(dst) = a0;
        *reinterpret_cast<f32x4*>(dst + 4) = a1;
    } else {
        uint16_t* dst = static_cast<uint16_t*>(c) + m * ldc + n;
        *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]),
                                                     pack_bf16x2(a1[0], a1[1]), pack_bf16x2(a1[2], a1[3]));
    }
}

template <int MODE>
hipError_t launch_dense(int ci, const KArgs& p, bool out_f32, hipStream_t st) {
    switch (ci) {
        case 0: return launch<MODE, false, 8, 8>(p, out_f32, st);
        case 1: return launch<MODE, false, 4, 8>(p, out_f32, st);
        case 2: return launch<MODE, false, 8, 5>(p, out_f32, st);
        case 3: return launch<MODE, false, 4, 6>(p, out_f32, st);
        case 4: return launch<MODE, false, 4, 8, 1>(p, out_f32, st);
        default: return launch<MODE, false, 4, 5, 2>(p, out_f32, st);
    }
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
    // scales constant along K: accumulate in the matrix unit, scale once
    const bool kinv = g.sa_sk == 0 && g.sb_sk == 0;
    p.kinv_row = g.bscale_row ? 1 : 0;
    auto go = [&](int ci, const KArgs& q) {
        if (kinv) return launch_dense<MODE_KINV>(ci, q, g.out_f32, st);
        if (g.bscale_row) return launch_dense<MODE_ROW128>(ci, q, g.out_f32, st);
        return launch_dense<MODE_BLOCK128>(ci, q, g.out_f32, st);
    };
    const DensePlan plan = plan_dense(g.M, g.N, g.K);
    if (plan.c2 < 0) return go(plan.c1, p);
    KArgs p1 = p, p2 = p;
    p1.N = (int32_t)plan.split;
    p2.N = (int32_t)(g.N - plan.split);
    p2.b = p.b + plan.split * p.ldb;
    p2.sb = p.sb + (g.bscale_row ? plan.split : plan.split / 128) * p.sb_sn * 4;
    p2.c = static_cast<uint8_t*>(p.c) + plan.split * (g.out_f32 ? 4 : 2);
    const hipError_t e = go(plan.c1, p1);
    if (e != hipSuccess) return e;
    return go(plan.c2, p2);
}

int32_t plan_gemm_splitk(int64_t M, int64_t N, int64_t K, bool out_f32) {
    return plan_splitk(M, N, K, out_f32 ? 4 : 2).splits;
}

hipError_t launch_gemm_blockscaled_splitk(const GemmArgs& g, int32_t splits, float* ws, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    if (splits <= 1) return launch_gemm_blockscaled(g, st);
    // the split GEMM: fp32 partial tiles into ws[split][M][N]
    KArgs p = base_args(g.M, g.N, g.K, g.a, g.lda, g.sa, g.b, g.ldb, g.sb, ws, g.N);
    p.sa_sm = g.sa_sm; p.sa_sk = g.sa_sk; p.sb_sn = g.sb_sn; p.sb_sk = g.sb_sk;
    p.kinv_row = g.bscale_row ? 1 : 0;
    p.ksplit = splits;
    p.c_split = g.M * g.N * 4;
    const int ci = plan_split_cfg(g.M, g.N, g.K / BK, splits, g.out_f32 ? 4 : 2).ci;
    hipError_t e;
    if (g.sa_sk == 0 && g.sb_sk == 0) e = launch_dense<MODE_KINV>(ci, p, true, st);
    else if (g.bscale_row) e = launch_dense<MODE_ROW128>(ci, p, true, st);
    else e = launch_dense<MODE_BLOCK128>(ci, p, true, st);
    if (e != hipSuccess) return e;
    const int32_t cpr = (int32_t)(g.N / 8);
    const int64_t chunks = g.M * cpr;
    const dim3 grid((unsigned)((chunks + 255) / 256));
    if (g.out_f32)
        hipLaunchKernelGGL(k_splitk_sum<true>, grid, dim3(256), 0, st, ws, g.M * g.N, splits, chunks, cpr, g.c, g.ldc);
    else
        hipLaunchKernelGGL(k_splitk_sum<false>, grid, dim3(256), 0, st, ws, g.M * g.N, splits, chunks, cpr, g.c, g.ldc);
    return hipGetLastError();
}

void plan_gemm_blockscaled(int64_t M, int64_t N, int64_t K, int32_t out[5]) {
    const DensePlan plan = plan_dense(M, N, K);
    out[0] = kDenseCfgs[plan.c1].waves;
    out[1] = (int32_t)cfg_bn(kDenseCfgs[plan.c1]);
    out[2] = plan.c2 < 0 ? 0 : kDenseCfgs[plan.c2].waves;
    out[3] = plan.c2 < 0 ? 0 : (int32_t)cfg_bn(kDenseCfgs[plan.c2]);
    out[4] = (int32_t)plan.split;
}

hipError_t launch_gemm_grouped(const GemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    KArgs p = base_args(g.M, g.N, g.K, g.a, g.lda, g.sa, g.b, g.ldb, g.sb, g.c, g.ldc);
    p.sa_sm = g.sa_sm; p.sa_sk = g.sa_sk; p.b_sg = g.b_sg; p.sb_sg = g.sb_sg; p.sb_sn = g.sb_sn; p.sb_sk = g.sb_sk;
    p.G = g.G; p.offsets = g.offsets; p.a_rows = g.a_rows;
    return waves_for(g.M, g.N, g.G / 2) == 8 ? launch<MODE_BLOCK128, true, 8, 8>(p, g.out_f32, st)
                                              : launch<MODE_BLOCK128, true, 4, 8>(p, g.out_f32, st);
}

hipError_t launch_gemm_grouped_swiglu(const GemmArgs& g, int64_t I, uint8_t* hq, int64_t ld_hq, float* hs,
                                      int64_t hs_sm, int64_t hs_sg, hipStream_t st) {
    if (g.M == 0 || I == 0) return hipSuccess;
    KArgs p = base_args(g.M, 2 * I, g.K, g.a, g.lda, g.sa, g.b, g.ldb, g.sb, nullptr, 0);
    p.sa_sm = g.sa_sm; p.sa_sk = g.sa_sk; p.b_sg = g.b_sg; p.sb_sg = g.sb_sg; p.sb_sn = g.sb_sn; p.sb_sk = g.sb_sk;
    p.G = g.G; p.offsets = g.offsets; p.a_rows = g.a_rows;
    p.swi = (int32_t)I; p.hq = hq; p.ld_hq = ld_hq; p.hs = hs; p.hs_sm = hs_sm; p.hs_sg = hs_sg;
    using C = Cfg<8, 8>;
    // upper bound on the work items (row tiles x 128-column blocks of h),
    // rounded up to a multiple of the 8 XCDs
    const int64_t items = ((int64_t)(g.M + C::BM - 1) / C::BM + g.G) * (I / 128);
    const dim3 grid((unsigned)std::min<int64_t>((items + 7) / 8 * 8, kCUs));
    if (p.a_rows != nullptr)
        hipLaunchKernelGGL((k_gemm<MODE_BLOCK128, true, false, 8, 8, 2, true, true>), grid, dim3(C::kThreads), 0, st, p);
    else
        hipLaunchKernelGGL((k_gemm<MODE_BLOCK128, true, false, 8, 8, 2, true>), grid, dim3(C::kThreads), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_gemm_mx_swiglu(const MxGemmArgs& g, int64_t I, uint8_t* hq, int64_t ld_hq, uint8_t* hs,
                                 int64_t hs_sm, int64_t hs_sg, hipStream_t st) {
    if (g.M == 0 || I == 0) return hipSuccess;
    KArgs p = base_args(g.M, 2 * I, g.K, g.a, g.lda, g.sa, g.b, g.ldb, g.sb, nullptr, 0);
    p.sa_sm = g.lds_a; p.sa_sk = 1; p.b_sg = g.b_sg; p.sb_sg = g.sb_sg; p.sb_sn = g.lds_b; p.sb_sk = 1;
    p.G = g.G; p.offsets = g.offsets; p.a_rows = g.a_rows;
    p.swi = (int32_t)I; p.hq = hq; p.ld_hq = ld_hq; p.hs = hs; p.hs_sm = hs_sm; p.hs_sg = hs_sg;
    using C = Cfg<8, 8>;
    const int64_t items = ((int64_t)(g.M + C::BM - 1) / C::BM + g.G) * (I / 128);
    const dim3 grid((unsigned)std::min<int64_t>((items + 7) / 8 * 8, kCUs));
    if (p.a_rows != nullptr)
        hipLaunchKernelGGL((k_gemm<MODE_MX, true, false, 8, 8, 2, true, true>), grid, dim3(C::kThreads), 0, st, p);
    else
        hipLaunchKernelGGL((k_gemm<MODE_MX, true, false, 8, 8, 2, true>), grid, dim3(C::kThreads), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_gemm_pow2(const Pow2GemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    KArgs p = base_args(g.M, g.N, g.K, g.a, g.lda, g.sa, g.b, g.ldb, g.sb, g.c, g.ldc);
    p.sa_sm = g.lds_a; p.sa_sk = 1; p.sb_sn = g.lds_b; p.sb_sk = 1;
    const DensePlan plan = plan_dense(g.M, g.N, g.K);
    if (plan.c2 < 0) return launch_dense<MODE_P2>(plan.c1, p, g.out_f32, st);
    KArgs p1 = p, p2 = p;
    p1.N = (int32_t)plan.split;
    p2.N = (int32_t)(g.N - plan.split);
    p2.b = p.b + plan.split * p.ldb;
    p2.sb = p.sb + (plan.split / 128) * p.sb_sn;
    p2.c = static_cast<uint8_t*>(p.c) + plan.split * (g.out_f32 ? 4 : 2);
    const hipError_t e = launch_dense<MODE_P2>(plan.c1, p1, g.out_f32, st);
    if (e != hipSuccess) return e;
    return launch_dense<MODE_P2>(plan.c2, p2, g.out_f32, st);
}

hipError_t launch_gemm_mx(const MxGemmArgs& g, hipStream_t st) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    KArgs p = base_args(g.M, g.N, g.K, g.a, g.lda, g.sa, g.b, g.ldb, g.sb, g.c, g.ldc);
    p.sa_sm = g.lds_a; p.sa_sk = 1; p.b_sg = g.b_sg; p.sb_sg = g.sb_sg; p.sb_sn = g.lds_b; p.sb_sk = 1;
    p.G = g.G; p.offsets = g.offsets; p.a_rows = g.a_rows;
    if (g.G == 0) {
        const DensePlan plan = plan_dense(g.M, g.N, g.K);
        if (plan.c2 < 0) return launch_dense<MODE_MX>(plan.c1, p, g.out_f32, st);
        KArgs p1 = p, p2 = p;
        p1.N = (int32_t)plan.split;
        p2.N = (int32_t)(g.N - plan.split);
        p2.b = p.b + plan.split * p.ldb;
        p2.sb = p.sb + plan.split * p.sb_sn;
        p2.c = static_cast<uint8_t*>(p.c) + plan.split * (g.out_f32 ? 4 : 2);
        const hipError_t e = launch_dense<MODE_MX>(plan.c1, p1, g.out_f32, st);
        if (e != hipSuccess) return e;
        return launch_dense<MODE_MX>(plan.c2, p2, g.out_f32, st);
    }
    return waves_for(g.M, g.N, g.G / 2) == 8 ? launch<MODE_MX, true, 8, 8>(p, g.out_f32, st)
                                              : launch<MODE_MX, true, 4, 8>(p, g.out_f32, st);
}

}  // namespace fp8bs
