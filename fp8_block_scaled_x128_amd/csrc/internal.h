// Internal launch interface between the C-ABI layer (capi.hip) and the kernel
// files.  Launchers assume their arguments were validated by capi.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

// quant.hip
hipError_t launch_quant_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                              int64_t ld_q, float* s, int64_t ssr, int64_t ssg, hipStream_t st);
hipError_t launch_quant_128x1_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qt,
                                int64_t ld_qt, float* s, int64_t ssr, int64_t ssg, hipStream_t st);
// X in 1x128 groups and W (rows w_rows, same cols) in 128x128 blocks, one launch.
hipError_t launch_quant_linear(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qx, int64_t ld_qx,
                               float* sx, int64_t ssr, int64_t ssg, const uint16_t* w, int64_t w_rows, int64_t ld_w,
                               uint8_t* qw, int64_t ld_qw, float* sw, hipStream_t st);
hipError_t launch_quant_128x128(const uint16_t* w, int64_t batch, int64_t rows, int64_t cols, int64_t ld_w,
                                uint8_t* q, int64_t ld_q, uint8_t* qt, int64_t ld_qt, float* s, hipStream_t st);
hipError_t launch_mx_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                           uint8_t* s, int64_t ssr, int64_t ssg, hipStream_t st);
hipError_t launch_mx_quant_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qt, int64_t ld_qt,
                             uint8_t* s, int64_t ssr, int64_t ssg, hipStream_t st);
// Row groups (1x128, or 1x32 MX) with row-major codes and column groups
// (128x1, or 32x1 MX) with transposed codes from one read of x.
hipError_t launch_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, bool mx, uint8_t* q,
                             int64_t ld_q, void* s, int64_t ssr, int64_t ssg, uint8_t* qt, int64_t ld_qt, void* st,
                             int64_t sstr, int64_t sstg, hipStream_t stream);
// Transposed copy of E4M3 codes, `batch` matrices [rows][ld_q] -> [cols][ld_qt].
hipError_t launch_transpose_codes(const uint8_t* q, int64_t batch, int64_t rows, int64_t cols, int64_t ld_q,
                                  uint8_t* qt, int64_t ld_qt, hipStream_t st);
hipError_t launch_silu_mul_quant(const uint16_t* gu, int64_t rows, int64_t I, int64_t ld_in, int mx, uint8_t* q,
                                 int64_t ld_q, void* s, int64_t ssr, int64_t ssg, uint16_t* h, int64_t ld_h,
                                 hipStream_t st);
hipError_t launch_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                                float* s, hipStream_t st);
hipError_t launch_quant_tensorwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                                   int64_t ld_q, float* s, hipStream_t st);
hipError_t launch_quant_pow2(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int block_rows, uint8_t* q,
                             int64_t ld_q, uint8_t* s, int64_t ld_s, hipStream_t st);
// Both operands with power-of-two block scales in one launch (as the two
// launch_quant_pow2 calls, block_rows 1 for X and 128 for W).
hipError_t launch_quant_linear_pow2(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qx,
                                    int64_t ld_qx, uint8_t* sx, int64_t ld_sx, const uint16_t* w, int64_t w_rows,
                                    int64_t ld_w, uint8_t* qw, int64_t ld_qw, uint8_t* sw, int64_t ld_sw,
                                    hipStream_t st);
hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t st);

// moe.hip
hipError_t launch_moe_combine(const uint16_t* y, int64_t rows, int64_t H, int64_t ld_y, const int32_t* pos,
                              const float* w, int64_t T, int32_t k, void* out, int64_t ld_out, int out_f32,
                              hipStream_t st);

// gemm.hip
struct GemmArgs {
    int64_t M, N, K;                 // M = total rows (grouped: rows of all groups)
    const uint8_t* a; int64_t lda;
    const float* sa; int64_t sa_sm, sa_sk;
    const uint8_t* b; int64_t ldb; int64_t b_sg;          // b_sg: expert stride (grouped)
    const float* sb; int64_t sb_sg, sb_sn, sb_sk;
    int bscale_row;                  // 0: sb indexed by n/128, 1: by n
    void* c; int64_t ldc; int out_f32;
    int32_t G; const int32_t* offsets; const int32_t* a_rows;   // grouped only
};
hipError_t launch_gemm_blockscaled(const GemmArgs& g, hipStream_t st);
// Tiling of a dense BLOCK128 problem: waves and weight rows per tile of the
// two column regions, and the first column of the second (N if one region).
void plan_gemm_blockscaled(int64_t M, int64_t N, int64_t K, int32_t out[5]);
// The same GEMM with its K slices divided among `splits` grid rows: fp32
// partials into ws[splits][M][N], then their sum in split order into c.
hipError_t launch_gemm_blockscaled_splitk(const GemmArgs& g, int32_t splits, float* ws, hipStream_t st);
// The split count the planner chooses (1: no split).
int32_t plan_gemm_splitk(int64_t M, int64_t N, int64_t K, bool out_f32);
hipError_t launch_gemm_grouped(const GemmArgs& g, hipStream_t st);
// Grouped gate/up GEMM (B = [G][2I][K], gate rows then up rows) whose epilogue
// forms h = bf16(silu(gate) * up) from the bf16-rounded outputs and writes
// h's 1x128 FP8 codes hq [M][ld_hq] and scales hs[m * hs_sm + g * hs_sg].
hipError_t launch_gemm_grouped_swiglu(const GemmArgs& g, int64_t I, uint8_t* hq, int64_t ld_hq, float* hs,
                                      int64_t hs_sm, int64_t hs_sg, hipStream_t st);

struct MxGemmArgs {
    int64_t M, N, K;
    const uint8_t* a; int64_t lda; const uint8_t* sa; int64_t lds_a;
    const uint8_t* b; int64_t ldb; int64_t b_sg; const uint8_t* sb; int64_t lds_b; int64_t sb_sg;
    void* c; int64_t ldc; int out_f32;
    int32_t G; const int32_t* offsets; const int32_t* a_rows;
};
hipError_t launch_gemm_mx(const MxGemmArgs& g, hipStream_t st);
// Grouped MXFP8 gate/up GEMM (B = [G][2I][K]) whose epilogue forms h =
// bf16(silu(gate) * up) and writes its 1x32 codes hq and UE8M0 scales
// hs[m * hs_sm + (j / 32) * hs_sg].
hipError_t launch_gemm_mx_swiglu(const MxGemmArgs& g, int64_t I, uint8_t* hq, int64_t ld_hq, uint8_t* hs,
                                 int64_t hs_sm, int64_t hs_sg, hipStream_t st);

// Block-wise GEMM with power-of-two UE8M0 scales: sa(m, kb) = sa[m * lds_a + kb],
// sb(n / 128, kb) = sb[(n / 128) * lds_b + kb] (bytes).
struct Pow2GemmArgs {
    int64_t M, N, K;
    const uint8_t* a; int64_t lda; const uint8_t* sa; int64_t lds_a;
    const uint8_t* b; int64_t ldb; const uint8_t* sb; int64_t lds_b;
    void* c; int64_t ldc; int out_f32;
};
hipError_t launch_gemm_pow2(const Pow2GemmArgs& g, hipStream_t st);

}  // namespace fp8bs
