/*
 * fp8bs: block-wise FP8 linear layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfp8bs.so.  The layer is the one the pages describe as shared by
 * RL rollout and training ("Low Precision RL", miles.radixark.com, section
 * "Unified training recipe" and section "2. Unified block-wise FP8
 * (DeepSeek-style)"): quantize activations per token and weights per
 * 128x128 block to E4M3 with FP32 scales, then run an FP8 GEMM that applies
 * the two scales once per 128-wide slice of the contraction axis, with FP32
 * accumulation.  The MXFP8 variant (1x32 blocks, UE8M0 scales) follows
 * section "3. Unified MXFP8 (Blackwell)" of the same page.
 *
 * Quantizer definition ("Unified FP8: Beyond Mixed Precision...",
 * winzheng.com, section "FP8 Quantization", Steps 1 and 2): per group,
 *     S = max|x| / 448          (IEEE fp32 division; 448 = largest E4M3FN value)
 *     q = E4M3(x / S)           (one IEEE fp32 division, then round to nearest
 *                                even, saturating to +-448)
 * An all-zero group has S = 0 and all codes 0x00.  FP8 codes are OCP E4M3FN
 * bytes.  Inputs are expected to be finite; NaN/Inf inputs give unspecified
 * codes.
 *
 * Conventions shared by every entry point
 *  - Every buffer argument is a device pointer owned by the caller.  The
 *    library never allocates, frees or synchronizes.
 *  - Every call is asynchronous on the caller's HIP stream `stream`
 *    (0 = the null stream) and returns once its kernels are enqueued.
 *  - Arguments are validated on the host before anything is launched; on a
 *    validation error nothing is launched and no output is touched.
 *  - FP8BS_ERR_DEVICE reports a launch error or a current device that is not
 *    gfx950; faults inside a kernel surface at the caller's next sync.
 *  - bf16 tensors are passed as uint16_t bit patterns, FP8 as uint8_t codes.
 *  - Strides and leading dimensions are in elements.  Matrices are row-major.
 *  - Scale arrays are addressed through two strides so the caller chooses
 *    their layout: the scale of (row r, group g) lives at
 *    s[r * s_stride_row + g * s_stride_group].  The GEMMs read activation
 *    scales fastest when s_stride_row == 1 ("M-major", [groups][rows]).
 *  - Calls are thread-safe and keep no state between calls apart from the
 *    per-device code-object load on first use.  The one exception is
 *    fp8_blockscaled_gemm_splitk_noalloc: its partials live in a device array
 *    that the library holds on each GPU, shared by every such call there
 *    (calls that overlap on one GPU race; see its declaration).
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8BS_OK = 0,
    FP8BS_ERR_NULL = 1,        /* a required pointer is NULL                          */
    FP8BS_ERR_SHAPE = 2,       /* a size is negative, or K % 128 (K % 32 for MX) != 0, ... */
    FP8BS_ERR_STRIDE = 3,      /* a leading dimension is smaller than the row length  */
    FP8BS_ERR_ALIGN = 4,       /* a base pointer or leading dimension breaks 16-byte alignment */
    FP8BS_ERR_UNSUPPORTED = 5, /* an enum value or a combination this build does not handle */
    FP8BS_ERR_DEVICE = 6       /* current device is not gfx950, or a launch failed    */
} fp8bs_status;

typedef enum {
    FP8BS_AXIS_ROW = 0,  /* 1x128 groups along the contiguous (column) axis: per-token activations */
    FP8BS_AXIS_COL = 1   /* 128x1 groups along the row (token) axis; q is written transposed       */
} fp8bs_axis;

typedef enum { FP8BS_OUT_BF16 = 0, FP8BS_OUT_FP32 = 1 } fp8bs_out;

typedef enum {
    FP8BS_BSCALE_BLOCK128 = 0, /* B scale per 128x128 block: index (n / 128, k / 128)   */
    FP8BS_BSCALE_ROW128 = 1    /* B scale per row and 128-wide K slice: index (n, k / 128) */
} fp8bs_bscale;

/* ------------------------------------------------------------------------
 * fp8_quant_rowblock -- per-token (1x128) or token-axis (128x1) quantization.
 *
 * x      : bf16 [rows][ld_x] (row-major), cols <= ld_x.
 * axis   : FP8BS_AXIS_ROW: groups are 1x128 runs of a row ("per-token"
 *          activations and gradients, "Unified FP8...", section "FP8
 *          Quantization", bullet list).  q is [rows][ld_q]; the scale of
 *          (row r, group g = col / 128) is s[r * s_stride_row + g * s_stride_group],
 *          g < ceil(cols / 128).
 *          FP8BS_AXIS_COL: groups are 128x1 runs of a column (128 consecutive
 *          tokens), for the operands of the weight-gradient GEMM whose
 *          contraction runs over tokens.  q is written transposed, [cols][ld_q]
 *          with the token axis contiguous; the scale of (column c, group
 *          g = row / 128) is s[c * s_stride_row + g * s_stride_group].
 *          This equals FP8BS_AXIS_ROW applied to the transpose of x.
 * The last group of a row (column) covers only the elements present.
 * Requirements: rows, cols >= 0; cols % 8 == 0, ld_x % 8 == 0 and x 16-byte
 * aligned; AXIS_ROW: ld_q >= cols, ld_q % 8 == 0, q 8-byte aligned;
 * AXIS_COL: rows % 16 == 0, ld_q >= rows, ld_q % 16 == 0, q 16-byte aligned.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_quant_rowblock(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                fp8bs_axis axis, uint8_t* q, int64_t ld_q,
                                float* s, int64_t s_stride_row, int64_t s_stride_group,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_quant_rowwise / fp8_quant_tensorwise -- one group per row, or one group
 * for the whole tensor: the coarser granularities named next to the
 * block-wise one ("per-tensor" in "Unified FP8: Beyond Mixed Precision...",
 * section "FP8 Quantization"; the tensorwise and rowwise scalings compared
 * with blockwise in "Towards Full Pipeline FP8 Reinforcement Learning for
 * LLMs").  The same two steps: S = max|x| / 448 over the group (fp32 IEEE
 * division), codes E4M3(x / S) (RNE, saturating); an all-zero group has
 * S = 0 and codes 0x00.
 *
 * x : bf16 [rows][ld_x];  q : [rows][ld_q] codes.
 * s : rowwise: fp32 [rows], s[r] the scale of row r;
 *     tensorwise: fp32 [1] (it holds the running maximum of the per-block
 *     scales while the call's kernels run, the tensor's scale when they end:
 *     fl(m / 448) is monotone in m).
 * Requirements: rows, cols >= 0; cols % 8 == 0; x 16-byte aligned with
 * ld_x % 8 == 0, ld_x >= cols; q 8-byte aligned with ld_q % 8 == 0,
 * ld_q >= cols.  The GEMM takes these scales as scales constant along K:
 * sa_stride_k = sb_stride_k = 0 in fp8_blockscaled_gemm (and
 * sa_stride_m = 0 or sb_stride_n = 0 for a tensorwise operand).
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                               uint8_t* q, int64_t ld_q, float* s, hipStream_t stream);
fp8bs_status fp8_quant_tensorwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                  uint8_t* q, int64_t ld_q, float* s, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_quant_block2d -- 128x128 block quantization of `batch` matrices
 * (weights: "Low Precision RL", table "Choose a precision" and section
 * "2. Unified block-wise FP8 (DeepSeek-style)").
 *
 * w   : bf16 [batch][rows][ld_w]; matrix b starts at w + b * rows * ld_w.
 * q   : [batch][rows][ld_q] codes; may be NULL when q_t is given (a caller
 *       that needs only the transposed copy, e.g. a weight stored [in][out]
 *       or the data-gradient operand, then writes no row-major codes).
 * q_t : nullable; if given, the transposed codes [batch][cols][ld_qt]
 *       (the same codes, so a GEMM contracting over `rows` reads them with
 *       the same block scales transposed).  At least one of q and q_t.
 * s   : [batch][ceil(rows/128)][ceil(cols/128)] fp32, contiguous; the scale of
 *       block (i, j) of matrix b is s[(b * nbr + i) * nbc + j].
 * Requirements: batch >= 1; rows, cols >= 0; cols % 8 == 0 and ld_w % 8 == 0;
 * w 16-byte aligned; if q: ld_q >= cols, ld_q % 8 == 0; if q_t: rows % 16 == 0,
 * ld_qt >= rows, ld_qt % 16 == 0, q_t 16-byte aligned.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_quant_block2d(const uint16_t* w, int64_t batch, int64_t rows, int64_t cols, int64_t ld_w,
                               uint8_t* q, int64_t ld_q, uint8_t* q_t, int64_t ld_qt,
                               float* s, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_transpose_codes -- the transposed copy of `batch` matrices of E4M3
 * codes: q_t[b][c][r] = q[b][r][c].  A 128x128 block scale is the same for a
 * block and its transpose, so the codes and scales that fp8_quant_block2d or
 * fp8_quant_linear wrote for a weight W in the forward pass give the
 * data-gradient GEMM dX = dY W its operand W^T (codes from here, the same
 * scales read with swapped strides) without reading the bf16 weight again
 * ("Low Precision RL", section "2. Unified block-wise FP8 (DeepSeek-style)":
 * 128x128 weight blocks, used by the forward and the backward GEMMs).
 *
 * q   : [batch][rows][ld_q] codes.   q_t : [batch][cols][ld_qt] codes.
 * Requirements: batch >= 1; rows % 16 == 0 and cols % 16 == 0; q and q_t
 * 16-byte aligned with ld_q % 16 == 0, ld_q >= cols, ld_qt % 16 == 0,
 * ld_qt >= rows; q and q_t must not overlap.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_transpose_codes(const uint8_t* q, int64_t batch, int64_t rows, int64_t cols, int64_t ld_q,
                                 uint8_t* q_t, int64_t ld_qt, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_quant_linear -- both operands of one block-wise FP8 linear layer in
 * one launch: the activation X [rows][cols] in 1x128 per-token groups and
 * the weight W [w_rows][cols] in 128x128 blocks, each with the scale
 * S = max|x| / 448 of its group and codes E4M3(x / S) ("Unified FP8: Beyond
 * Mixed Precision...", section "FP8 Quantization"; groupings of "Low
 * Precision RL", table "Choose a precision").  The results are identical
 * to fp8_quant_rowblock(x, ..., FP8BS_AXIS_ROW, qx, ld_qx, sx, ...) followed
 * by fp8_quant_block2d(w, 1, w_rows, cols, ...) without a transposed copy;
 * one grid carries both, so their memory traffic overlaps and the pair
 * costs one launch.
 *
 * x, qx, sx : as x, q, s of fp8_quant_rowblock with FP8BS_AXIS_ROW
 *             (scale of row r, group g at sx[r * sx_stride_row +
 *             g * sx_stride_group]).
 * w, qw, sw : as w, q, s of fp8_quant_block2d with batch 1 (sw is
 *             [ceil(w_rows/128)][ceil(cols/128)], contiguous).
 * Either operand may be empty (rows == 0 or w_rows == 0; its pointers are
 * then not read).  Requirements: as the two calls above; the buffers of
 * the two operands must not overlap.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_quant_linear(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                              uint8_t* qx, int64_t ld_qx, float* sx, int64_t sx_stride_row, int64_t sx_stride_group,
                              const uint16_t* w, int64_t w_rows, int64_t ld_w,
                              uint8_t* qw, int64_t ld_qw, float* sw, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_blockscaled_gemm -- C = A B^T with block scales, FP32 accumulation.
 *
 *   C[m, n] = sum_kb (sa(m, kb) * sb(n, kb)) * sum_{k in kb} dec(a[m, k]) dec(b[n, k])
 *
 * over 128-wide K slices kb, the per-slice scale product applied to the FP32
 * partial of each slice (the GEMM the rollout and the trainer forward share,
 * "Low Precision RL", section "Unified training recipe").
 *
 * a  : [M][lda] E4M3 codes, K contiguous.      sa(m, kb) = sa[m * sa_stride_m + kb * sa_stride_k]
 * b  : [N][ldb] E4M3 codes, K contiguous.      sb(n, kb) = sb[r * sb_stride_n + kb * sb_stride_k]
 *      with r = n / 128 (FP8BS_BSCALE_BLOCK128) or r = n (FP8BS_BSCALE_ROW128).
 *      B is always [N][K] with K contiguous; there is no [K][N] layout flag.
 *      The data-gradient GEMM dX = dY W reads W through the transposed copy
 *      q_t of fp8_quant_block2d (the same codes, written once per weight
 *      quantization: 1 more byte per weight element) and W's 128x128 scales
 *      with the two strides swapped (the blocks are transpose-invariant).
 * c  : [M][ldc] bf16 (round to nearest even) or fp32, per `out`.
 * Scales constant along K (sa_stride_k == 0 and sb_stride_k == 0: the
 * rowwise and tensorwise scalings of fp8_quant_rowwise/_tensorwise, or any
 * other K-invariant scale) take a path on which the matrix unit accumulates
 * the whole contraction and sa * sb multiplies each output once; with the
 * same product in every slice this is the formula above.
 * Requirements: M, N >= 0; K % 128 == 0; N % 128 == 0; lda >= K, ldb >= K,
 * lda % 16 == 0, ldb % 16 == 0, a and b 16-byte aligned; ldc >= N.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_blockscaled_gemm(int64_t M, int64_t N, int64_t K,
                                  const uint8_t* a, int64_t lda,
                                  const float* sa, int64_t sa_stride_m, int64_t sa_stride_k,
                                  const uint8_t* b, int64_t ldb,
                                  const float* sb, int64_t sb_stride_n, int64_t sb_stride_k,
                                  fp8bs_bscale bscale,
                                  void* c, int64_t ldc, fp8bs_out out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_blockscaled_gemm_plan -- the tiling fp8_blockscaled_gemm launches for
 * an FP8BS_BSCALE_BLOCK128 problem of this shape.  Host only: launches
 * nothing and needs no device.  (A description of the launch, not an
 * operation of the layer.)
 *
 * plan : int32[5], written on FP8BS_OK:
 *   plan[0], plan[1]  waves per workgroup and weight rows (n) per tile for
 *                     output columns [0, plan[4]);
 *   plan[2], plan[3]  the same for columns [plan[4], N), or 0, 0 when one
 *                     tiling covers all columns (then plan[4] == N);
 *   a tile covers 32 * waves activation rows (m), except the tile of 128
 *   weight rows (4 waves, two workgroups per compute unit), which covers
 *   256.  The 4-wave tile of 160 weight rows also runs two workgroups per
 *   compute unit.
 * Requirements: M, N, K >= 0; K % 128 == 0; N % 128 == 0.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_blockscaled_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t* plan);

/* ------------------------------------------------------------------------
 * fp8_blockscaled_gemm_splitk -- fp8_blockscaled_gemm (same formula, modes,
 * arguments and requirements) with its 128-wide K slices divided into
 * `splits` contiguous ranges, for problems with few output tiles and a long
 * K: the decode-sized GEMMs of the rollout side that the pages' recipe shares
 * with the trainer ("Low Precision RL", section "Unified training recipe"),
 * where one range per tile would leave most of the GPU idle.  Range s (the
 * first (K/128) % splits ranges hold one slice more) accumulates its
 * per-slice-scaled FP32 partials, exactly as fp8_blockscaled_gemm does over
 * all slices, into ws[s][M][N]; a second kernel adds the ranges in order
 * s = 0, 1, ... in FP32 and rounds to c (bf16, nearest even) or stores it
 * (fp32).  The sum differs from fp8_blockscaled_gemm only in FP32 rounding
 * order: it is deterministic, and identical wherever every partial is exact.
 *
 * splits   : 1 .. K/128 (1: exactly fp8_blockscaled_gemm, ws unused), or 0:
 *            the count fp8_blockscaled_gemm_splitk_plan gives.
 * ws       : device fp32 workspace owned by the caller, 16-byte aligned, at
 *            least splits * M * N * 4 bytes (ws_bytes); its contents on entry
 *            are ignored and on return undefined.  Calls that overlap in time
 *            need separate workspaces.
 * Errors   : those of fp8_blockscaled_gemm; FP8BS_ERR_SHAPE for splits < 0,
 *            splits > K/128 or ws_bytes too small; FP8BS_ERR_NULL for a NULL
 *            ws when splits > 1.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_blockscaled_gemm_splitk(int64_t M, int64_t N, int64_t K,
                                         const uint8_t* a, int64_t lda,
                                         const float* sa, int64_t sa_stride_m, int64_t sa_stride_k,
                                         const uint8_t* b, int64_t ldb,
                                         const float* sb, int64_t sb_stride_n, int64_t sb_stride_k,
                                         fp8bs_bscale bscale, void* c, int64_t ldc, fp8bs_out out,
                                         int32_t splits, float* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_blockscaled_gemm_splitk_noalloc -- fp8_blockscaled_gemm_splitk without
 * the workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It allocates nothing: the partials go to a scratch array of
 * 64 MiB (67,108,864 bytes) that the library holds on each GPU for the life
 * of the process; the first call on a device looks up that device's copy.
 * splits * M * N * 4 bytes must fit it: splits == 0 takes the planner's count
 * capped to what fits (1, no split, if two do not), and an explicit count
 * that does not fit is rejected with FP8BS_ERR_SHAPE.  Results are those of
 * fp8_blockscaled_gemm_splitk with the same split count.  Calls that overlap
 * in time on one GPU share the scratch and race: serialize them (one stream,
 * or events between streams).
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_blockscaled_gemm_splitk_noalloc(int64_t M, int64_t N, int64_t K,
                                                 const uint8_t* a, int64_t lda,
                                                 const float* sa, int64_t sa_stride_m, int64_t sa_stride_k,
                                                 const uint8_t* b, int64_t ldb,
                                                 const float* sb, int64_t sb_stride_n, int64_t sb_stride_k,
                                                 fp8bs_bscale bscale, void* c, int64_t ldc, fp8bs_out out,
                                                 int32_t splits, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_blockscaled_gemm_splitk_plan -- the split count the planner chooses
 * for this shape and output type (1 when splitting does not pay: the
 * estimate prices the extra partial traffic and the second launch against
 * the idle compute units of one range per tile) and the workspace it needs
 * (0 when splits == 1).  Host only: launches nothing and needs no device.
 * Requirements: M, N, K >= 0; K % 128 == 0; N % 128 == 0.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_blockscaled_gemm_splitk_plan(int64_t M, int64_t N, int64_t K, fp8bs_out out,
                                              int32_t* splits, size_t* ws_bytes);

/* ------------------------------------------------------------------------
 * fp8_grouped_gemm -- the block-scaled GEMM over G expert groups of rows
 * (the MoE layers the pages run the recipe on, Qwen3-30B-A3B, "Low
 * Precision RL", table "Choose a precision").
 *
 * offsets : device int32 [G + 1]; rows offsets[g] .. offsets[g+1]-1 of the
 *           output belong to expert g.  offsets[0] == 0, non-decreasing,
 *           offsets[G] == total_rows; empty groups are allowed.  The offsets
 *           stay on the device (no host synchronization); a violation of this
 *           contract is not detected.
 * a_rows  : nullable device int32 [total_rows]; if given, output row r reads
 *           A row a_rows[r] (and its scales) -- the MoE dispatch gather fused
 *           into the GEMM's operand load.  Every entry must be in [0, a_count).
 * a, sa   : as in fp8_blockscaled_gemm, a has a_count rows (a_count = total_rows
 *           when a_rows is NULL).
 * b       : expert g's [N][ldb] codes start at b + g * b_stride_g.
 * sb      : 128x128 block scales; expert g, block (n/128, kb) at
 *           sb[g * sb_stride_g + (n/128) * sb_stride_n + kb * sb_stride_k].
 * c       : [total_rows][ldc], bf16 or fp32.
 * The schedule needs no workspace: every workgroup derives its work items
 * from the device offsets (see fp8_grouped_gemm_ws_size).
 * Requirements: as fp8_blockscaled_gemm; G >= 1; b_stride_g % 16 == 0.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_grouped_gemm(int64_t total_rows, int64_t N, int64_t K, int32_t G,
                              const int32_t* offsets, const int32_t* a_rows, int64_t a_count,
                              const uint8_t* a, int64_t lda,
                              const float* sa, int64_t sa_stride_m, int64_t sa_stride_k,
                              const uint8_t* b, int64_t ldb, int64_t b_stride_g,
                              const float* sb, int64_t sb_stride_g, int64_t sb_stride_n, int64_t sb_stride_k,
                              void* c, int64_t ldc, fp8bs_out out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_grouped_gemm_ws_size -- device workspace, in bytes, that the grouped
 * GEMMs (fp8_grouped_gemm, fp8_grouped_gemm_swiglu_quant, grouped
 * mxfp8_gemm and mxfp8_grouped_gemm_swiglu_quant) need for a problem of at
 * most max_total_rows rows over G groups with N output columns.  Always 0:
 * the persistent workgroups find each work item's group with a prefix scan
 * of the per-group tile counts, read from the device offsets, so the
 * scheduler keeps no table in memory and the calls take no workspace
 * argument.  Kept so that a caller can size (and skip) a workspace from the
 * problem statement alone.  Host only; launches nothing.
 * bytes : written on FP8BS_OK.
 * Requirements: max_total_rows >= 0, G >= 1, N >= 0; bytes not NULL.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_grouped_gemm_ws_size(int64_t max_total_rows, int32_t G, int64_t N, size_t* bytes);

/* ------------------------------------------------------------------------
 * fp8_grouped_gemm_swiglu_quant -- the MoE expert gate/up GEMM
 * (fp8_grouped_gemm) with the step that follows it, SiLU*mul and the 1x128
 * re-quantization of h (fp8_silu_mul_quant, mx == 0), in the GEMM's
 * epilogue: for callers who need only h's codes and scales (the operand of
 * the down GEMM).
 *
 * Per expert g and row m of its group, with GU = the block-scaled product of
 * fp8_grouped_gemm rounded to bf16 (N = 2 I, B = [G][2I][K], rows [0, I) of
 * each expert gate, rows [I, 2I) up):
 *   h[m, j] = bf16(silu(GU[m, j]) * GU[m, I + j]),  j < I,
 * and h is quantized in 1x128 groups: hs = max|h| / 448 per group, codes
 * E4M3(h / hs).  The codes and scales equal those of fp8_grouped_gemm (bf16
 * out) followed by fp8_silu_mul_quant(mx = 0); the bf16 gate/up output and h
 * are never written to memory.
 *
 * a .. sb_stride_k : as fp8_grouped_gemm with N = 2 I.
 * hq : [total_rows][ld_hq] h codes.   hs(m, j/128) = hs[m * hs_stride_row +
 *      (j / 128) * hs_stride_group] (pass 1 and total_rows for the M-major
 *      layout the down GEMM reads).
 * Requirements: as fp8_grouped_gemm; I % 128 == 0; ld_hq >= I, ld_hq % 8 ==
 * 0, hq 8-byte aligned; hs 4-byte aligned.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_grouped_gemm_swiglu_quant(int64_t total_rows, int64_t I, int64_t K, int32_t G, const int32_t* offsets,
                                           const int32_t* a_rows, int64_t a_count, const uint8_t* a, int64_t lda,
                                           const float* sa, int64_t sa_stride_m, int64_t sa_stride_k,
                                           const uint8_t* b, int64_t ldb, int64_t b_stride_g, const float* sb,
                                           int64_t sb_stride_g, int64_t sb_stride_n, int64_t sb_stride_k, uint8_t* hq,
                                           int64_t ld_hq, float* hs, int64_t hs_stride_row, int64_t hs_stride_group,
                                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * mxfp8_grouped_gemm_swiglu_quant -- the MXFP8 counterpart: the grouped
 * mxfp8_gemm gate/up product (G >= 1, N = 2 I, B = [G][2I][K] with rows
 * [0, I) gate and [I, 2I) up, UE8M0 scales per row and 32-wide K block)
 * rounded to bf16, h = bf16(silu(gate) * up), and h quantized in 1x32
 * blocks with UE8M0 scales.  Codes and scales equal those of mxfp8_gemm (bf16
 * out) followed by fp8_silu_mul_quant(mx = 1).
 *
 * a .. sb_stride_g : as mxfp8_gemm with G >= 1 and N = 2 I.
 * hq : [total_rows][ld_hq] h codes.   hs(m, j/32) = hs[m * hs_stride_row +
 *      (j / 32) * hs_stride_group] (UE8M0 bytes).
 * Requirements: as mxfp8_gemm; I % 128 == 0; ld_hq >= I, ld_hq % 8 == 0,
 * hq 8-byte aligned.
 * ------------------------------------------------------------------------ */
fp8bs_status mxfp8_grouped_gemm_swiglu_quant(int64_t total_rows, int64_t I, int64_t K, int32_t G,
                                             const int32_t* offsets, const int32_t* a_rows, int64_t a_count,
                                             const uint8_t* a, int64_t lda, const uint8_t* sa, int64_t lds_a,
                                             const uint8_t* b, int64_t ldb, int64_t b_stride_g, const uint8_t* sb,
                                             int64_t lds_b, int64_t sb_stride_g, uint8_t* hq, int64_t ld_hq,
                                             uint8_t* hs, int64_t hs_stride_row, int64_t hs_stride_group,
                                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_silu_mul_quant -- the step between the MoE gate/up and down GEMMs:
 * h = bf16(silu(g) * u) with silu(g) = g / (1 + exp(-g)), then
 * quantization of h, 1x128 with FP32 scales (mx == 0) or 1x32 with UE8M0
 * scales (mx == 1, see mxfp8_quant).
 * The pages do not describe this step.  It is the plainest reading of the
 * expert MLP of the Qwen3-30B-A3B MoE layer that "Low Precision RL" runs in
 * block-wise FP8 and MXFP8 (table "Choose a precision"): the gate/up GEMM's
 * output, rounded to bf16, feeds SiLU*mul, and h is the activation operand of
 * the down GEMM, so it is quantized with the activation grouping of the
 * recipe (1x128, section "2. Unified block-wise FP8 (DeepSeek-style)"; 1x32,
 * section "3. Unified MXFP8 (Blackwell)").
 *
 * gate_up : bf16 [rows][ld_in]; columns [0, I) hold the gate projection and
 *           columns [I, 2I) the up projection.
 * q       : [rows][ld_q] codes of h.   s : float* (mx == 0) or uint8_t* (mx == 1),
 *           scale of (row r, group g) at s[r * s_stride_row + g * s_stride_group].
 * h_out   : nullable bf16 [rows][ld_h]; receives h itself.
 * Requirements: I % 128 == 0 (I % 32 == 0 when mx == 1); ld_in >= 2 I,
 * ld_in % 8 == 0, gate_up 16-byte aligned; ld_q >= I, ld_q % 8 == 0;
 * ld_h >= I if h_out.
 * h is bit-exact against g / (1 + exp(-g)) * u evaluated in fp64 and
 * rounded once to bf16, for every finite bf16 g and u: an fp32 evaluation
 * (hardware exp2 and reciprocal, within 3.72 fp32 ulps of the exact value)
 * rounds it wherever it lies farther than 5 fp32 ulps from a bf16 rounding
 * midpoint, and an fp64 evaluation decides the rest (about 2^-12 of the
 * values at GEMM-output magnitudes, and every g below -44).
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_silu_mul_quant(const uint16_t* gate_up, int64_t rows, int64_t I, int64_t ld_in, int mx,
                                uint8_t* q, int64_t ld_q, void* s, int64_t s_stride_row, int64_t s_stride_group,
                                uint16_t* h_out, int64_t ld_h, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_moe_combine -- the step after the MoE down GEMM: each token's output is
 * the routing-weighted sum of its k experts' outputs,
 *
 *   out[t][n] = sum_{j=0}^{k-1} weights[t*k + j] * y[token_rows[t*k + j]][n]
 *
 * (the MoE layer of Qwen3-30B-A3B that "Low Precision RL" runs in block-wise
 * FP8, section "2. Unified block-wise FP8 (DeepSeek-style)").  The sum is an
 * fp32 FMA chain in slot order j = 0, 1, ..., k-1 starting from 0
 * (deterministic), then rounded to nearest even for bf16 output.
 *
 * y          : bf16 [rows][ld_y], the grouped down-projection output in
 *              expert-sorted order (fp8_grouped_gemm's c).
 * token_rows : device int32 [T][k]: the row of y that holds token t's j-th
 *              assignment.  Entries outside [0, rows) are clamped into it
 *              (never read outside y; the result is then meaningless).
 * weights    : device fp32 [T][k] routing weights.
 * out        : [T][ld_out], bf16 or fp32 per `out_type`.
 * Requirements: rows, H, T >= 0, k >= 1; rows >= 1 if T > 0; H % 8 == 0;
 * ld_y >= H, ld_y % 8 == 0, y 16-byte aligned; ld_out >= H, ld_out % 8 == 0,
 * out 16-byte aligned; token_rows and weights 4-byte aligned.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_moe_combine(const uint16_t* y, int64_t rows, int64_t H, int64_t ld_y,
                             const int32_t* token_rows, const float* weights, int64_t T, int32_t k,
                             void* out, int64_t ld_out, fp8bs_out out_type, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_quant_pow2 / fp8_blockscaled_gemm_pow2 -- the block-wise recipe with
 * power-of-two scales: the form TransformerEngine uses when it runs the
 * 1x128 / 128x128 recipe on Blackwell through MXFP8 ("Low Precision RL",
 * section "2. Unified block-wise FP8 (DeepSeek-style)", on
 * NVTE_FP8_BLOCK_SCALING_FP32_SCALES).  Each group's scale is 2^e with e the
 * smallest integer such that max|x| <= 448 * 2^e, clamped to [-127, 127]
 * (-127 for an all-zero group), stored as the UE8M0 byte e + 127; the codes
 * are E4M3(x * 2^-e) (exact scaling, one rounding).  The GEMM applies the
 * scales inside the scaled matrix instruction (exact), so it needs no
 * per-slice FP32 promotion.
 *
 * fp8_quant_pow2:
 *   block_rows : 1 (1x128 groups along each row) or 128 (128x128 blocks).
 *   x : bf16 [rows][ld_x];  q : [rows][ld_q];
 *   s : uint8, byte of (row group i, column group g = col / 128) at
 *       s[i * ld_s + g], i = row / block_rows.
 *   Requirements: cols % 8 == 0; ld_x % 8 == 0, x 16-byte aligned;
 *   ld_q >= cols, ld_q % 8 == 0, q 8-byte aligned; ld_s >= ceil(cols / 128).
 *   For the GEMM, choose ld_s % 4 == 0 and ld_s >= 4 * ceil(cols / 512).
 *
 * fp8_blockscaled_gemm_pow2:  C = A B^T,
 *   C[m, n] = sum_kb 2^(sa(m, kb) - 127) * 2^(sb(n/128, kb) - 127) * sum_{k in kb} dec(a[m,k]) dec(b[n,k])
 *   a : [M][lda] codes (1x128 groups), sa(m, kb) = sa[m * lds_a + kb];
 *   b : [N][ldb] codes (128x128 blocks), sb(n / 128, kb) = sb[(n / 128) * lds_b + kb];
 *   c : [M][ldc] bf16 or fp32.
 *   Requirements: as fp8_blockscaled_gemm for a, b, c; lds_a and lds_b
 *   multiples of 4 and >= 4 * ceil(K / 512) (each slice's byte is read with
 *   the 4-byte word of its group of four slices); sa, sb 4-byte aligned.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_quant_pow2(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t block_rows,
                            uint8_t* q, int64_t ld_q, uint8_t* s, int64_t ld_s, hipStream_t stream);
fp8bs_status fp8_blockscaled_gemm_pow2(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                       const uint8_t* sa, int64_t lds_a, const uint8_t* b, int64_t ldb,
                                       const uint8_t* sb, int64_t lds_b, void* c, int64_t ldc, fp8bs_out out,
                                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_quant_linear_pow2 -- both operands of a linear layer with power-of-two
 * block scales in one launch: X [rows][cols] in 1x128 groups and W
 * [w_rows][cols] in 128x128 blocks, each scale the UE8M0 byte of
 * fp8_quant_pow2 (same section of the same page).  The results are identical
 * to fp8_quant_pow2(x, ..., block_rows 1, qx, ld_qx, sx, ld_sx) followed by
 * fp8_quant_pow2(w, ..., block_rows 128, qw, ld_qw, sw, ld_sw); one grid
 * carries both, as fp8_quant_linear does for FP32 scales.
 * Either operand may be empty (rows == 0 or w_rows == 0; its pointers are
 * then not read).  Requirements: as the two calls; the buffers of the two
 * operands must not overlap.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_quant_linear_pow2(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qx,
                                   int64_t ld_qx, uint8_t* sx, int64_t ld_sx, const uint16_t* w, int64_t w_rows,
                                   int64_t ld_w, uint8_t* qw, int64_t ld_qw, uint8_t* sw, int64_t ld_sw,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * mxfp8_quant -- MXFP8 quantization: 32 consecutive values along a row share
 * one UE8M0 scale ("Low Precision RL", section "3. Unified MXFP8
 * (Blackwell)").  The block exponent is the smallest integer e with
 * max|x| <= 448 * 2^e, clamped to [-127, 127] (-127 for an all-zero block);
 * the scale byte is e + 127 and the codes are E4M3(x * 2^-e) (exact scaling,
 * one rounding).  An all-zero block has all codes 0x00.
 *
 * x : bf16 [rows][ld_x]; q : [rows][ld_q]; s : uint8 scale of (row r, block
 *     g = col / 32) at s[r * s_stride_row + g * s_stride_group].
 * Requirements: cols % 32 == 0; ld_x % 8 == 0 and x 16-byte aligned;
 * ld_q >= cols, ld_q % 8 == 0.
 * ------------------------------------------------------------------------ */
fp8bs_status mxfp8_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                         uint8_t* q, int64_t ld_q, uint8_t* s, int64_t s_stride_row, int64_t s_stride_group,
                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * mxfp8_quant_t -- MXFP8 quantization along the other axis: 32 consecutive
 * values of a COLUMN share one UE8M0 scale (same exponent rule and encoding
 * as mxfp8_quant), written transposed.  It equals mxfp8_quant applied to the
 * transpose of x.  1x32 blocks are not transpose-invariant, so the MXFP8
 * backward GEMMs ("Low Precision RL", section "3. Unified MXFP8
 * (Blackwell)": the recipe runs the weight-gradient and data-gradient GEMMs
 * in MXFP8) need their operands re-quantized along the contraction axis:
 *   dgrad dX = dY W : B operand = W quantized along its rows (output features);
 *   wgrad dW = dY^T X : both operands quantized along tokens.
 *
 * x  : bf16 [rows][ld_x].   qt : [cols][ld_qt] codes, the row axis contiguous.
 * s  : uint8, scale of (column c, block g = row / 32) at
 *      s[c * s_stride_row + g * s_stride_group] (s_stride_row = lds,
 *      s_stride_group = 1 gives mxfp8_gemm's [cols][lds] layout).
 * Requirements: rows % 32 == 0, rows <= 65535 * 128; cols % 8 == 0;
 * ld_x % 8 == 0, x 16-byte aligned; ld_qt >= rows, ld_qt % 16 == 0,
 * qt 16-byte aligned.
 * ------------------------------------------------------------------------ */
fp8bs_status mxfp8_quant_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t* qt, int64_t ld_qt, uint8_t* s, int64_t s_stride_row,
                           int64_t s_stride_group, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8_quant_dual_axis -- both quantizations a tensor needs when one GEMM
 * contracts over its columns and another over its rows, from one read of
 * it.  The output gradient dY of a block-wise FP8 linear layer is the case:
 * the data-gradient GEMM dX = dY W takes dY in per-token 1x128 groups
 * ("Unified FP8: Beyond Mixed Precision...", section "FP8 Quantization",
 * per-token gradients), the weight-gradient GEMM dW = dY^T X in 128x1
 * groups along tokens; with mx == 1 the MXFP8 recipe's 1x32 blocks and
 * their re-quantization along the other axis ("Low Precision RL", section
 * "3. Unified MXFP8 (Blackwell)").  The results are identical to
 *   mx == 0: fp8_quant_rowblock(x, ..., FP8BS_AXIS_ROW, q, ld_q, s, ...)
 *            and fp8_quant_rowblock(x, ..., FP8BS_AXIS_COL, qt, ld_qt, st, ...);
 *   mx == 1: mxfp8_quant(x, ..., q, ld_q, s, ...)
 *            and mxfp8_quant_t(x, ..., qt, ld_qt, st, ...);
 * the bf16 tensor is read once (2 bytes per element instead of 4).
 *
 * x  : bf16 [rows][ld_x].
 * q  : [rows][ld_q] codes of the row groups; scale of (row r, group g =
 *      col / 128, or col / 32 with mx) at s[r * s_stride_row + g * s_stride_group].
 * qt : [cols][ld_qt] codes of the column groups, the row axis contiguous;
 *      scale of (column c, group g = row / 128, or row / 32 with mx) at
 *      st[c * st_stride_row + g * st_stride_group].
 * s, st : fp32 scales (mx == 0) or UE8M0 bytes (mx == 1).
 * Requirements: rows % 16 == 0 and cols % 8 == 0 (mx: rows % 32 == 0 and
 * cols % 32 == 0); ceil(cols / 128) <= 65535; x 16-byte aligned with
 * ld_x % 8 == 0, ld_x >= cols; q and qt 8-byte aligned with ld_q % 8 == 0,
 * ld_q >= cols, ld_qt % 8 == 0, ld_qt >= rows; fp32 scales 4-byte aligned.
 * The output buffers must not overlap one another.
 * ------------------------------------------------------------------------ */
fp8bs_status fp8_quant_dual_axis(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t mx,
                                 uint8_t* q, int64_t ld_q, void* s, int64_t s_stride_row, int64_t s_stride_group,
                                 uint8_t* qt, int64_t ld_qt, void* st, int64_t st_stride_row,
                                 int64_t st_stride_group, hipStream_t stream);

/* ------------------------------------------------------------------------
 * mxfp8_gemm -- C = A B^T on MXFP8 operands (dense when G == 0, grouped over
 * experts when G >= 1), exact power-of-two block scaling inside gfx950's
 * scaled FP8 matrix instructions, FP32 accumulation.
 *
 *   C[m, n] = sum_k 2^(sa(m, k/32) - 127) dec(a[m, k]) * 2^(sb(n, k/32) - 127) dec(b[n, k])
 *
 * a   : [rows][lda] codes (or a_count rows gathered through a_rows, as in
 *       fp8_grouped_gemm);  sa : uint8 [.][lds_a], row m's scales at sa + m * lds_a.
 * b   : [G or 1][N][ldb] codes, expert stride b_stride_g;
 * sb  : uint8, expert g row n's scales at sb + g * sb_stride_g + n * lds_b.
 * offsets : device int32 [G + 1] (ignored when G == 0), as in fp8_grouped_gemm.
 * Requirements: K % 128 == 0; N % 128 == 0; lda, ldb % 16 == 0; lds_a >= K/32,
 * lds_b >= K/32, lds_a % 4 == 0, lds_b % 4 == 0, sa and sb 4-byte aligned.
 * ------------------------------------------------------------------------ */
fp8bs_status mxfp8_gemm(int64_t rows, int64_t N, int64_t K, int32_t G,
                        const int32_t* offsets, const int32_t* a_rows, int64_t a_count,
                        const uint8_t* a, int64_t lda, const uint8_t* sa, int64_t lds_a,
                        const uint8_t* b, int64_t ldb, int64_t b_stride_g,
                        const uint8_t* sb, int64_t lds_b, int64_t sb_stride_g,
                        void* c, int64_t ldc, fp8bs_out out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * fp8bs_e4m3_encode -- encode n fp32 values with the same device routine the
 * quantizers use (round to nearest even, saturating to +-448).  For checking
 * the device codec against a table; not on the layer's hot path.
 * in : device float [n]; out : device uint8 [n].
 * ------------------------------------------------------------------------ */
fp8bs_status fp8bs_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* fp8bs_status_string(fp8bs_status s);
/* Thread-local detail message of the last failing call on this thread ("" if none). */
const char* fp8bs_last_error_detail(void);

#ifdef __cplusplus
}
#endif
#endif /* FP8BS_H */
