// C ABI of libfp8bs: argument validation, device check and dispatch to the
// kernel launchers.  Declarations and the contract of every entry point are
// in include/fp8bs.h.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fp8bs.h"
#include "internal.h"

using namespace fp8bs;

// Scratch of fp8_blockscaled_gemm_splitk_noalloc: the fp32 partials of the
// K ranges, in one file-scope array per device (each GPU holds its copy for
// the life of the process).  Nothing in it needs to start at zero (every
// partial the sum reads is written first by the same call); calls that
// overlap in time on one GPU share it and race.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

thread_local char g_detail[512];

fp8bs_status fail(fp8bs_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return s;
}

fp8bs_status ok() {
    g_detail[0] = '\0';
    return FP8BS_OK;
}

// Per-device result of the gfx950 check: 0 unknown, 1 yes, 2 no.
std::atomic<int> g_dev_ok[64];

fp8bs_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(FP8BS_ERR_DEVICE, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(FP8BS_ERR_DEVICE, "device index %d out of range", dev);
    int st = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(FP8BS_ERR_DEVICE, "hipGetDeviceProperties failed");
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_ok[dev].store(st, std::memory_order_relaxed);
    }
    if (st != 1) return fail(FP8BS_ERR_DEVICE, "current device %d is not gfx950", dev);
    return FP8BS_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

fp8bs_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FP8BS_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

constexpr int64_t kMaxRuns = (int64_t)1 << 30;   // row-group kernels index runs with int32

// Host code never uses the array's name (`scratch`, above) as an address:
// the first call on a device looks up that device's copy with
// hipGetSymbolAddress and keeps it here.
std::atomic<float*> g_scratch[64];

fp8bs_status scratch_ptr(float** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(FP8BS_ERR_DEVICE, "hipGetDevice failed");
    if (dev < 0 || dev >= 64) return fail(FP8BS_ERR_DEVICE, "device index %d out of range", dev);
    float* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* q = nullptr;
        const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess || q == nullptr)
            return fail(FP8BS_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                        hipGetErrorString(e));
        p = static_cast<float*>(q);
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return FP8BS_OK;
}

}  // namespace

extern "C" {

const char* fp8bs_status_string(fp8bs_status s) {
    switch (s) {
        case FP8BS_OK: return "FP8BS_OK";
        case FP8BS_ERR_NULL: return "FP8BS_ERR_NULL";
        case FP8BS_ERR_SHAPE: return "FP8BS_ERR_SHAPE";
        case FP8BS_ERR_STRIDE: return "FP8BS_ERR_STRIDE";
        case FP8BS_ERR_ALIGN: return "FP8BS_ERR_ALIGN";
        case FP8BS_ERR_UNSUPPORTED: return "FP8BS_ERR_UNSUPPORTED";
        case FP8BS_ERR_DEVICE: return "FP8BS_ERR_DEVICE";
    }
    return "FP8BS_UNKNOWN_STATUS";
}

const char* fp8bs_last_error_detail(void) { return g_detail; }

fp8bs_status fp8_quant_rowblock(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, fp8bs_axis axis,
                                uint8_t* q, int64_t ld_q, float* s, int64_t s_stride_row, int64_t s_stride_group,
                                hipStream_t stream) {
    if (axis != FP8BS_AXIS_ROW && axis != FP8BS_AXIS_COL) return fail(FP8BS_ERR_UNSUPPORTED, "axis %d", (int)axis);
    if (rows < 0 || cols < 0) return fail(FP8BS_ERR_SHAPE, "rows=%lld cols=%lld", (long long)rows, (long long)cols);
    if (cols % 8) return fail(FP8BS_ERR_SHAPE, "cols %% 8 != 0 (cols=%lld)", (long long)cols);
    if (axis == FP8BS_AXIS_COL && rows % 16) return fail(FP8BS_ERR_SHAPE, "AXIS_COL needs rows %% 16 == 0");
    if (rows * ((cols + 127) / 128) > kMaxRuns || rows > INT32_MAX / 2 || cols > INT32_MAX / 2)
        return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (rows == 0 || cols == 0) return ok();
    if (!x || !q || !s) return fail(FP8BS_ERR_NULL, "x, q and s are required");
    if (ld_x < cols) return fail(FP8BS_ERR_STRIDE, "ld_x < cols");
    if (ld_x % 8 || !aligned(x, 16)) return fail(FP8BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    if (axis == FP8BS_AXIS_ROW) {
        if (ld_q < cols) return fail(FP8BS_ERR_STRIDE, "ld_q < cols");
        if (ld_q % 8 || !aligned(q, 8)) return fail(FP8BS_ERR_ALIGN, "q must be 8-byte aligned with ld_q %% 8 == 0");
    } else {
        if (ld_q < rows) return fail(FP8BS_ERR_STRIDE, "ld_q < rows (transposed output)");
        if (ld_q % 16 || !aligned(q, 16)) return fail(FP8BS_ERR_ALIGN, "q must be 16-byte aligned with ld_q %% 16 == 0");
    }
    if (!aligned(s, 4)) return fail(FP8BS_ERR_ALIGN, "s must be 4-byte aligned");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    if (axis == FP8BS_AXIS_ROW)
        return launched(launch_quant_1x128(x, rows, cols, ld_x, q, ld_q, s, s_stride_row, s_stride_group, stream),
                        "fp8_quant_rowblock");
    return launched(launch_quant_128x1_t(x, rows, cols, ld_x, q, ld_q, s, s_stride_row, s_stride_group, stream),
                    "fp8_quant_rowblock");
}

// The checks both operand-pair entry points make: each operand as its own
// quantizer call would check it (an empty operand's pointers are not read).
// pow2: UE8M0 scale bytes with row strides ld_sx / ld_sw; otherwise fp32
// scales, 4-byte aligned.
static fp8bs_status linear_pair_args(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const uint8_t* qx,
                                     int64_t ld_qx, const void* sx, int64_t ld_sx, const uint16_t* w, int64_t w_rows,
                                     int64_t ld_w, const uint8_t* qw, int64_t ld_qw, const void* sw, int64_t ld_sw,
                                     bool pow2) {
    if (rows < 0 || cols < 0 || w_rows < 0)
        return fail(FP8BS_ERR_SHAPE, "rows=%lld cols=%lld w_rows=%lld", (long long)rows, (long long)cols,
                    (long long)w_rows);
    if (cols % 8) return fail(FP8BS_ERR_SHAPE, "cols %% 8 != 0 (cols=%lld)", (long long)cols);
    if (rows * ((cols + 127) / 128) > kMaxRuns || rows > INT32_MAX / 2 || cols > INT32_MAX / 2 ||
        w_rows > INT32_MAX / 2 || (w_rows + 127) / 128 > 65535 || ((w_rows + 127) / 128) * ((cols + 127) / 128) > kMaxRuns)
        return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (cols == 0 || (rows == 0 && w_rows == 0)) return ok();
    const int64_t groups = (cols + 127) / 128;
    if (rows > 0) {
        if (!x || !qx || !sx) return fail(FP8BS_ERR_NULL, "x, qx and sx are required");
        if (ld_x < cols || ld_qx < cols) return fail(FP8BS_ERR_STRIDE, "ld_x and ld_qx must be >= cols");
        if (pow2 && ld_sx < groups) return fail(FP8BS_ERR_STRIDE, "ld_sx must be >= ceil(cols / 128)");
        if (ld_x % 8 || !aligned(x, 16)) return fail(FP8BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
        if (ld_qx % 8 || !aligned(qx, 8)) return fail(FP8BS_ERR_ALIGN, "qx must be 8-byte aligned with ld_qx %% 8 == 0");
        if (!pow2 && !aligned(sx, 4)) return fail(FP8BS_ERR_ALIGN, "sx must be 4-byte aligned");
    }
    if (w_rows > 0) {
        if (!w || !qw || !sw) return fail(FP8BS_ERR_NULL, "w, qw and sw are required");
        if (ld_w < cols || ld_qw < cols) return fail(FP8BS_ERR_STRIDE, "ld_w and ld_qw must be >= cols");
        if (pow2 && ld_sw < groups) return fail(FP8BS_ERR_STRIDE, "ld_sw must be >= ceil(cols / 128)");
        if (pow2 && ld_sw > INT32_MAX / 2) return fail(FP8BS_ERR_SHAPE, "ld_sw too large");
        if (ld_w % 8 || !aligned(w, 16)) return fail(FP8BS_ERR_ALIGN, "w must be 16-byte aligned with ld_w %% 8 == 0");
        if (ld_qw % 8 || !aligned(qw, 8)) return fail(FP8BS_ERR_ALIGN, "qw must be 8-byte aligned with ld_qw %% 8 == 0");
        if (!pow2 && !aligned(sw, 4)) return fail(FP8BS_ERR_ALIGN, "sw must be 4-byte aligned");
    }
    return check_device();
}

fp8bs_status fp8_quant_linear(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qx, int64_t ld_qx,
                              float* sx, int64_t sx_stride_row, int64_t sx_stride_group, const uint16_t* w,
                              int64_t w_rows, int64_t ld_w, uint8_t* qw, int64_t ld_qw, float* sw,
                              hipStream_t stream) {
    fp8bs_status v = linear_pair_args(x, rows, cols, ld_x, qx, ld_qx, sx, 0, w, w_rows, ld_w, qw, ld_qw, sw, 0, false);
    if (v != FP8BS_OK || cols == 0 || (rows == 0 && w_rows == 0)) return v;
    return launched(launch_quant_linear(x, rows, cols, ld_x, qx, ld_qx, sx, sx_stride_row, sx_stride_group, w, w_rows,
                                        ld_w, qw, ld_qw, sw, stream),
                    "fp8_quant_linear");
}

fp8bs_status fp8_quant_linear_pow2(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qx,
                                   int64_t ld_qx, uint8_t* sx, int64_t ld_sx, const uint16_t* w, int64_t w_rows,
                                   int64_t ld_w, uint8_t* qw, int64_t ld_qw, uint8_t* sw, int64_t ld_sw,
                                   hipStream_t stream) {
    fp8bs_status v = linear_pair_args(x, rows, cols, ld_x, qx, ld_qx, sx, ld_sx, w, w_rows, ld_w, qw, ld_qw, sw, ld_sw,
                                      true);
    if (v != FP8BS_OK || cols == 0 || (rows == 0 && w_rows == 0)) return v;
    return launched(launch_quant_linear_pow2(x, rows, cols, ld_x, qx, ld_qx, sx, ld_sx, w, w_rows, ld_w, qw, ld_qw, sw,
                                             ld_sw, stream),
                    "fp8_quant_linear_pow2");
}

fp8bs_status fp8_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                               float* s, hipStream_t stream) {
    if (rows < 0 || cols < 0) return fail(FP8BS_ERR_SHAPE, "rows=%lld cols=%lld", (long long)rows, (long long)cols);
    if (cols % 8) return fail(FP8BS_ERR_SHAPE, "cols %% 8 != 0 (cols=%lld)", (long long)cols);
    if (rows > INT32_MAX / 2 || cols > INT32_MAX / 2) return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (rows == 0) return ok();
    if (!x || !q || !s) return fail(FP8BS_ERR_NULL, "x, q and s are required");
    if (ld_x < cols || ld_q < cols) return fail(FP8BS_ERR_STRIDE, "ld_x and ld_q must be >= cols");
    if (ld_x % 8 || !aligned(x, 16)) return fail(FP8BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    if (ld_q % 8 || !aligned(q, 8)) return fail(FP8BS_ERR_ALIGN, "q must be 8-byte aligned with ld_q %% 8 == 0");
    if (!aligned(s, 4)) return fail(FP8BS_ERR_ALIGN, "s must be 4-byte aligned");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_quant_rowwise(x, rows, cols, ld_x, q, ld_q, s, stream), "fp8_quant_rowwise");
}

fp8bs_status fp8_quant_tensorwise(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                                  int64_t ld_q, float* s, hipStream_t stream) {
    if (rows < 0 || cols < 0) return fail(FP8BS_ERR_SHAPE, "rows=%lld cols=%lld", (long long)rows, (long long)cols);
    if (cols % 8) return fail(FP8BS_ERR_SHAPE, "cols %% 8 != 0 (cols=%lld)", (long long)cols);
    if (rows > INT32_MAX / 2 || cols > INT32_MAX / 2) return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (!s) return fail(FP8BS_ERR_NULL, "s is required");
    if (!aligned(s, 4)) return fail(FP8BS_ERR_ALIGN, "s must be 4-byte aligned");
    if (rows > 0 && cols > 0) {
        if (!x || !q) return fail(FP8BS_ERR_NULL, "x and q are required");
        if (ld_x < cols || ld_q < cols) return fail(FP8BS_ERR_STRIDE, "ld_x and ld_q must be >= cols");
        if (ld_x % 8 || !aligned(x, 16)) return fail(FP8BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
        if (ld_q % 8 || !aligned(q, 8)) return fail(FP8BS_ERR_ALIGN, "q must be 8-byte aligned with ld_q %% 8 == 0");
    }
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_quant_tensorwise(x, rows, cols, ld_x, q, ld_q, s, stream), "fp8_quant_tensorwise");
}

fp8bs_status fp8_quant_block2d(const uint16_t* w, int64_t batch, int64_t rows, int64_t cols, int64_t ld_w,
                               uint8_t* q, int64_t ld_q, uint8_t* q_t, int64_t ld_qt, float* s, hipStream_t stream) {
    if (batch < 1 || rows < 0 || cols < 0) return fail(FP8BS_ERR_SHAPE, "batch=%lld rows=%lld cols=%lld",
                                                      (long long)batch, (long long)rows, (long long)cols);
    if (cols % 8) return fail(FP8BS_ERR_SHAPE, "cols %% 8 != 0");
    if (q_t && rows % 16) return fail(FP8BS_ERR_SHAPE, "a transposed copy needs rows %% 16 == 0");
    if (rows > INT32_MAX / 2 || cols > INT32_MAX / 2 || batch > 65535 || (rows + 127) / 128 > 65535)
        return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (rows == 0 || cols == 0) return ok();
    if (!w || !s || (!q && !q_t)) return fail(FP8BS_ERR_NULL, "w, s and at least one of q and q_t are required");
    if (ld_w < cols || (q && ld_q < cols)) return fail(FP8BS_ERR_STRIDE, "ld_w and ld_q must be >= cols");
    if (q_t && ld_qt < rows) return fail(FP8BS_ERR_STRIDE, "ld_qt < rows");
    if (ld_w % 8 || !aligned(w, 16)) return fail(FP8BS_ERR_ALIGN, "w must be 16-byte aligned with ld_w %% 8 == 0");
    if (q && (ld_q % 8 || !aligned(q, 8))) return fail(FP8BS_ERR_ALIGN, "q must be 8-byte aligned with ld_q %% 8 == 0");
    if (q_t && (ld_qt % 16 || !aligned(q_t, 16))) return fail(FP8BS_ERR_ALIGN, "q_t must be 16-byte aligned with ld_qt %% 16 == 0");
    if (!aligned(s, 4)) return fail(FP8BS_ERR_ALIGN, "s must be 4-byte aligned");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_quant_128x128(w, batch, rows, cols, ld_w, q, ld_q, q_t, ld_qt, s, stream),
                    "fp8_quant_block2d");
}

fp8bs_status fp8_transpose_codes(const uint8_t* q, int64_t batch, int64_t rows, int64_t cols, int64_t ld_q,
                                 uint8_t* q_t, int64_t ld_qt, hipStream_t stream) {
    if (batch < 1 || rows < 0 || cols < 0) return fail(FP8BS_ERR_SHAPE, "batch=%lld rows=%lld cols=%lld",
                                                      (long long)batch, (long long)rows, (long long)cols);
    if (rows % 16 || cols % 16) return fail(FP8BS_ERR_SHAPE, "rows %% 16 and cols %% 16 must be 0");
    if (rows > INT32_MAX / 2 || cols > INT32_MAX / 2 || batch > 65535 || (rows + 127) / 128 > 65535)
        return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (rows == 0 || cols == 0) return ok();
    if (!q || !q_t) return fail(FP8BS_ERR_NULL, "q and q_t are required");
    if (ld_q < cols || ld_qt < rows) return fail(FP8BS_ERR_STRIDE, "ld_q >= cols and ld_qt >= rows required");
    if (ld_q % 16 || !aligned(q, 16)) return fail(FP8BS_ERR_ALIGN, "q must be 16-byte aligned with ld_q %% 16 == 0");
    if (ld_qt % 16 || !aligned(q_t, 16))
        return fail(FP8BS_ERR_ALIGN, "q_t must be 16-byte aligned with ld_qt %% 16 == 0");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_transpose_codes(q, batch, rows, cols, ld_q, q_t, ld_qt, stream), "fp8_transpose_codes");
}

// The kernels address a scale array with 32-bit byte offsets within one
// group: the largest offset (rows - 1) * s_row + (slices - 1) * s_slice, in
// elements of `bytes`, must stay below 4 GiB, and strides must not be negative.
static fp8bs_status check_scale_extent(const char* name, int64_t rows, int64_t s_row, int64_t slices,
                                       int64_t s_slice, int bytes) {
    if (s_row < 0 || s_slice < 0) return fail(FP8BS_ERR_STRIDE, "%s: negative scale stride", name);
    const double hi = ((double)(rows - 1) * (double)s_row + (double)(slices - 1) * (double)s_slice) * bytes;
    if (hi >= 4294967296.0) return fail(FP8BS_ERR_SHAPE, "%s: scale array extent exceeds 4 GiB", name);
    return FP8BS_OK;
}

static fp8bs_status check_gemm_common(int64_t M, int64_t N, int64_t K, const void* a, int64_t lda, const void* b,
                                      int64_t ldb, const void* c, int64_t ldc, int out, int kmul) {
    if (M < 0 || N < 0 || K < 0) return fail(FP8BS_ERR_SHAPE, "negative size");
    if (K % kmul) return fail(FP8BS_ERR_SHAPE, "K %% %d != 0 (K=%lld)", kmul, (long long)K);
    if (N % 128) return fail(FP8BS_ERR_SHAPE, "N %% 128 != 0 (N=%lld)", (long long)N);
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return fail(FP8BS_ERR_SHAPE, "size too large");
    if (out != FP8BS_OUT_BF16 && out != FP8BS_OUT_FP32) return fail(FP8BS_ERR_UNSUPPORTED, "out %d", out);
    if (M == 0 || N == 0) return FP8BS_OK;
    if (K == 0) return fail(FP8BS_ERR_SHAPE, "K == 0");
    if (!a || !b || !c) return fail(FP8BS_ERR_NULL, "a, b and c are required");
    if (lda < K || ldb < K || ldc < N) return fail(FP8BS_ERR_STRIDE, "lda, ldb must be >= K and ldc >= N");
    if (lda % 16 || ldb % 16 || !aligned(a, 16) || !aligned(b, 16))
        return fail(FP8BS_ERR_ALIGN, "a, b must be 16-byte aligned with lda, ldb %% 16 == 0");
    if (ldc % 8 || !aligned(c, 16)) return fail(FP8BS_ERR_ALIGN, "c must be 16-byte aligned with ldc %% 8 == 0");
    return FP8BS_OK;
}

}  // extern "C"

// Validation shared by fp8_blockscaled_gemm and its K-split form; fills g
// (g.M = g.N = 0 when there is nothing to compute).
static fp8bs_status blockscaled_args(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                                     int64_t sa_stride_m, int64_t sa_stride_k, const uint8_t* b, int64_t ldb,
                                     const float* sb, int64_t sb_stride_n, int64_t sb_stride_k, fp8bs_bscale bscale,
                                     void* c, int64_t ldc, fp8bs_out out, GemmArgs* g) {
    if (bscale != FP8BS_BSCALE_BLOCK128 && bscale != FP8BS_BSCALE_ROW128)
        return fail(FP8BS_ERR_UNSUPPORTED, "bscale %d", (int)bscale);
    fp8bs_status v = check_gemm_common(M, N, K, a, lda, b, ldb, c, ldc, out, 128);
    if (v != FP8BS_OK) return v;
    if (M == 0 || N == 0) return ok();
    if (!sa || !sb) return fail(FP8BS_ERR_NULL, "sa and sb are required");
    if (!aligned(sa, 4) || !aligned(sb, 4)) return fail(FP8BS_ERR_ALIGN, "scales must be 4-byte aligned");
    if ((uint64_t)M * (uint64_t)lda >= (1ull << 32) || (uint64_t)N * (uint64_t)ldb >= (1ull << 32))
        return fail(FP8BS_ERR_SHAPE, "an operand exceeds 4 GiB");
    // tiles (at least 128 rows x 160 columns) are counted in int32 on the device
    if (((M + 127) / 128) * ((N + 159) / 160) >= (1ll << 31) - 8) return fail(FP8BS_ERR_SHAPE, "too many tiles");
    if ((v = check_scale_extent("sa", M, sa_stride_m, K / 128, sa_stride_k, 4)) != FP8BS_OK) return v;
    if ((v = check_scale_extent("sb", bscale == FP8BS_BSCALE_ROW128 ? N : N / 128, sb_stride_n, K / 128,
                                sb_stride_k, 4)) != FP8BS_OK)
        return v;
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    g->M = M; g->N = N; g->K = K; g->a = a; g->lda = lda; g->sa = sa; g->sa_sm = sa_stride_m; g->sa_sk = sa_stride_k;
    g->b = b; g->ldb = ldb; g->b_sg = 0; g->sb = sb; g->sb_sg = 0; g->sb_sn = sb_stride_n; g->sb_sk = sb_stride_k;
    g->bscale_row = bscale == FP8BS_BSCALE_ROW128; g->c = c; g->ldc = ldc; g->out_f32 = out == FP8BS_OUT_FP32;
    return FP8BS_OK;
}

extern "C" {

fp8bs_status fp8_blockscaled_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const float* sa,
                                  int64_t sa_stride_m, int64_t sa_stride_k, const uint8_t* b, int64_t ldb,
                                  const float* sb, int64_t sb_stride_n, int64_t sb_stride_k, fp8bs_bscale bscale,
                                  void* c, int64_t ldc, fp8bs_out out, hipStream_t stream) {
    GemmArgs g{};
    const fp8bs_status v = blockscaled_args(M, N, K, a, lda, sa, sa_stride_m, sa_stride_k, b, ldb, sb, sb_stride_n,
                                            sb_stride_k, bscale, c, ldc, out, &g);
    if (v != FP8BS_OK || g.M == 0) return v;
    return launched(launch_gemm_blockscaled(g, stream), "fp8_blockscaled_gemm");
}

fp8bs_status fp8_blockscaled_gemm_splitk(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                         const float* sa, int64_t sa_stride_m, int64_t sa_stride_k, const uint8_t* b,
                                         int64_t ldb, const float* sb, int64_t sb_stride_n, int64_t sb_stride_k,
                                         fp8bs_bscale bscale, void* c, int64_t ldc, fp8bs_out out, int32_t splits,
                                         float* ws, size_t ws_bytes, hipStream_t stream) {
    if (splits < 0) return fail(FP8BS_ERR_SHAPE, "splits %d < 0", (int)splits);
    GemmArgs g{};
    const fp8bs_status v = blockscaled_args(M, N, K, a, lda, sa, sa_stride_m, sa_stride_k, b, ldb, sb, sb_stride_n,
                                            sb_stride_k, bscale, c, ldc, out, &g);
    if (v != FP8BS_OK || g.M == 0) return v;
    if (splits > K / 128) return fail(FP8BS_ERR_SHAPE, "splits %d > K / 128 = %lld", (int)splits, (long long)(K / 128));
    if (splits == 0) splits = plan_gemm_splitk(M, N, K, out == FP8BS_OUT_FP32);
    if (splits > 1) {
        if (!ws) return fail(FP8BS_ERR_NULL, "ws is required when splits > 1");
        if (!aligned(ws, 16)) return fail(FP8BS_ERR_ALIGN, "ws must be 16-byte aligned");
        const uint64_t need = (uint64_t)splits * (uint64_t)M * (uint64_t)N * 4u;
        if ((uint64_t)ws_bytes < need)
            return fail(FP8BS_ERR_SHAPE, "workspace of %llu bytes, %llu needed for %d splits",
                        (unsigned long long)ws_bytes, (unsigned long long)need, (int)splits);
        if ((uint64_t)M * (uint64_t)N / 8 / 256 >= (1ull << 31)) return fail(FP8BS_ERR_SHAPE, "output too large");
    }
    return launched(launch_gemm_blockscaled_splitk(g, splits, ws, stream), "fp8_blockscaled_gemm_splitk");
}

fp8bs_status fp8_blockscaled_gemm_splitk_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                                 const float* sa, int64_t sa_stride_m, int64_t sa_stride_k,
                                                 const uint8_t* b, int64_t ldb, const float* sb, int64_t sb_stride_n,
                                                 int64_t sb_stride_k, fp8bs_bscale bscale, void* c, int64_t ldc,
                                                 fp8bs_out out, int32_t splits, hipStream_t stream) {
    if (splits < 0) return fail(FP8BS_ERR_SHAPE, "splits %d < 0", (int)splits);
    GemmArgs g{};
    const fp8bs_status v = blockscaled_args(M, N, K, a, lda, sa, sa_stride_m, sa_stride_k, b, ldb, sb, sb_stride_n,
                                            sb_stride_k, bscale, c, ldc, out, &g);
    if (v != FP8BS_OK || g.M == 0) return v;
    if (splits > K / 128) return fail(FP8BS_ERR_SHAPE, "splits %d > K / 128 = %lld", (int)splits, (long long)(K / 128));
    const uint64_t per_split = (uint64_t)M * (uint64_t)N * 4u;
    if (splits == 0) {
        // the planner's count, capped to what the scratch holds
        splits = plan_gemm_splitk(M, N, K, out == FP8BS_OUT_FP32);
        const uint64_t fit = kScratchBytes / per_split;
        if ((uint64_t)splits > fit) splits = fit >= 2 ? (int32_t)fit : 1;
    }
    float* ws = nullptr;
    if (splits > 1) {
        if ((uint64_t)splits * per_split > kScratchBytes)
            return fail(FP8BS_ERR_SHAPE, "%d splits of a %lld x %lld output need %llu bytes of scratch; the limit is %llu",
                        (int)splits, (long long)M, (long long)N, (unsigned long long)((uint64_t)splits * per_split),
                        (unsigned long long)kScratchBytes);
        const fp8bs_status e = scratch_ptr(&ws);
        if (e != FP8BS_OK) return e;
    }
    return launched(launch_gemm_blockscaled_splitk(g, splits, ws, stream), "fp8_blockscaled_gemm_splitk_noalloc");
}

fp8bs_status fp8_blockscaled_gemm_splitk_plan(int64_t M, int64_t N, int64_t K, fp8bs_out out, int32_t* splits,
                                              size_t* ws_bytes) {
    if (!splits || !ws_bytes) return fail(FP8BS_ERR_NULL, "splits and ws_bytes are required");
    if (out != FP8BS_OUT_BF16 && out != FP8BS_OUT_FP32) return fail(FP8BS_ERR_UNSUPPORTED, "out %d", out);
    if (M < 0 || N < 0 || K < 0 || K % 128 || N % 128) return fail(FP8BS_ERR_SHAPE, "M %lld N %lld K %lld",
                                                                   (long long)M, (long long)N, (long long)K);
    *splits = (M == 0 || N == 0 || K == 0) ? 1 : plan_gemm_splitk(M, N, K, out == FP8BS_OUT_FP32);
    *ws_bytes = *splits > 1 ? (size_t)*splits * (size_t)M * (size_t)N * 4u : 0;
    return ok();
}

fp8bs_status fp8_blockscaled_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t* plan) {
    if (!plan) return fail(FP8BS_ERR_NULL, "plan is required");
    if (M < 0 || N < 0 || K < 0 || K % 128 || N % 128) return fail(FP8BS_ERR_SHAPE, "M %lld N %lld K %lld",
                                                                   (long long)M, (long long)N, (long long)K);
    plan_gemm_blockscaled(M, N, K, plan);
    return ok();
}

fp8bs_status fp8_grouped_gemm(int64_t total_rows, int64_t N, int64_t K, int32_t G, const int32_t* offsets,
                              const int32_t* a_rows, int64_t a_count, const uint8_t* a, int64_t lda, const float* sa,
                              int64_t sa_stride_m, int64_t sa_stride_k, const uint8_t* b, int64_t ldb,
                              int64_t b_stride_g, const float* sb, int64_t sb_stride_g, int64_t sb_stride_n,
                              int64_t sb_stride_k, void* c, int64_t ldc, fp8bs_out out, hipStream_t stream) {
    if (G < 1) return fail(FP8BS_ERR_SHAPE, "G must be >= 1");
    fp8bs_status v = check_gemm_common(total_rows, N, K, a, lda, b, ldb, c, ldc, out, 128);
    if (v != FP8BS_OK) return v;
    if (total_rows == 0 || N == 0) return ok();
    if (!offsets || !sa || !sb) return fail(FP8BS_ERR_NULL, "offsets, sa and sb are required");
    if (b_stride_g % 16) return fail(FP8BS_ERR_ALIGN, "b_stride_g %% 16 != 0");
    if (!aligned(sa, 4) || !aligned(sb, 4) || !aligned(offsets, 4)) return fail(FP8BS_ERR_ALIGN, "misaligned scales/offsets");
    const int64_t arows = a_rows ? a_count : total_rows;
    if (a_rows && a_count < 1) return fail(FP8BS_ERR_SHAPE, "a_count must be >= 1 with a_rows");
    if ((uint64_t)arows * (uint64_t)lda >= (1ull << 32) || (uint64_t)N * (uint64_t)ldb >= (1ull << 32))
        return fail(FP8BS_ERR_SHAPE, "an operand exceeds 4 GiB");
    // work items (row tiles of at least 128 rows over all groups x 256-column
    // n-tiles) are counted in int32 on the device
    if (((total_rows + 127) / 128 + G) * ((N + 255) / 256) >= (1ll << 31) - 8)
        return fail(FP8BS_ERR_SHAPE, "too many tiles");
    if ((v = check_scale_extent("sa", arows, sa_stride_m, K / 128, sa_stride_k, 4)) != FP8BS_OK) return v;
    if ((v = check_scale_extent("sb", N / 128, sb_stride_n, K / 128, sb_stride_k, 4)) != FP8BS_OK) return v;
    if (sb_stride_g < 0 || b_stride_g < 0) return fail(FP8BS_ERR_STRIDE, "negative group stride");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    GemmArgs g{};
    g.M = total_rows; g.N = N; g.K = K; g.a = a; g.lda = lda; g.sa = sa; g.sa_sm = sa_stride_m; g.sa_sk = sa_stride_k;
    g.b = b; g.ldb = ldb; g.b_sg = b_stride_g; g.sb = sb; g.sb_sg = sb_stride_g; g.sb_sn = sb_stride_n;
    g.sb_sk = sb_stride_k; g.bscale_row = 0; g.c = c; g.ldc = ldc; g.out_f32 = out == FP8BS_OUT_FP32;
    g.G = G; g.offsets = offsets; g.a_rows = a_rows;
    return launched(launch_gemm_grouped(g, stream), "fp8_grouped_gemm");
}

fp8bs_status fp8_grouped_gemm_ws_size(int64_t max_total_rows, int32_t G, int64_t N, size_t* bytes) {
    if (!bytes) return fail(FP8BS_ERR_NULL, "bytes is required");
    if (max_total_rows < 0 || G < 1 || N < 0)
        return fail(FP8BS_ERR_SHAPE, "max_total_rows=%lld G=%d N=%lld", (long long)max_total_rows, (int)G,
                    (long long)N);
    *bytes = 0;     // the work-item lookup reads the device offsets; no table in memory
    return ok();
}

fp8bs_status fp8_grouped_gemm_swiglu_quant(int64_t total_rows, int64_t I, int64_t K, int32_t G, const int32_t* offsets,
                                           const int32_t* a_rows, int64_t a_count, const uint8_t* a, int64_t lda,
                                           const float* sa, int64_t sa_stride_m, int64_t sa_stride_k,
                                           const uint8_t* b, int64_t ldb, int64_t b_stride_g, const float* sb,
                                           int64_t sb_stride_g, int64_t sb_stride_n, int64_t sb_stride_k, uint8_t* hq,
                                           int64_t ld_hq, float* hs, int64_t hs_stride_row, int64_t hs_stride_group,
                                           hipStream_t stream) {
    if (G < 1) return fail(FP8BS_ERR_SHAPE, "G must be >= 1");
    if (I < 0 || I % 128) return fail(FP8BS_ERR_SHAPE, "I %% 128 != 0 (I=%lld)", (long long)I);
    if (I > INT32_MAX / 4) return fail(FP8BS_ERR_SHAPE, "size too large");
    // the operands are checked as for fp8_grouped_gemm with N = 2 I; the
    // bf16 gate/up output is never written (b stands in for it)
    fp8bs_status v = check_gemm_common(total_rows, 2 * I, K, a, lda, b, ldb, b, 2 * I, FP8BS_OUT_BF16, 128);
    if (v != FP8BS_OK) return v;
    if (total_rows == 0 || I == 0) return ok();
    if (!offsets || !sa || !sb || !hq || !hs) return fail(FP8BS_ERR_NULL, "offsets, sa, sb, hq and hs are required");
    if (ld_hq < I) return fail(FP8BS_ERR_STRIDE, "ld_hq < I");
    if (ld_hq % 8 || !aligned(hq, 8)) return fail(FP8BS_ERR_ALIGN, "hq must be 8-byte aligned with ld_hq %% 8 == 0");
    if (!aligned(hs, 4)) return fail(FP8BS_ERR_ALIGN, "hs must be 4-byte aligned");
    if (b_stride_g % 16) return fail(FP8BS_ERR_ALIGN, "b_stride_g %% 16 != 0");
    if (!aligned(sa, 4) || !aligned(sb, 4) || !aligned(offsets, 4)) return fail(FP8BS_ERR_ALIGN, "misaligned scales/offsets");
    const int64_t arows = a_rows ? a_count : total_rows;
    if (a_rows && a_count < 1) return fail(FP8BS_ERR_SHAPE, "a_count must be >= 1 with a_rows");
    if ((uint64_t)arows * (uint64_t)lda >= (1ull << 32) || (uint64_t)(2 * I) * (uint64_t)ldb >= (1ull << 32))
        return fail(FP8BS_ERR_SHAPE, "an operand exceeds 4 GiB");
    if (((total_rows + 127) / 128 + G) * (I / 128) >= (1ll << 31) - 8) return fail(FP8BS_ERR_SHAPE, "too many tiles");
    if ((v = check_scale_extent("sa", arows, sa_stride_m, K / 128, sa_stride_k, 4)) != FP8BS_OK) return v;
    if ((v = check_scale_extent("sb", 2 * I / 128, sb_stride_n, K / 128, sb_stride_k, 4)) != FP8BS_OK) return v;
    if ((v = check_scale_extent("hs", total_rows, hs_stride_row, I / 128, hs_stride_group, 4)) != FP8BS_OK) return v;
    if (sb_stride_g < 0 || b_stride_g < 0) return fail(FP8BS_ERR_STRIDE, "negative group stride");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    GemmArgs g{};
    g.M = total_rows; g.N = 2 * I; g.K = K; g.a = a; g.lda = lda; g.sa = sa; g.sa_sm = sa_stride_m;
    g.sa_sk = sa_stride_k; g.b = b; g.ldb = ldb; g.b_sg = b_stride_g; g.sb = sb; g.sb_sg = sb_stride_g;
    g.sb_sn = sb_stride_n; g.sb_sk = sb_stride_k; g.G = G; g.offsets = offsets; g.a_rows = a_rows;
    return launched(launch_gemm_grouped_swiglu(g, I, hq, ld_hq, hs, hs_stride_row, hs_stride_group, stream),
                    "fp8_grouped_gemm_swiglu_quant");
}

fp8bs_status fp8_silu_mul_quant(const uint16_t* gate_up, int64_t rows, int64_t I, int64_t ld_in, int mx, uint8_t* q,
                                int64_t ld_q, void* s, int64_t s_stride_row, int64_t s_stride_group, uint16_t* h_out,
                                int64_t ld_h, hipStream_t stream) {
    if (mx != 0 && mx != 1) return fail(FP8BS_ERR_UNSUPPORTED, "mx %d", mx);
    if (rows < 0 || I < 0) return fail(FP8BS_ERR_SHAPE, "negative size");
    if (I % (mx ? 32 : 128)) return fail(FP8BS_ERR_SHAPE, "I %% %d != 0", mx ? 32 : 128);
    if (rows * ((I + 127) / 128) > kMaxRuns || rows > INT32_MAX / 2 || I > INT32_MAX / 4)
        return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (rows == 0 || I == 0) return ok();
    if (!gate_up || !q || !s) return fail(FP8BS_ERR_NULL, "gate_up, q and s are required");
    if (ld_in < 2 * I || ld_q < I || (h_out && ld_h < I)) return fail(FP8BS_ERR_STRIDE, "leading dimension too small");
    if (ld_in % 8 || !aligned(gate_up, 16)) return fail(FP8BS_ERR_ALIGN, "gate_up must be 16-byte aligned, ld_in %% 8 == 0");
    if (ld_q % 8 || !aligned(q, 8)) return fail(FP8BS_ERR_ALIGN, "q must be 8-byte aligned with ld_q %% 8 == 0");
    if (h_out && (ld_h % 8 || !aligned(h_out, 16))) return fail(FP8BS_ERR_ALIGN, "h_out must be 16-byte aligned, ld_h %% 8 == 0");
    if (!mx && !aligned(s, 4)) return fail(FP8BS_ERR_ALIGN, "s must be 4-byte aligned");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_silu_mul_quant(gate_up, rows, I, ld_in, mx, q, ld_q, s, s_stride_row, s_stride_group, h_out,
                                          ld_h, stream),
                    "fp8_silu_mul_quant");
}

fp8bs_status fp8_moe_combine(const uint16_t* y, int64_t rows, int64_t H, int64_t ld_y, const int32_t* token_rows,
                             const float* weights, int64_t T, int32_t k, void* out, int64_t ld_out, fp8bs_out out_type,
                             hipStream_t stream) {
    if (out_type != FP8BS_OUT_BF16 && out_type != FP8BS_OUT_FP32) return fail(FP8BS_ERR_UNSUPPORTED, "out %d", out_type);
    if (rows < 0 || H < 0 || T < 0 || k < 1) return fail(FP8BS_ERR_SHAPE, "rows, H, T >= 0 and k >= 1 required");
    if (H % 8) return fail(FP8BS_ERR_SHAPE, "H %% 8 != 0 (H=%lld)", (long long)H);
    // one work-item per (token, 8-column chunk), all in grid dimension x
    if (rows > INT32_MAX || H > INT32_MAX / 2 || T > INT32_MAX / 2 || T * (H / 8) > (1ll << 31))
        return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (T == 0 || H == 0) return ok();
    if (rows == 0) return fail(FP8BS_ERR_SHAPE, "rows == 0 with T > 0");
    if (!y || !token_rows || !weights || !out) return fail(FP8BS_ERR_NULL, "y, token_rows, weights and out are required");
    if (ld_y < H || ld_out < H) return fail(FP8BS_ERR_STRIDE, "ld_y and ld_out must be >= H");
    if (ld_y % 8 || !aligned(y, 16)) return fail(FP8BS_ERR_ALIGN, "y must be 16-byte aligned with ld_y %% 8 == 0");
    if (ld_out % 8 || !aligned(out, 16)) return fail(FP8BS_ERR_ALIGN, "out must be 16-byte aligned with ld_out %% 8 == 0");
    if (!aligned(token_rows, 4) || !aligned(weights, 4)) return fail(FP8BS_ERR_ALIGN, "token_rows, weights misaligned");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_moe_combine(y, rows, H, ld_y, token_rows, weights, T, k, out, ld_out,
                                       out_type == FP8BS_OUT_FP32, stream),
                    "fp8_moe_combine");
}

fp8bs_status mxfp8_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q, int64_t ld_q,
                         uint8_t* s, int64_t s_stride_row, int64_t s_stride_group, hipStream_t stream) {
    if (rows < 0 || cols < 0) return fail(FP8BS_ERR_SHAPE, "negative size");
    if (cols % 32) return fail(FP8BS_ERR_SHAPE, "cols %% 32 != 0");
    if (rows * ((cols + 127) / 128) > kMaxRuns || rows > INT32_MAX / 2 || cols > INT32_MAX / 2)
        return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (rows == 0 || cols == 0) return ok();
    if (!x || !q || !s) return fail(FP8BS_ERR_NULL, "x, q and s are required");
    if (ld_x < cols || ld_q < cols) return fail(FP8BS_ERR_STRIDE, "ld_x and ld_q must be >= cols");
    if (ld_x % 8 || !aligned(x, 16)) return fail(FP8BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    if (ld_q % 8 || !aligned(q, 8)) return fail(FP8BS_ERR_ALIGN, "q must be 8-byte aligned with ld_q %% 8 == 0");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_mx_quant(x, rows, cols, ld_x, q, ld_q, s, s_stride_row, s_stride_group, stream), "mxfp8_quant");
}

fp8bs_status mxfp8_quant_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* qt, int64_t ld_qt,
                           uint8_t* s, int64_t s_stride_row, int64_t s_stride_group, hipStream_t stream) {
    if (rows < 0 || cols < 0) return fail(FP8BS_ERR_SHAPE, "negative size");
    if (rows % 32) return fail(FP8BS_ERR_SHAPE, "rows %% 32 != 0 (rows=%lld)", (long long)rows);
    if (cols % 8) return fail(FP8BS_ERR_SHAPE, "cols %% 8 != 0 (cols=%lld)", (long long)cols);
    // grid: 64-column tiles in x, 128-row tiles in y (at most 65535)
    if ((rows + 127) / 128 > 65535 || cols > INT32_MAX / 2) return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (rows == 0 || cols == 0) return ok();
    if (!x || !qt || !s) return fail(FP8BS_ERR_NULL, "x, qt and s are required");
    if (ld_x < cols || ld_qt < rows) return fail(FP8BS_ERR_STRIDE, "ld_x >= cols and ld_qt >= rows required");
    if (ld_x % 8 || !aligned(x, 16)) return fail(FP8BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    if (ld_qt % 16 || !aligned(qt, 16)) return fail(FP8BS_ERR_ALIGN, "qt must be 16-byte aligned with ld_qt %% 16 == 0");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_mx_quant_t(x, rows, cols, ld_x, qt, ld_qt, s, s_stride_row, s_stride_group, stream),
                    "mxfp8_quant_t");
}

fp8bs_status fp8_quant_dual_axis(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t mx, uint8_t* q,
                                 int64_t ld_q, void* s, int64_t s_stride_row, int64_t s_stride_group, uint8_t* qt,
                                 int64_t ld_qt, void* st, int64_t st_stride_row, int64_t st_stride_group,
                                 hipStream_t stream) {
    if (mx != 0 && mx != 1) return fail(FP8BS_ERR_UNSUPPORTED, "mx %d", (int)mx);
    if (rows < 0 || cols < 0) return fail(FP8BS_ERR_SHAPE, "rows=%lld cols=%lld", (long long)rows, (long long)cols);
    const int64_t rmul = mx ? 32 : 16, cmul = mx ? 32 : 8;
    if (rows % rmul || cols % cmul)
        return fail(FP8BS_ERR_SHAPE, "rows %% %lld and cols %% %lld must be 0 (rows=%lld cols=%lld)", (long long)rmul,
                    (long long)cmul, (long long)rows, (long long)cols);
    // grid: 128-row tiles in x, 128-column tiles in y (at most 65535)
    if (rows > INT32_MAX / 2 || cols > INT32_MAX / 2 || (cols + 127) / 128 > 65535)
        return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (rows == 0 || cols == 0) return ok();
    if (!x || !q || !s || !qt || !st) return fail(FP8BS_ERR_NULL, "x, q, s, qt and st are required");
    if (ld_x < cols || ld_q < cols || ld_qt < rows)
        return fail(FP8BS_ERR_STRIDE, "ld_x >= cols, ld_q >= cols and ld_qt >= rows required");
    if (ld_x % 8 || !aligned(x, 16)) return fail(FP8BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    if (ld_q % 8 || !aligned(q, 8)) return fail(FP8BS_ERR_ALIGN, "q must be 8-byte aligned with ld_q %% 8 == 0");
    if (ld_qt % 8 || !aligned(qt, 8)) return fail(FP8BS_ERR_ALIGN, "qt must be 8-byte aligned with ld_qt %% 8 == 0");
    if (!mx && (!aligned(s, 4) || !aligned(st, 4))) return fail(FP8BS_ERR_ALIGN, "s and st must be 4-byte aligned");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_quant_dual(x, rows, cols, ld_x, mx != 0, q, ld_q, s, s_stride_row, s_stride_group, qt, ld_qt,
                                      st, st_stride_row, st_stride_group, stream),
                    "fp8_quant_dual_axis");
}

fp8bs_status fp8_quant_pow2(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t block_rows, uint8_t* q,
                            int64_t ld_q, uint8_t* s, int64_t ld_s, hipStream_t stream) {
    if (block_rows != 1 && block_rows != 128) return fail(FP8BS_ERR_UNSUPPORTED, "block_rows %d", (int)block_rows);
    if (rows < 0 || cols < 0) return fail(FP8BS_ERR_SHAPE, "negative size");
    if (cols % 8) return fail(FP8BS_ERR_SHAPE, "cols %% 8 != 0 (cols=%lld)", (long long)cols);
    if (rows > INT32_MAX / 2 || cols > INT32_MAX / 2 || (block_rows == 1 && rows * ((cols + 127) / 128) > kMaxRuns) ||
        (block_rows == 128 && (rows + 127) / 128 > 65535))
        return fail(FP8BS_ERR_SHAPE, "tensor too large");
    if (rows == 0 || cols == 0) return ok();
    if (!x || !q || !s) return fail(FP8BS_ERR_NULL, "x, q and s are required");
    if (ld_x < cols || ld_q < cols || ld_s < (cols + 127) / 128)
        return fail(FP8BS_ERR_STRIDE, "ld_x, ld_q >= cols and ld_s >= ceil(cols / 128) required");
    if (ld_x % 8 || !aligned(x, 16)) return fail(FP8BS_ERR_ALIGN, "x must be 16-byte aligned with ld_x %% 8 == 0");
    if (ld_q % 8 || !aligned(q, 8)) return fail(FP8BS_ERR_ALIGN, "q must be 8-byte aligned with ld_q %% 8 == 0");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_quant_pow2(x, rows, cols, ld_x, block_rows, q, ld_q, s, ld_s, stream), "fp8_quant_pow2");
}

fp8bs_status fp8_blockscaled_gemm_pow2(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                       const uint8_t* sa, int64_t lds_a, const uint8_t* b, int64_t ldb,
                                       const uint8_t* sb, int64_t lds_b, void* c, int64_t ldc, fp8bs_out out,
                                       hipStream_t stream) {
    fp8bs_status v = check_gemm_common(M, N, K, a, lda, b, ldb, c, ldc, out, 128);
    if (v != FP8BS_OK) return v;
    if (M == 0 || N == 0) return ok();
    if (!sa || !sb) return fail(FP8BS_ERR_NULL, "sa and sb are required");
    // each 128-K slice's byte is read as part of the 4-byte word of slices 4(kb/4) .. +3
    const int64_t words = 4 * ((K / 128 + 3) / 4);
    if (lds_a < words || lds_b < words) return fail(FP8BS_ERR_STRIDE, "lds_a, lds_b must be >= 4 * ceil(K / 512)");
    if (lds_a % 4 || lds_b % 4 || !aligned(sa, 4) || !aligned(sb, 4))
        return fail(FP8BS_ERR_ALIGN, "scale arrays must be 4-byte aligned with lds %% 4 == 0");
    if ((uint64_t)M * (uint64_t)lda >= (1ull << 32) || (uint64_t)N * (uint64_t)ldb >= (1ull << 32))
        return fail(FP8BS_ERR_SHAPE, "an operand exceeds 4 GiB");
    if (((M + 127) / 128) * ((N + 159) / 160) >= (1ll << 31) - 8) return fail(FP8BS_ERR_SHAPE, "too many tiles");
    if ((v = check_scale_extent("sa", M, lds_a, 1, 0, 1)) != FP8BS_OK) return v;
    if ((v = check_scale_extent("sb", N / 128, lds_b, 1, 0, 1)) != FP8BS_OK) return v;
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    Pow2GemmArgs g{};
    g.M = M; g.N = N; g.K = K; g.a = a; g.lda = lda; g.sa = sa; g.lds_a = lds_a;
    g.b = b; g.ldb = ldb; g.sb = sb; g.lds_b = lds_b; g.c = c; g.ldc = ldc; g.out_f32 = out == FP8BS_OUT_FP32;
    return launched(launch_gemm_pow2(g, stream), "fp8_blockscaled_gemm_pow2");
}

fp8bs_status mxfp8_gemm(int64_t rows, int64_t N, int64_t K, int32_t G, const int32_t* offsets, const int32_t* a_rows,
                        int64_t a_count, const uint8_t* a, int64_t lda, const uint8_t* sa, int64_t lds_a,
                        const uint8_t* b, int64_t ldb, int64_t b_stride_g, const uint8_t* sb, int64_t lds_b,
                        int64_t sb_stride_g, void* c, int64_t ldc, fp8bs_out out, hipStream_t stream) {
    if (G < 0) return fail(FP8BS_ERR_SHAPE, "G < 0");
    fp8bs_status v = check_gemm_common(rows, N, K, a, lda, b, ldb, c, ldc, out, 128);
    if (v != FP8BS_OK) return v;
    if (rows == 0 || N == 0) return ok();
    if (!sa || !sb) return fail(FP8BS_ERR_NULL, "sa and sb are required");
    if (G > 0 && !offsets) return fail(FP8BS_ERR_NULL, "offsets required when G > 0");
    if (lds_a < K / 32 || lds_b < K / 32) return fail(FP8BS_ERR_STRIDE, "scale leading dimension < K/32");
    if (lds_a % 4 || lds_b % 4 || !aligned(sa, 4) || !aligned(sb, 4))
        return fail(FP8BS_ERR_ALIGN, "scale arrays must be 4-byte aligned with lds %% 4 == 0");
    if (G > 0 && b_stride_g % 16) return fail(FP8BS_ERR_ALIGN, "b_stride_g %% 16 != 0");
    const int64_t arows = (G > 0 && a_rows) ? a_count : rows;
    if (G > 0 && a_rows && a_count < 1) return fail(FP8BS_ERR_SHAPE, "a_count must be >= 1 with a_rows");
    if ((uint64_t)arows * (uint64_t)lda >= (1ull << 32) || (uint64_t)N * (uint64_t)ldb >= (1ull << 32))
        return fail(FP8BS_ERR_SHAPE, "an operand exceeds 4 GiB");
    // work items (row tiles of at least 128 rows, over all groups) x n-tiles
    // are counted in int32 on the device
    if (((rows + 127) / 128 + G) * ((N + 255) / 256) >= (1ll << 31) - 8)
        return fail(FP8BS_ERR_SHAPE, "too many tiles");
    if ((v = check_scale_extent("sa", arows, lds_a, 1, 0, 1)) != FP8BS_OK) return v;
    if ((v = check_scale_extent("sb", N, lds_b, 1, 0, 1)) != FP8BS_OK) return v;
    if (G > 0 && (sb_stride_g < 0 || b_stride_g < 0)) return fail(FP8BS_ERR_STRIDE, "negative group stride");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    MxGemmArgs g{};
    g.M = rows; g.N = N; g.K = K; g.a = a; g.lda = lda; g.sa = sa; g.lds_a = lds_a;
    g.b = b; g.ldb = ldb; g.b_sg = G > 0 ? b_stride_g : 0; g.sb = sb; g.lds_b = lds_b; g.sb_sg = G > 0 ? sb_stride_g : 0;
    g.c = c; g.ldc = ldc; g.out_f32 = out == FP8BS_OUT_FP32; g.G = G; g.offsets = G > 0 ? offsets : nullptr;
    g.a_rows = G > 0 ? a_rows : nullptr;
    return launched(launch_gemm_mx(g, stream), "mxfp8_gemm");
}

fp8bs_status mxfp8_grouped_gemm_swiglu_quant(int64_t total_rows, int64_t I, int64_t K, int32_t G,
                                             const int32_t* offsets, const int32_t* a_rows, int64_t a_count,
                                             const uint8_t* a, int64_t lda, const uint8_t* sa, int64_t lds_a,
                                             const uint8_t* b, int64_t ldb, int64_t b_stride_g, const uint8_t* sb,
                                             int64_t lds_b, int64_t sb_stride_g, uint8_t* hq, int64_t ld_hq,
                                             uint8_t* hs, int64_t hs_stride_row, int64_t hs_stride_group,
                                             hipStream_t stream) {
    if (G < 1) return fail(FP8BS_ERR_SHAPE, "G must be >= 1");
    if (I < 0 || I % 128) return fail(FP8BS_ERR_SHAPE, "I %% 128 != 0 (I=%lld)", (long long)I);
    if (I > INT32_MAX / 4) return fail(FP8BS_ERR_SHAPE, "size too large");
    // the operands are checked as for the grouped mxfp8_gemm with N = 2 I;
    // the bf16 gate/up output is never written (b stands in for it)
    fp8bs_status v = check_gemm_common(total_rows, 2 * I, K, a, lda, b, ldb, b, 2 * I, FP8BS_OUT_BF16, 128);
    if (v != FP8BS_OK) return v;
    if (total_rows == 0 || I == 0) return ok();
    if (!offsets || !sa || !sb || !hq || !hs) return fail(FP8BS_ERR_NULL, "offsets, sa, sb, hq and hs are required");
    if (lds_a < K / 32 || lds_b < K / 32) return fail(FP8BS_ERR_STRIDE, "scale leading dimension < K/32");
    if (lds_a % 4 || lds_b % 4 || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(offsets, 4))
        return fail(FP8BS_ERR_ALIGN, "scale arrays must be 4-byte aligned with lds %% 4 == 0");
    if (ld_hq < I) return fail(FP8BS_ERR_STRIDE, "ld_hq < I");
    if (ld_hq % 8 || !aligned(hq, 8)) return fail(FP8BS_ERR_ALIGN, "hq must be 8-byte aligned with ld_hq %% 8 == 0");
    if (b_stride_g % 16) return fail(FP8BS_ERR_ALIGN, "b_stride_g %% 16 != 0");
    const int64_t arows = a_rows ? a_count : total_rows;
    if (a_rows && a_count < 1) return fail(FP8BS_ERR_SHAPE, "a_count must be >= 1 with a_rows");
    if ((uint64_t)arows * (uint64_t)lda >= (1ull << 32) || (uint64_t)(2 * I) * (uint64_t)ldb >= (1ull << 32))
        return fail(FP8BS_ERR_SHAPE, "an operand exceeds 4 GiB");
    if (((total_rows + 127) / 128 + G) * (I / 128) >= (1ll << 31) - 8) return fail(FP8BS_ERR_SHAPE, "too many tiles");
    if ((v = check_scale_extent("sa", arows, lds_a, 1, 0, 1)) != FP8BS_OK) return v;
    if ((v = check_scale_extent("sb", 2 * I, lds_b, 1, 0, 1)) != FP8BS_OK) return v;
    if ((v = check_scale_extent("hs", total_rows, hs_stride_row, I / 32, hs_stride_group, 1)) != FP8BS_OK) return v;
    if (sb_stride_g < 0 || b_stride_g < 0) return fail(FP8BS_ERR_STRIDE, "negative group stride");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    MxGemmArgs g{};
    g.M = total_rows; g.N = 2 * I; g.K = K; g.a = a; g.lda = lda; g.sa = sa; g.lds_a = lds_a;
    g.b = b; g.ldb = ldb; g.b_sg = b_stride_g; g.sb = sb; g.lds_b = lds_b; g.sb_sg = sb_stride_g;
    g.G = G; g.offsets = offsets; g.a_rows = a_rows;
    return launched(launch_gemm_mx_swiglu(g, I, hq, ld_hq, hs, hs_stride_row, hs_stride_group, stream),
                    "mxfp8_grouped_gemm_swiglu_quant");
}

fp8bs_status fp8bs_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
    if (n < 0) return fail(FP8BS_ERR_SHAPE, "n < 0");
    if (n == 0) return ok();
    if (!in || !out) return fail(FP8BS_ERR_NULL, "in and out are required");
    if (!aligned(in, 4)) return fail(FP8BS_ERR_ALIGN, "in must be 4-byte aligned");
    fp8bs_status d = check_device();
    if (d != FP8BS_OK) return d;
    return launched(launch_e4m3_encode(in, out, n, stream), "fp8bs_e4m3_encode");
}

}  // extern "C"
