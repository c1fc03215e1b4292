// MoE combine: each token's output is the routing-weighted sum of its
// experts' outputs, read from the grouped (expert-sorted) down-projection
// output through the token's row positions.  It closes the MoE layer whose
// grouped GEMMs run in block-wise FP8 ("Low Precision RL", section
// "2. Unified block-wise FP8 (DeepSeek-style)", the Qwen3-30B-A3B recipe).
//
// HBM-bound: k bf16 rows read per token, one row written.  One thread owns
// one (token, 8-column chunk) pair: the k rows of a token are each read as
// one contiguous run across the workgroup (16-byte loads), all k loads are
// issued before the FMAs, and the sum is an fp32 FMA chain in slot order
// (deterministic: no atomics, no order that depends on scheduling).
#include "device_common.h"
#include "internal.h"

namespace fp8bs {
namespace {

constexpr int kThreads = 256;

template <bool OUTF32>
__global__ void __launch_bounds__(kThreads) k_moe_combine(const uint16_t* __restrict__ y, int32_t rows, int32_t nch,
                                                          int64_t ld_y, const int32_t* __restrict__ pos,
                                                          const float* __restrict__ w, int64_t T, int32_t k,
                                                          void* __restrict__ out, int64_t ld_out) {
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= T * nch) return;
    const int64_t t = idx / nch;
    const int c = (int)(idx - t * nch);
    const int32_t* pt = pos + t * k;
    const float* wt = w + t * k;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 8) {
        uint4 raw[8];
        float wj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
                // positions outside [0, rows) are clamped: a bad map reads
                // wrong rows, never outside y
                const int r = min(max(pt[j0 + u], 0), rows - 1);
                raw[u] = load_nt16(y + (int64_t)r * ld_y + 8 * c);
                wj[u] = wt[j0 + u];
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
                const uint32_t v[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = __builtin_fmaf(wj[u], bf16_lo(v[i]), acc[2 * i]);
                    acc[2 * i + 1] = __builtin_fmaf(wj[u], bf16_hi(v[i]), acc[2 * i + 1]);
                }
            }
        }
    }
    if (OUTF32) {
        float* dst = static_cast<float*>(out) + t * ld_out + 8 * c;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
        uint16_t* dst = static_cast<uint16_t*>(out) + t * ld_out + 8 * c;
        *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
}

}  // namespace

hipError_t launch_moe_combine(const uint16_t* y, int64_t rows, int64_t H, int64_t ld_y, const int32_t* pos,
                              const float* w, int64_t T, int32_t k, void* out, int64_t ld_out, int out_f32,
                              hipStream_t st) {
    if (T == 0 || H == 0) return hipSuccess;
    const int32_t nch = (int32_t)(H / 8);
    const int64_t blocks = (T * nch + kThreads - 1) / kThreads;
    if (out_f32)
        hipLaunchKernelGGL(k_moe_combine<true>, dim3((unsigned)blocks), dim3(kThreads), 0, st, y, (int32_t)rows, nch,
                           ld_y, pos, w, T, k, out, ld_out);
    else
        hipLaunchKernelGGL(k_moe_combine<false>, dim3((unsigned)blocks), dim3(kThreads), 0, st, y, (int32_t)rows, nch,
                           ld_y, pos, w, T, k, out, ld_out);
    return hipGetLastError();
}

}  // namespace fp8bs
