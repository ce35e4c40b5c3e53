// Combine kernel for gfx950: K-way gather of expert output rows with an fp32 weighted sum.
//
// Arithmetic of ReadBufferAndWeightedSum ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 7.8):
// fp32 accumulator from zero; for k ascending, widen the bf16 row to fp32, multiply by the k-th
// weight, add; round once to bf16 with ties-to-even (CAST_RINT). This file is compiled with
// -ffp-contract=off, so each product and sum is rounded to fp32 on its own, as the separate
// Muls / Add steps on the page do.
//
// One workgroup per token. The K gathered rows are contiguous runs of 2H bytes; consecutive lanes
// read consecutive 16-byte vectors of each row, and all K loads of a vector position are issued
// before any arithmetic so K x 16 bytes per lane are in flight. Slots and weights are uniform per
// workgroup and live in scalar registers.

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int MAXV, int KMAX>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const uint8_t *__restrict__ expert_out, int64_t stride, int64_t rows,
    const int32_t *__restrict__ slot_idx, const float *__restrict__ weights, int K, int nvec,
    u32x4 *__restrict__ y) {
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    int64_t off[KMAX];
    float wk[KMAX];
    bool live[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        live[k] = false;
        off[k] = 0;
        wk[k] = 0.0f;
        if (k < K) {
            const int64_t s = slot_idx[(int64_t)t * K + k];
            if (s >= 0 && s < rows) {
                live[k] = true;
                off[k] = s * stride;
                wk[k] = weights[(int64_t)t * K + k];
            }
        }
    }
    u32x4 *dst = y + (int64_t)t * nvec;
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
        const int v = tid + j * kThreads;
        if (v < nvec) {
            u32x4 xv[KMAX];
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (live[k])
                    xv[k] = *reinterpret_cast<const u32x4 *>(expert_out + off[k] + ((int64_t)v << 4));
            }
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (live[k]) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const float lo = __uint_as_float(xv[k][w] << 16);
                        const float hi = __uint_as_float(xv[k][w] & 0xFFFF0000u);
                        acc[2 * w] = acc[2 * w] + wk[k] * lo;
                        acc[2 * w + 1] = acc[2 * w + 1] + wk[k] * hi;
                    }
                }
            }
            u32x4 out;
#pragma unroll
            for (int w = 0; w < 4; ++w) out[w] = bf16_rne(acc[2 * w]) | (bf16_rne(acc[2 * w + 1]) << 16);
            dst[v] = out;
        }
    }
}

template <int MAXV, int KMAX>
hipError_t launch(const void *expert_out, int64_t stride, int64_t rows, const int32_t *slot_idx,
                  const float *weights, int S, int K, int nvec, void *y, hipStream_t stream) {
    hipLaunchKernelGGL((combine_kernel<MAXV, KMAX>), dim3(S), dim3(kThreads), 0, stream,
                       static_cast<const uint8_t *>(expert_out), stride, rows, slot_idx, weights, K,
                       nvec, static_cast<u32x4 *>(y));
    return hipGetLastError();
}

template <int MAXV>
hipError_t launch_k(const void *expert_out, int64_t stride, int64_t rows, const int32_t *slot_idx,
                    const float *weights, int S, int K, int nvec, void *y, hipStream_t stream) {
    if (K <= 2) return launch<MAXV, 2>(expert_out, stride, rows, slot_idx, weights, S, K, nvec, y, stream);
    if (K <= 4) return launch<MAXV, 4>(expert_out, stride, rows, slot_idx, weights, S, K, nvec, y, stream);
    if (K <= 8) return launch<MAXV, 8>(expert_out, stride, rows, slot_idx, weights, S, K, nvec, y, stream);
    return launch<MAXV, 16>(expert_out, stride, rows, slot_idx, weights, S, K, nvec, y, stream);
}

}  // namespace

hipError_t launch_combine(const void *expert_out, int64_t row_stride_bytes, int64_t expert_rows,
                          const int32_t *slot_idx, const float *topk_weights, int32_t S,
                          int32_t H, int32_t K, void *y, hipStream_t stream) {
    const int nvec = H / 8;
    const int per = (nvec + kThreads - 1) / kThreads;
    if (per <= 1) return launch_k<1>(expert_out, row_stride_bytes, expert_rows, slot_idx, topk_weights, S, K, nvec, y, stream);
    if (per <= 2) return launch_k<2>(expert_out, row_stride_bytes, expert_rows, slot_idx, topk_weights, S, K, nvec, y, stream);
    if (per <= 4) return launch_k<4>(expert_out, row_stride_bytes, expert_rows, slot_idx, topk_weights, S, K, nvec, y, stream);
    return launch_k<8>(expert_out, row_stride_bytes, expert_rows, slot_idx, topk_weights, S, K, nvec, y, stream);
}

}  // namespace moe
