// Combine kernels for gfx950: K-way gather of expert output rows with an fp32 weighted sum, and the
// CAM two-pass form (scatter the rows to position t*K + k, then reduce K contiguous rows).
//
// Arithmetic of ReadBufferAndWeightedSum ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 7.8):
// fp32 accumulator from zero; for k ascending, widen the bf16 row to fp32, multiply by the k-th
// weight, add; round once to bf16 with ties-to-even (CAST_RINT). This file is compiled with
// -ffp-contract=off, so each product and sum is rounded to fp32 on its own, as the separate
// Muls / Add steps on the page do.
//
// Each token row is split into parts of 32 16-byte vectors and one half-wave workgroup owns one
// (token, part): each lane issues its K gathered 16-byte loads back to back, then reduces them and
// stores one 16-byte vector of y. All parts of a token run on one XCD. Measured on MI355X at S=4096..8192, H=7168, K=8, 32-lane parts
// are 1-3% faster than 64- or 128-lane parts and 16-lane parts a third slower. Slots and weights
// are uniform per workgroup and live in scalar registers. The gathered rows are read exactly once,
// so they are loaded with the non-temporal policy and do not displace reusable data from the
// caches; y is stored with the sc0 sc1 policy. Each gathered row gets its own buffer descriptor
// whose range is the row, so an out-of-range offset reads zero instead of faulting.

#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPartThreads = 32;
constexpr int kLoadPolicy = 2;        // nt
constexpr int kStorePolicy = 1 | 16;  // sc0 sc1
constexpr int kScatterStorePolicy = 1 | 16 | 2;  // sc0 sc1 nt: staging rows stream to HBM
// Lanes per scatter workgroup. At S=4096, H=7168, K=8: 167 us with 128 lanes against 208 us with
// 32, 169 us with 64 and 180 us with 256.
constexpr int kScatterThreads = 128;

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

__device__ inline uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// grid = 8 * ceil(S / 8) * nparts; workgroup b runs on XCD x = b % 8 (the dispatcher hands
// workgroups to the XCDs in turn) and produces vectors [q, q + 1) * kPartThreads of y[t], with
// m = b / 8, t = 8 * (m / nparts) + x and q = m % nparts: all parts of token t on XCD t % 8, so each
// XCD writes whole rows of y (about 1% faster than token-major order at S = 4096..8192, H = 7168).
// STAGED: the rows were first scattered to position t*K + k, so row t*K + k is read for every
// valid k.
template <int KMAX, bool STAGED>
__global__ __launch_bounds__(kPartThreads) void combine_kernel(
    const uint8_t *__restrict__ expert_out, int64_t stride, int64_t rows,
    const int32_t *__restrict__ slot_idx, const float *__restrict__ weights, int S, int K,
    int nvec, int nparts, uint8_t *__restrict__ y) {
    const int m = blockIdx.x >> 3;
    const int i = m / nparts;
    const int q = m - i * nparts;
    const int t = 8 * i + (blockIdx.x & 7);
    if (t >= S) return;
    const int v = q * kPartThreads + threadIdx.x;
    const int row_bytes = nvec << 4;
    __amdgpu_buffer_rsrc_t src[KMAX];
    float wk[KMAX];
    bool live[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        live[k] = false;
        wk[k] = 0.0f;
        src[k] = rsrc(expert_out, 0);
        if (k < K) {
            int64_t s = slot_idx[(int64_t)t * K + k];
            if (STAGED && s >= 0) s = (int64_t)t * K + k;
            if (s >= 0 && s < rows) {
                live[k] = true;
                src[k] = rsrc(expert_out + s * stride, row_bytes);
                wk[k] = weights[(int64_t)t * K + k];
            }
        }
    }
    if (v >= nvec) return;
    u32x4 xv[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        if (live[k]) xv[k] = __builtin_amdgcn_raw_buffer_load_b128(src[k], v << 4, 0, kLoadPolicy);
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
    const __amdgpu_buffer_rsrc_t dst = rsrc(y + (int64_t)t * row_bytes, row_bytes);
    __builtin_amdgcn_raw_buffer_store_b128(out, dst, v << 4, 0, kStorePolicy);
}

// Scatter pass of the two-pass combine ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 7.5
// CopyBufferToShareAndSetStatus): expert output row s goes to staging row t*K + k, (t, k) from the
// triple the row's slot carried (expand_idx[s] = (src_rank, t, k)). grid = max_rows * nparts;
// workgroup (s, q) moves vectors [q, q + 1) * kScatterThreads of row s. The row load is issued before
// N and the triple arrive; rows at or past N, and triples outside [0, S) x [0, K), move nothing.
__global__ __launch_bounds__(kScatterThreads) void combine_scatter_kernel(
    const uint8_t *__restrict__ expert_out, int64_t stride, const int32_t *__restrict__ expand_idx,
    const int32_t *__restrict__ num_rows, int64_t max_rows, int S, int K, int nvec, int nparts,
    uint8_t *__restrict__ staging, int64_t staging_stride) {
    const int64_t s = blockIdx.x / nparts;
    const int q = blockIdx.x - (int)(s * nparts);
    const int v = q * kScatterThreads + threadIdx.x;
    const int row_bytes = nvec << 4;
    const bool in_row = v < nvec;
    const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(rsrc(expert_out + s * stride, row_bytes),
                                                          in_row ? v << 4 : 0, 0, kLoadPolicy);
    const int64_t n = min((int64_t)*num_rows, max_rows);
    const int t = expand_idx[s * 3 + 1], k = expand_idx[s * 3 + 2];
    if (s >= n || t < 0 || t >= S || k < 0 || k >= K || !in_row) return;
    const __amdgpu_buffer_rsrc_t dst =
        rsrc(staging + ((int64_t)t * K + k) * staging_stride, row_bytes);
    __builtin_amdgcn_raw_buffer_store_b128(d, dst, v << 4, 0, kScatterStorePolicy);
}

template <int KMAX, bool STAGED>
hipError_t launch(const void *expert_out, int64_t stride, int64_t rows, const int32_t *slot_idx,
                  const float *weights, int S, int K, int nvec, void *y, hipStream_t stream) {
    const int nparts = (nvec + kPartThreads - 1) / kPartThreads;
    const uint32_t grid = 8u * (uint32_t)((S + 7) / 8) * (uint32_t)nparts;
    hipLaunchKernelGGL((combine_kernel<KMAX, STAGED>), dim3(grid), dim3(kPartThreads), 0, stream,
                       static_cast<const uint8_t *>(expert_out), stride, rows, slot_idx, weights, S,
                       K, nvec, nparts, static_cast<uint8_t *>(y));
    return hipGetLastError();
}

template <bool STAGED>
hipError_t launch_k(const void *expert_out, int64_t stride, int64_t rows, const int32_t *slot_idx,
                    const float *weights, int S, int K, int nvec, void *y, hipStream_t stream) {
    if (K <= 2) return launch<2, STAGED>(expert_out, stride, rows, slot_idx, weights, S, K, nvec, y, stream);
    if (K <= 4) return launch<4, STAGED>(expert_out, stride, rows, slot_idx, weights, S, K, nvec, y, stream);
    if (K <= 8) return launch<8, STAGED>(expert_out, stride, rows, slot_idx, weights, S, K, nvec, y, stream);
    return launch<16, STAGED>(expert_out, stride, rows, slot_idx, weights, S, K, nvec, y, stream);
}

}  // namespace

hipError_t launch_combine(const void *expert_out, int64_t row_stride_bytes, int64_t expert_rows,
                          const int32_t *slot_idx, const float *topk_weights, int32_t S,
                          int32_t H, int32_t K, void *y, hipStream_t stream) {
    return launch_k<false>(expert_out, row_stride_bytes, expert_rows, slot_idx, topk_weights, S, K,
                           H / 8, y, stream);
}

hipError_t launch_combine_scatter(const void *expert_out, int64_t row_stride_bytes,
                                  int64_t expert_rows, const int32_t *expand_idx,
                                  const int32_t *num_rows, int32_t S, int32_t K, int32_t H,
                                  void *staging, int64_t staging_stride_bytes, hipStream_t stream) {
    if (expert_rows == 0) return hipSuccess;
    const int nvec = H / 8;
    const int nparts = (nvec + kScatterThreads - 1) / kScatterThreads;
    hipLaunchKernelGGL(combine_scatter_kernel, dim3((uint32_t)(expert_rows * nparts)),
                       dim3(kScatterThreads), 0, stream, static_cast<const uint8_t *>(expert_out),
                       row_stride_bytes, expand_idx, num_rows, expert_rows, S, K, nvec, nparts,
                       static_cast<uint8_t *>(staging), staging_stride_bytes);
    return hipGetLastError();
}

hipError_t launch_combine_staged(const void *staging, int64_t staging_stride_bytes,
                                 const int32_t *slot_idx, const float *topk_weights, int32_t S,
                                 int32_t H, int32_t K, void *y, hipStream_t stream) {
    return launch_k<true>(staging, staging_stride_bytes, (int64_t)S * K, slot_idx, topk_weights, S,
                          K, H / 8, y, stream);
}

}  // namespace moe
