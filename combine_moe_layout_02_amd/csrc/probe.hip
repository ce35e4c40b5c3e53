// Bandwidth probes for the measurement (declared in include/moe_probe.h): a write-only fill, a
// read-only stream and a copy over caller buffers, with the cache policies of the path's kernels
// (streaming stores, default loads). They give the practical ceilings of the three access
// patterns on the running GPU, next to the 8 TB/s HBM specification. Nothing on the hot path
// calls them.

#include "pack_rows.h"

namespace moe {
namespace {

using namespace rows;

constexpr int kProbeThreads = 256;
constexpr int kProbeVecs = 8;  // 16-byte vectors per lane per workgroup: 32 KB per workgroup

__device__ inline __amdgpu_buffer_rsrc_t span_rsrc(const void *base, int64_t off, int64_t bytes) {
    const int64_t left = bytes - off;
    const int32_t n = left < 0x40000000 ? (int32_t)left : 0x40000000;
    return rsrc(static_cast<const uint8_t *>(base) + off, n);
}

// workgroup g covers bytes [g * 32 KB, (g + 1) * 32 KB), lane-interleaved 4 KB rows
__global__ __launch_bounds__(kProbeThreads) void probe_fill_kernel(uint8_t *__restrict__ dst, int64_t bytes) {
    const int64_t off = (int64_t)blockIdx.x * (kProbeThreads * kProbeVecs * 16);
    const __amdgpu_buffer_rsrc_t d = span_rsrc(dst, off, bytes);
    const u32x4 v = {blockIdx.x, threadIdx.x, 0x9e3779b9u, 0u};
#pragma unroll
    for (int i = 0; i < kProbeVecs; ++i) store16(v, d, (i * kProbeThreads + threadIdx.x) << 4);
}

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint8_t *__restrict__ src, int64_t bytes,
                                                                   uint32_t *__restrict__ sink) {
    const int64_t off = (int64_t)blockIdx.x * (kProbeThreads * kProbeVecs * 16);
    const __amdgpu_buffer_rsrc_t s = span_rsrc(src, off, bytes);
    u32x4 r[kProbeVecs];
#pragma unroll
    for (int i = 0; i < kProbeVecs; ++i) r[i] = load16(s, (i * kProbeThreads + threadIdx.x) << 4);
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kProbeVecs; ++i) acc ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
    if (acc == 0x6d2b79f5u) sink[0] = acc;  // keeps the loads; true for almost no data
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const uint8_t *__restrict__ src,
                                                                   uint8_t *__restrict__ dst, int64_t bytes) {
    const int64_t off = (int64_t)blockIdx.x * (kProbeThreads * kProbeVecs * 16);
    const __amdgpu_buffer_rsrc_t s = span_rsrc(src, off, bytes);
    const __amdgpu_buffer_rsrc_t d = span_rsrc(dst, off, bytes);
    u32x4 r[kProbeVecs];
#pragma unroll
    for (int i = 0; i < kProbeVecs; ++i) r[i] = load16(s, (i * kProbeThreads + threadIdx.x) << 4);
#pragma unroll
    for (int i = 0; i < kProbeVecs; ++i) store16(r[i], d, (i * kProbeThreads + threadIdx.x) << 4);
}

constexpr int64_t kProbeChunk = kProbeThreads * kProbeVecs * 16;

bool probe_ok(const void *p, int64_t bytes) {
    return p && bytes > 0 && bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0 &&
           (bytes + kProbeChunk - 1) / kProbeChunk < 0x7fffffff;
}

}  // namespace
}  // namespace moe

extern "C" {

int moe_probe_fill(void *dst, int64_t bytes, hipStream_t stream) {
    if (!moe::probe_ok(dst, bytes)) return MOE_ERR_ARG;
    const uint32_t grid = (uint32_t)((bytes + moe::kProbeChunk - 1) / moe::kProbeChunk);
    hipLaunchKernelGGL(moe::probe_fill_kernel, dim3(grid), dim3(moe::kProbeThreads), 0, stream,
                       static_cast<uint8_t *>(dst), bytes);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream) {
    if (!moe::probe_ok(src, bytes) || !sink) return MOE_ERR_ARG;
    const uint32_t grid = (uint32_t)((bytes + moe::kProbeChunk - 1) / moe::kProbeChunk);
    hipLaunchKernelGGL(moe::probe_read_kernel, dim3(grid), dim3(moe::kProbeThreads), 0, stream,
                       static_cast<const uint8_t *>(src), bytes, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream) {
    if (!moe::probe_ok(src, bytes) || !moe::probe_ok(dst, bytes)) return MOE_ERR_ARG;
    const uint32_t grid = (uint32_t)((bytes + moe::kProbeChunk - 1) / moe::kProbeChunk);
    hipLaunchKernelGGL(moe::probe_copy_kernel, dim3(grid), dim3(moe::kProbeThreads), 0, stream,
                       static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), bytes);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
