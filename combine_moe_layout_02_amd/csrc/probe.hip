// Bandwidth probes for the measurement (declared in include/moe_probe.h): a write-only fill, a
// read-only stream and a copy over caller buffers, with the cache policies of the path's kernels
// (streaming stores, nt loads for data read once). They give the practical ceilings of the three
// access patterns on the running GPU, next to the 8 TB/s HBM specification. Nothing on the hot
// path calls them.

#include "pack_rows.h"

namespace moe {
namespace {

using namespace rows;

constexpr int kPolicyNtLoad = 2;  // nt: loads of data read once, as the combine's row loads

// Shapes measured on MI355X over 1 GiB (the fastest of the shapes tried for each pattern): fill
// 7.0 TB/s with one 16-byte streaming store per lane in 256-lane workgroups (4 KB each; four or
// eight stores per lane: 5.9 and 5.6 TB/s); read 7.0 TB/s with four nt loads per lane in 512-lane
// workgroups (32 KB each); copy 6.6 TB/s of read + write bytes with one nt load and one streaming
// store per lane in 256-lane workgroups.
constexpr int kFillThreads = 256, kFillVecs = 1;
constexpr int kReadThreads = 512, kReadVecs = 4;
constexpr int kCopyThreads = 256, kCopyVecs = 1;

__device__ inline __amdgpu_buffer_rsrc_t span_rsrc(const void *base, int64_t off, int64_t bytes) {
    const int64_t left = bytes - off;
    const int32_t n = left < 0x40000000 ? (int32_t)left : 0x40000000;
    return rsrc(static_cast<const uint8_t *>(base) + off, n);
}

// workgroup g covers bytes [g * T * V * 16, (g + 1) * T * V * 16); the buffer range drops the
// part of the last workgroup past `bytes`
__global__ __launch_bounds__(kFillThreads) void probe_fill_kernel(uint8_t *__restrict__ dst, int64_t bytes) {
    const int64_t off = (int64_t)blockIdx.x * (kFillThreads * kFillVecs * 16);
    const __amdgpu_buffer_rsrc_t d = span_rsrc(dst, off, bytes);
    const u32x4 v = {blockIdx.x, threadIdx.x, 0x9e3779b9u, 0u};
#pragma unroll
    for (int i = 0; i < kFillVecs; ++i) store16(v, d, (i * kFillThreads + threadIdx.x) << 4);
}

__global__ __launch_bounds__(kReadThreads) void probe_read_kernel(const uint8_t *__restrict__ src, int64_t bytes,
                                                                  uint32_t *__restrict__ sink) {
    const int64_t off = (int64_t)blockIdx.x * (kReadThreads * kReadVecs * 16);
    const __amdgpu_buffer_rsrc_t s = span_rsrc(src, off, bytes);
    u32x4 r[kReadVecs];
#pragma unroll
    for (int i = 0; i < kReadVecs; ++i)
        r[i] = __builtin_amdgcn_raw_buffer_load_b128(s, (i * kReadThreads + threadIdx.x) << 4, 0, kPolicyNtLoad);
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kReadVecs; ++i) acc ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
    if (acc == 0x6d2b79f5u) sink[0] = acc;  // keeps the loads; true for almost no data
}

__global__ __launch_bounds__(kCopyThreads) void probe_copy_kernel(const uint8_t *__restrict__ src,
                                                                  uint8_t *__restrict__ dst, int64_t bytes) {
    const int64_t off = (int64_t)blockIdx.x * (kCopyThreads * kCopyVecs * 16);
    const __amdgpu_buffer_rsrc_t s = span_rsrc(src, off, bytes);
    const __amdgpu_buffer_rsrc_t d = span_rsrc(dst, off, bytes);
    u32x4 r[kCopyVecs];
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i)
        r[i] = __builtin_amdgcn_raw_buffer_load_b128(s, (i * kCopyThreads + threadIdx.x) << 4, 0, kPolicyNtLoad);
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i) store16(r[i], d, (i * kCopyThreads + threadIdx.x) << 4);
}

bool probe_ok(const void *p, int64_t bytes) {
    return p && bytes > 0 && bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0 &&
           bytes / 4096 < 0x7fffffff;
}

uint32_t probe_grid(int64_t bytes, int64_t per_group) { return (uint32_t)((bytes + per_group - 1) / per_group); }

}  // namespace
}  // namespace moe

extern "C" {

int moe_probe_fill(void *dst, int64_t bytes, hipStream_t stream) {
    if (!moe::probe_ok(dst, bytes)) return MOE_ERR_ARG;
    const uint32_t grid = moe::probe_grid(bytes, moe::kFillThreads * moe::kFillVecs * 16);
    hipLaunchKernelGGL(moe::probe_fill_kernel, dim3(grid), dim3(moe::kFillThreads), 0, stream,
                       static_cast<uint8_t *>(dst), bytes);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream) {
    if (!moe::probe_ok(src, bytes) || !sink) return MOE_ERR_ARG;
    const uint32_t grid = moe::probe_grid(bytes, moe::kReadThreads * moe::kReadVecs * 16);
    hipLaunchKernelGGL(moe::probe_read_kernel, dim3(grid), dim3(moe::kReadThreads), 0, stream,
                       static_cast<const uint8_t *>(src), bytes, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream) {
    if (!moe::probe_ok(src, bytes) || !moe::probe_ok(dst, bytes)) return MOE_ERR_ARG;
    const uint32_t grid = moe::probe_grid(bytes, moe::kCopyThreads * moe::kCopyVecs * 16);
    hipLaunchKernelGGL(moe::probe_copy_kernel, dim3(grid), dim3(moe::kCopyThreads), 0, stream,
                       static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), bytes);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
