// Unpack kernel for gfx950: window slots -> compact expert input rows, triples and scales.
//
// The CAM receive side ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.9 ShareToOutput)
// copies every received slot's token data to the next row of expandXOut and its triple to
// expandIdxOut, in (local expert, source rank) order. On one GPU the window is already in
// expert-major, source-token order, so compact row s is slot s with its padding and tail stripped:
// the result is the contiguous per-expert input of a grouped GEMM.
//
// The number of used slots N is read on the device (for example expert_slot_base[E] written by the
// layout), so no count is read back to the host; the grid covers the worst case S*K and workgroups
// past N exit at once. Like the bf16 pack, each workgroup owns one (slot, part) of kPartThreads
// 16-byte vectors: one non-temporal load (the slot is read once) and one streaming store per lane.

#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPartThreads = 128;
constexpr int kLoadPolicy = 2;             // nt
constexpr int kStorePolicy = 1 | 16 | 2;   // sc0 sc1 nt

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// grid = max_slots * nparts; workgroup (s, q) copies vectors [q*kPartThreads, (q+1)*kPartThreads)
// of slot s's payload to row s; lane 0 of the last part also moves the triple and the scale.
__global__ __launch_bounds__(kPartThreads) void unpack_kernel(
    const uint8_t *__restrict__ window, const int32_t *__restrict__ num_slots, int max_slots,
    int nparts, SlotGeom g, bool quantised, uint8_t *__restrict__ expand_x,
    float *__restrict__ expand_scales, int32_t *__restrict__ expand_idx) {
    const int s = blockIdx.x / nparts;
    const int q = blockIdx.x - s * nparts;
    const int lane = threadIdx.x;
    const int v = q * kPartThreads + lane;
    const __amdgpu_buffer_rsrc_t src = rsrc(window + (int64_t)s * g.slot_bytes, g.tail_end);
    // the load is issued before N arrives: slot s < max_slots always lies inside the window
    const bool in_row = (v << 4) < g.payload_bytes;
    const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(src, in_row ? v << 4 : 0, 0, kLoadPolicy);
    const int n = min(*num_slots, max_slots);
    if (s >= n) return;
    if (in_row) {
        const __amdgpu_buffer_rsrc_t dst =
            rsrc(expand_x + (int64_t)s * g.payload_bytes, g.payload_bytes);
        __builtin_amdgcn_raw_buffer_store_b128(d, dst, v << 4, 0, kStorePolicy);
    }
    if (q == nparts - 1 && lane == 0) {
        const u32x4 tr = __builtin_amdgcn_raw_buffer_load_b128(src, g.triple_off, 0, kLoadPolicy);
        int32_t *idx = expand_idx + (int64_t)s * 3;
        idx[0] = (int32_t)tr.x;
        idx[1] = (int32_t)tr.y;
        idx[2] = (int32_t)tr.z;
        if (quantised)
            expand_scales[s] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(src, g.scale_off, 0, kLoadPolicy));
    }
}

}  // namespace

hipError_t launch_unpack(const void *window, const int32_t *num_slots, int32_t S, int32_t K,
                         int32_t H, int32_t quant, void *expand_x, float *expand_scales,
                         int32_t *expand_idx, hipStream_t stream) {
    const SlotGeom g = slot_geom(H, quant);
    const int max_slots = S * K;
    const int nvec = g.payload_bytes / 16;
    const int nparts = (nvec + kPartThreads - 1) / kPartThreads;
    hipLaunchKernelGGL(unpack_kernel, dim3((uint32_t)max_slots * nparts), dim3(kPartThreads), 0,
                       stream, static_cast<const uint8_t *>(window), num_slots, max_slots, nparts,
                       g, quant != MOE_QUANT_NONE, static_cast<uint8_t *>(expand_x), expand_scales,
                       expand_idx);
    return hipGetLastError();
}

}  // namespace moe
