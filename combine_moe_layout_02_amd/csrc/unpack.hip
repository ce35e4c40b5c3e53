// Unpack kernels for gfx950: window slots -> compact expert input rows, triples and scales, and a
// padded form with expert_alignment-rounded row blocks and a fixed number of output rows.
//
// The CAM receive side ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.9 ShareToOutput)
// copies every received slot's token data to the next row of expandXOut and its triple to
// expandIdxOut, in (local expert, source rank) order. On one GPU the window is already in
// expert-major, source-token order, so compact row s is slot s with its padding and tail stripped:
// the result is the contiguous per-expert input of a grouped GEMM.
//
// The number of used slots N is read on the device (for example expert_slot_base[E] written by the
// layout), so no count is read back to the host; the grid covers the worst case S*K and workgroups
// past N exit at once. Each workgroup owns one (slot, part) of V 16-byte vectors per lane: V
// non-temporal loads (the slot is read once) and V streaming stores per lane. One-wave parts were
// fastest on MI355X at H=7168 (bf16: 146 us against 148 us for 128 lanes; fp8 codes, whose 448
// vectors split evenly into 64-lane parts but not 128-lane ones: 76 us against 94 us).
//
// The padded form follows two options of DeepEP's normal dispatch: expert_alignment, which rounds
// every per-expert row count up to a multiple of the alignment ("internode.cu", section 1
// notify_dispatch), and num_worst_tokens, a fixed output length that needs no count read back on
// the host, with zero data and -1 indices in the rows past the real ones ("Ascend DeepEP MoE
// Dispatch Optimization", section "输出长度有动态和固定两种模式"). Expert e's rows start at the
// aligned offset row_base[e], so every expert's block of a grouped GEMM starts on a tile boundary.

#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPartThreads = 64;
// 16-byte vectors per lane, by kernel (a part is V KB). Measured at S=4096, H=7168 bf16 (fp8):
// the plain unpack takes 151 (82) us with one vector per lane against 155 (90) us with two; the
// padded unpack, whose workgroups first look up their row's expert, 172 (98) us with two against
// 182 (103) us with one and 182 (102) us with four.
constexpr int kVecsUnpack = 1;
constexpr int kVecsPadded = 2;
constexpr int kVecsExpand = 1;
constexpr int kLoadPolicy = 2;             // nt
constexpr int kStorePolicy = 1 | 16 | 2;   // sc0 sc1 nt

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// grid = max_slots * nparts; workgroup (s, q) copies vectors [q*V*64, (q+1)*V*64) of slot s's
// payload to row s (vector (q*V + i)*64 + lane in lane's i-th load); lane 0 of the last part also
// moves the triple and the scale.
template <int V>
__global__ __launch_bounds__(kPartThreads) void unpack_kernel(
    const uint8_t *__restrict__ window, const int32_t *__restrict__ num_slots, int max_slots,
    int nparts, SlotGeom g, bool quantised, uint8_t *__restrict__ expand_x,
    float *__restrict__ expand_scales, int32_t *__restrict__ expand_idx) {
    const int s = blockIdx.x / nparts;
    const int q = blockIdx.x - s * nparts;
    const int lane = threadIdx.x;
    const __amdgpu_buffer_rsrc_t src = rsrc(window + (int64_t)s * g.slot_bytes, g.tail_end);
    // the loads are issued before N arrives: slot s < max_slots always lies inside the window
    u32x4 d[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int off = ((q * V + i) * kPartThreads + lane) << 4;
        d[i] = __builtin_amdgcn_raw_buffer_load_b128(src, off < g.payload_bytes ? off : 0, 0, kLoadPolicy);
    }
    const int n = min(*num_slots, max_slots);
    if (s >= n) return;
    const __amdgpu_buffer_rsrc_t dst = rsrc(expand_x + (int64_t)s * g.payload_bytes, g.payload_bytes);
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int off = ((q * V + i) * kPartThreads + lane) << 4;
        if (off < g.payload_bytes) __builtin_amdgcn_raw_buffer_store_b128(d[i], dst, off, 0, kStorePolicy);
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

constexpr int kBaseThreads = 512;  // >= MOE_MAX_EXPERTS: one expert per lane

// row_base[e] = sum over e' < e of ceil(count[e'] / A) * A with count[e] = esb[e+1] - esb[e]
// (the expert_alignment rounding of "internode.cu", section 1 notify_dispatch); row_base[E] is the
// aligned total, and status = 1 when it exceeds the out_rows rows of the output.
__global__ __launch_bounds__(kBaseThreads) void unpack_row_base_kernel(
    const int32_t *__restrict__ esb, int E, int A, int64_t out_rows, int32_t *__restrict__ row_base,
    int32_t *__restrict__ status) {
    __shared__ int32_t wave_sum[kBaseThreads / 64];
    const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
    int n = 0;
    if (e < E) {
        const int cnt = max(esb[e + 1] - esb[e], 0);
        n = (cnt + A - 1) / A * A;
    }
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d, 64);
        if (lane >= d) incl += u;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kBaseThreads / 64; ++w) {
        before += w < wave ? wave_sum[w] : 0;
        total += wave_sum[w];
    }
    if (e < E) row_base[e] = before + incl - n;
    if (e == 0) {
        row_base[E] = total;
        *status = (int64_t)total > out_rows ? 1 : 0;
    }
}

// grid = out_rows * nparts; workgroup (r, q) writes vectors [q*V*64, (q+1)*V*64) of output row
// r: the part of its source slot's payload, or zeros for a padding row. Lane 0 of
// the last part writes the triple and the scale (-1s and 0 for padding). The row's expert is
// found by a binary search over row_base (E + 1 values, uniform per workgroup).
template <int V>
__global__ __launch_bounds__(kPartThreads) void unpack_padded_kernel(
    const uint8_t *__restrict__ window, const int32_t *__restrict__ esb,
    const int32_t *__restrict__ row_base, int E, int64_t max_slots, int nparts, SlotGeom g,
    bool quantised, uint8_t *__restrict__ expand_x, float *__restrict__ expand_scales,
    int32_t *__restrict__ expand_idx) {
    const int64_t r = blockIdx.x / nparts;
    const int q = blockIdx.x - (int)(r * nparts);
    const int lane = threadIdx.x;
    int64_t s = -1;
    // The expert of output row r is the largest e < E with row_base[e] <= r. row_base is
    // non-decreasing, so that e is the number of such entries minus one: the wave loads its lanes'
    // share of the table in one round of independent loads and counts with ballots; the expert's
    // three values are then uniform scalar loads. Measured at S=4096, H=7168, A=16: 184 us, against
    // 188 us for a binary search (a chain of up to nine dependent scalar loads), 208 us for a
    // two-round vector lookup and 222 us with esb prefetched for every expert.
    const int total = row_base[E];
    int count = 0;
#pragma unroll
    for (int i = 0; i < (MOE_MAX_EXPERTS + kPartThreads - 1) / kPartThreads; ++i) {
        const int e = i * kPartThreads + lane;
        const int base = row_base[min(e, E)];  // row_base holds E + 1 entries
        count += __popcll(__ballot(e < E && base <= r));
    }
    if (r < total) {
        const int lo = count - 1;  // >= 0: row_base[0] = 0 <= r
        const int64_t j = r - row_base[lo];
        if (j < (int64_t)esb[lo + 1] - esb[lo]) s = esb[lo] + j;
        if (s >= max_slots) s = -1;  // a corrupt base table never reads past the window
    }
    u32x4 d[V];
    __amdgpu_buffer_rsrc_t src = rsrc(window, 0);
    if (s >= 0) src = rsrc(window + s * g.slot_bytes, g.tail_end);
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int off = ((q * V + i) * kPartThreads + lane) << 4;
        d[i] = u32x4{0u, 0u, 0u, 0u};
        if (s >= 0 && off < g.payload_bytes)
            d[i] = __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, kLoadPolicy);
    }
    const __amdgpu_buffer_rsrc_t dst = rsrc(expand_x + r * g.payload_bytes, g.payload_bytes);
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int off = ((q * V + i) * kPartThreads + lane) << 4;
        if (off < g.payload_bytes) __builtin_amdgcn_raw_buffer_store_b128(d[i], dst, off, 0, kStorePolicy);
    }
    if (q == nparts - 1 && lane == 0) {
        int32_t *idx = expand_idx + r * 3;
        float scale = 0.0f;
        if (s >= 0) {
            const u32x4 tr = __builtin_amdgcn_raw_buffer_load_b128(src, g.triple_off, 0, kLoadPolicy);
            idx[0] = (int32_t)tr.x;
            idx[1] = (int32_t)tr.y;
            idx[2] = (int32_t)tr.z;
            if (quantised)
                scale = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(src, g.scale_off, 0, kLoadPolicy));
        } else {
            idx[0] = -1;
            idx[1] = -1;
            idx[2] = -1;
        }
        if (quantised) expand_scales[r] = scale;
    }
}

// Receive-side expansion of the deduplicated rows ("Ascend DeepEP MoE Dispatch Optimization",
// section "一条 token 如何走完 MoE": the destination rank rearranges the rows it received into
// contiguous per-local-expert input). For every valid (t, k) the row rank_row_idx[t, k] (token t on
// the rank of expert k) goes to expert-major row slot_idx[t, k] with the triple (src_rank, t, k):
// the same output the K-fold window's unpack gives. Two launches, output-major so that the rows
// are written in order: expand_index_kernel writes (t, k) into fields 1-2 of expand_idx[s] for
// every valid entry; expand_rows_kernel (one workgroup per (output row, part)) then reads them,
// copies its part of row rank_row_idx[t, k] and fills field 0 with the row's source rank (and, for
// quantised rows, expand_scales[s] with the row's scale). An
// expert's rows list its tokens in ascending order, as does a rank's segment, so the reads sweep
// each segment in order.
__global__ __launch_bounds__(256) void expand_index_kernel(const int32_t *__restrict__ slot_idx,
                                                           int K, int64_t n_entries,
                                                           int64_t max_slots,
                                                           int32_t *__restrict__ expand_idx) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_entries) return;
    const int64_t s = slot_idx[i];
    if (s < 0 || s >= max_slots) return;
    expand_idx[s * 3 + 1] = (int32_t)(i / K);
    expand_idx[s * 3 + 2] = (int32_t)(i % K);
}

template <int V>
__global__ __launch_bounds__(kPartThreads) void expand_rows_kernel(
    const uint8_t *__restrict__ window, const int32_t *__restrict__ rank_row_idx,
    const int32_t *__restrict__ num_slots, int S, int K, int64_t max_rows, int64_t max_slots,
    int nparts, SlotGeom g, bool quantised, uint8_t *__restrict__ expand_x,
    float *__restrict__ expand_scales, int32_t *__restrict__ expand_idx) {
    const int64_t s = blockIdx.x / nparts;
    const int q = blockIdx.x - (int)(s * nparts);
    const int lane = threadIdx.x;
    const int64_t n = min((int64_t)*num_slots, max_slots);
    if (s >= n) return;
    const int t = expand_idx[s * 3 + 1], k = expand_idx[s * 3 + 2];
    if (t < 0 || t >= S || k < 0 || k >= K) return;
    const int64_t j = rank_row_idx[(int64_t)t * K + k];
    if (j < 0 || j >= max_rows) return;
    const __amdgpu_buffer_rsrc_t src = rsrc(window + j * g.slot_bytes, g.tail_end);
    u32x4 d[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int off = ((q * V + i) * kPartThreads + lane) << 4;
        d[i] = __builtin_amdgcn_raw_buffer_load_b128(src, off < g.payload_bytes ? off : 0, 0, kLoadPolicy);
    }
    const __amdgpu_buffer_rsrc_t dst = rsrc(expand_x + s * g.payload_bytes, g.payload_bytes);
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int off = ((q * V + i) * kPartThreads + lane) << 4;
        if (off < g.payload_bytes) __builtin_amdgcn_raw_buffer_store_b128(d[i], dst, off, 0, kStorePolicy);
    }
    if (q == nparts - 1 && lane == 0) {
        expand_idx[s * 3] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(src, g.triple_off, 0, kLoadPolicy);
        if (quantised)
            expand_scales[s] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(src, g.scale_off, 0, kLoadPolicy));
    }
}

}  // namespace

hipError_t launch_expand_dedup(const void *window, const int32_t *rank_row_idx,
                               const int32_t *slot_idx, const int32_t *num_slots, int32_t S,
                               int32_t K, int32_t P, int32_t H, int32_t quant, void *expand_x,
                               float *expand_scales, int32_t *expand_idx, hipStream_t stream) {
    const SlotGeom g = slot_geom(H, quant);
    const int64_t n_entries = (int64_t)S * K;
    hipLaunchKernelGGL(expand_index_kernel, dim3((uint32_t)((n_entries + 255) / 256)), dim3(256), 0,
                       stream, slot_idx, K, n_entries, n_entries, expand_idx);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int nvec = g.payload_bytes / 16;
    const int nparts = (nvec + kVecsExpand * kPartThreads - 1) / (kVecsExpand * kPartThreads);
    hipLaunchKernelGGL(expand_rows_kernel<kVecsExpand>, dim3((uint32_t)(n_entries * nparts)), dim3(kPartThreads),
                       0, stream, static_cast<const uint8_t *>(window), rank_row_idx, num_slots, S,
                       K, (int64_t)S * (K < P ? K : P), n_entries, nparts, g,
                       quant != MOE_QUANT_NONE, static_cast<uint8_t *>(expand_x), expand_scales,
                       expand_idx);
    return hipGetLastError();
}

hipError_t launch_unpack_padded(const void *window, const int32_t *expert_slot_base, int32_t E,
                                int32_t S, int32_t K, int32_t H, int32_t quant,
                                int32_t expert_alignment, int64_t out_rows, void *expand_x,
                                float *expand_scales, int32_t *expand_idx,
                                int32_t *expert_row_base, int32_t *status, hipStream_t stream) {
    const SlotGeom g = slot_geom(H, quant);
    hipLaunchKernelGGL(unpack_row_base_kernel, dim3(1), dim3(kBaseThreads), 0, stream,
                       expert_slot_base, E, expert_alignment, out_rows, expert_row_base, status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int nvec = g.payload_bytes / 16;
    const int nparts = (nvec + kVecsPadded * kPartThreads - 1) / (kVecsPadded * kPartThreads);
    hipLaunchKernelGGL(unpack_padded_kernel<kVecsPadded>, dim3((uint32_t)(out_rows * nparts)),
                       dim3(kPartThreads), 0, stream, static_cast<const uint8_t *>(window),
                       expert_slot_base, expert_row_base, E, (int64_t)S * K, nparts, g,
                       quant != MOE_QUANT_NONE, static_cast<uint8_t *>(expand_x), expand_scales,
                       expand_idx);
    return hipGetLastError();
}

hipError_t launch_unpack(const void *window, const int32_t *num_slots, int32_t S, int32_t K,
                         int32_t H, int32_t quant, void *expand_x, float *expand_scales,
                         int32_t *expand_idx, hipStream_t stream) {
    const SlotGeom g = slot_geom(H, quant);
    const int max_slots = S * K;
    const int nvec = g.payload_bytes / 16;
    const int nparts = (nvec + kVecsUnpack * kPartThreads - 1) / (kVecsUnpack * kPartThreads);
    hipLaunchKernelGGL(unpack_kernel<kVecsUnpack>, dim3((uint32_t)max_slots * nparts), dim3(kPartThreads), 0,
                       stream, static_cast<const uint8_t *>(window), num_slots, max_slots, nparts,
                       g, quant != MOE_QUANT_NONE, static_cast<uint8_t *>(expand_x), expand_scales,
                       expand_idx);
    return hipGetLastError();
}

}  // namespace moe
