// Dispatch pack kernels for gfx950: K-fold expanded copy of token rows into window slots, and the
// per-rank deduplicated copy.
//
// The CAM pack ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.6 InputToShare) walks the
// (token, k) pairs and re-reads the token row for every copy. Here each row is read from HBM once
// and stored K times; slot addresses come from the layout's slot_idx, so the pack is a pure scatter
// with no atomics.
//
// bf16: the row is split into parts of kPartThreads 16-byte vectors and each workgroup owns one
// (token, part): every lane loads one vector and stores it to the K slots. Small workgroups with
// one store per lane per slot keep the HBM write stream dense; measured on MI355X this writes
// markedly faster than one large workgroup per token storing many vectors per lane. Half-wave
// workgroups (512 bytes per slot each) were fastest when x has to come from HBM rather than from
// the memory-side cache (S=4096, H=7168, K=8: 100 us against 106 us for 128-lane workgroups, with
// the same time when x is cached); 16-lane workgroups were slower in both cases.
//
// fp8 / int8: the DynamicQuant branch of the same section (bf16 -> fp32 -> abs -> row max ->
// scale -> narrow; the page's narrow type is INT8, E4M3FN is the second format) needs the whole
// row's maximum before any code is known, so one workgroup owns one token: each lane holds 16
// elements (one 16-byte vector of codes), the row max is a wave shuffle reduction followed by an
// LDS reduction across waves, then codes are written to the K slots. The arithmetic (the correctly
// rounded quotient by a reciprocal and two FMA corrections, the hardware E4M3 convert) and the
// slot stores are in pack_rows.h, shared with the fused small-table layout + pack.
//
// The deduplicated variants (DeepEP's one copy per destination rank, "Ascend DeepEP MoE Dispatch
// Optimization", section "一条 token 如何走完 MoE") keep the same workgroup shapes and store each row
// once per destination rank instead of once per k.
//
// Stores use buffer instructions with the sc0 sc1 nt cache policy: the window is written once and
// not read back by this kernel, so the lines stream to HBM instead of filling L2 and the
// memory-side cache with dirty data that later kernels would have to evict. Buffer descriptors are
// built per slot with the slot's written size as their range, so an out-of-range offset is dropped
// by the hardware instead of touching a neighbour.

#include "pack_rows.h"

namespace moe {
namespace {

using namespace rows;

constexpr int kPartThreads = 32;  // bf16: lanes (= 16-byte vectors) per (token, part) workgroup
constexpr int kDedupThreads = 128;  // the same for the deduplicated bf16 pack

// grid = S * nparts; workgroup (t, q) copies vectors [q*kPartThreads, (q+1)*kPartThreads) of
// x[t] into the K slots of token t; the last part also writes the slot tails. (Loading the K slot
// indices up front and unrolling the K stores was measured slower here: 114 us against 101 us at
// S=4096, H=7168, K=8.)
__global__ __launch_bounds__(kPartThreads) void pack_bf16_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ slot_idx, int K, int nvec,
    int nparts, SlotGeom g, int src_rank, int64_t max_slots, uint8_t *__restrict__ window) {
    const int t = blockIdx.x / nparts;
    const int q = blockIdx.x - t * nparts;
    const int lane = threadIdx.x;
    const int v = q * kPartThreads + lane;
    const int row_bytes = nvec << 4;
    const __amdgpu_buffer_rsrc_t src = rsrc(x + (int64_t)t * row_bytes, row_bytes);
    const u32x4 r = load16(src, v << 4);  // out of range (v >= nvec) reads as zero, never stored
    const bool tail_lane = q == nparts - 1 && lane < ((g.tail_end - g.payload_bytes) >> 4);
    const int32_t *slots = slot_idx + (int64_t)t * K;
    for (int k = 0; k < K; ++k) {
        const int64_t s = slots[k];
        if (s < 0 || s >= max_slots) continue;
        const __amdgpu_buffer_rsrc_t dst = rsrc(window + s * g.slot_bytes, g.tail_end);
        if (v < nvec) store16(r, dst, v << 4);
        if (tail_lane) store_tail(dst, g, lane, 0u, src_rank, t, k);
    }
}

// Deduplicated bf16 pack: one row per (token, destination rank) instead of per (token, k)
// ("Ascend DeepEP MoE Dispatch Optimization", section "一条 token 如何走完 MoE": the row is copied once
// to every rank that holds one of the token's experts). rank_row_idx[t, k] names the row of the
// rank of expert k (equal for every k of the token on that rank), so only the first k with a given
// row stores. Row format as the K-fold slot, with the triple (src_rank, t, destination rank).
// grid = S * nparts; workgroup (t, q) copies vectors [q*kDedupThreads, (q+1)*kDedupThreads) of
// x[t]. The row part is loaded first, then the token's K rows (and, for the tail lanes, its K ids)
// into registers: KMAX >= K. Measured at S=4096, H=7168, P=8 (5.3 rows per token) with x cold: 66
// us with 128-lane parts against 95 us with 32-lane parts loading the indices first (68 and 72 us
// for 64 and 256 lanes); 59 against 68 us with x cached. At P=128 (7.9 rows per token) 169 against
// 228 us cold, 154 against 145 us cached.
template <int KMAX>
__global__ __launch_bounds__(kDedupThreads) void pack_dedup_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ rank_row_idx,
    const int32_t *__restrict__ topk, int K, int E, int epr, int nvec, int nparts, SlotGeom g,
    int src_rank, int64_t max_rows, uint8_t *__restrict__ window) {
    const int t = blockIdx.x / nparts;
    const int q = blockIdx.x - t * nparts;
    const int lane = threadIdx.x;
    const int v = q * kDedupThreads + lane;
    const int row_bytes = nvec << 4;
    const u32x4 r = load16(rsrc(x + (int64_t)t * row_bytes, row_bytes), v << 4);
    int64_t j[KMAX];
    int e[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        j[k] = k < K ? rank_row_idx[(int64_t)t * K + k] : -1;
        e[k] = k < K ? topk[(int64_t)t * K + k] : -1;
    }
    const bool tail_lane = q == nparts - 1 && lane < ((g.tail_end - g.payload_bytes) >> 4);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        bool store = j[k] >= 0 && j[k] < max_rows;
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2) store = store && j[k2] != j[k];  // first k of this rank
        if (store) {
            const __amdgpu_buffer_rsrc_t dst = rsrc(window + j[k] * g.slot_bytes, g.tail_end);
            if (v < nvec) store16(r, dst, v << 4);
            if (tail_lane)
                store_tail(dst, g, lane, 0u, src_rank, t, (e[k] >= 0 && e[k] < E) ? e[k] / epr : -1);
        }
    }
}

// grid = S; workgroup t quantises x[t] and writes the codes to its K slots. blockDim.x = ngroups
// rounded up to whole waves (at most 1024): on MI355X a workgroup with no idle wave is about 3%
// faster than a fixed 512 lanes.
template <int QUANT>
__global__ __launch_bounds__(1024) void pack_quant_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ slot_idx, int K, int ngroups,
    SlotGeom g, int src_rank, int64_t max_slots, uint8_t *__restrict__ window) {
    __shared__ float wave_max[16];
    const int t = blockIdx.x;
    const int u = threadIdx.x;
    u32x4 codes;
    uint32_t scale_bits;
    quantise_row<QUANT>(x, t, ngroups, wave_max, codes, scale_bits);
    const bool tail_lane = u < ((g.tail_end - g.payload_bytes) >> 4);
    const int32_t *slots = slot_idx + (int64_t)t * K;
    for (int k = 0; k < K; ++k) {
        const int64_t s = slots[k];
        if (s < 0 || s >= max_slots) continue;
        const __amdgpu_buffer_rsrc_t dst = rsrc(window + s * g.slot_bytes, g.tail_end);
        if (u < ngroups) store16(codes, dst, u << 4);
        if (tail_lane) store_tail(dst, g, u, scale_bits, src_rank, t, k);
    }
}

// Deduplicated quantised pack: the codes of row t go once to each destination rank's row (the
// first k of each rank in rank_row_idx), with the scale and the triple (src_rank, t, rank).
template <int KMAX, int QUANT>
__global__ __launch_bounds__(1024) void pack_dedup_quant_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ rank_row_idx,
    const int32_t *__restrict__ topk, int K, int E, int epr, int ngroups, SlotGeom g, int src_rank,
    int64_t max_rows, uint8_t *__restrict__ window) {
    __shared__ float wave_max[16];
    const int t = blockIdx.x;
    const int u = threadIdx.x;
    int64_t j[KMAX];
    int e[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        j[k] = k < K ? rank_row_idx[(int64_t)t * K + k] : -1;
        e[k] = k < K ? topk[(int64_t)t * K + k] : -1;
    }
    u32x4 codes;
    uint32_t scale_bits;
    quantise_row<QUANT>(x, t, ngroups, wave_max, codes, scale_bits);
    const bool tail_lane = u < ((g.tail_end - g.payload_bytes) >> 4);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        bool store = j[k] >= 0 && j[k] < max_rows;
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2) store = store && j[k2] != j[k];  // first k of this rank
        if (store) {
            const __amdgpu_buffer_rsrc_t dst = rsrc(window + j[k] * g.slot_bytes, g.tail_end);
            if (u < ngroups) store16(codes, dst, u << 4);
            if (tail_lane)
                store_tail(dst, g, u, scale_bits, src_rank, t,
                           (e[k] >= 0 && e[k] < E) ? e[k] / epr : -1);
        }
    }
}

template <int QUANT>
hipError_t launch_quant(const uint8_t *x, const int32_t *slot_idx, int S, int K, int ngroups,
                        const SlotGeom &g, int src_rank, int64_t max_slots, uint8_t *window,
                        hipStream_t stream) {
    const int threads = (ngroups + 63) & ~63;
    hipLaunchKernelGGL((pack_quant_kernel<QUANT>), dim3(S), dim3(threads), 0, stream, x, slot_idx,
                       K, ngroups, g, src_rank, max_slots, window);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                       int32_t quant, int32_t src_rank, void *window, hipStream_t stream) {
    const SlotGeom g = slot_geom(H, quant);
    const int64_t max_slots = (int64_t)S * K;
    const uint8_t *xb = static_cast<const uint8_t *>(x);
    uint8_t *wb = static_cast<uint8_t *>(window);
    if (quant == MOE_QUANT_NONE) {
        const int nvec = H / 8;  // 16-byte vectors per bf16 row
        const int nparts = (nvec + kPartThreads - 1) / kPartThreads;
        hipLaunchKernelGGL(pack_bf16_kernel, dim3((uint32_t)S * nparts), dim3(kPartThreads), 0,
                           stream, xb, slot_idx, K, nvec, nparts, g, src_rank, max_slots, wb);
        return hipGetLastError();
    }
    const int ngroups = H / 16;  // 16 elements -> one 16-byte vector of codes
    if (quant == MOE_QUANT_FP8_E4M3_DYN)
        return launch_quant<MOE_QUANT_FP8_E4M3_DYN>(xb, slot_idx, S, K, ngroups, g, src_rank,
                                                    max_slots, wb, stream);
    return launch_quant<MOE_QUANT_INT8_DYN>(xb, slot_idx, S, K, ngroups, g, src_rank, max_slots,
                                            wb, stream);
}

template <int KMAX>
hipError_t launch_dedup_k(const void *x, const int32_t *rank_row_idx, const int32_t *topk_idx,
                          int32_t S, int32_t H, int32_t K, int32_t E, int32_t P, int32_t quant,
                          int32_t src_rank, void *window, hipStream_t stream) {
    const SlotGeom g = slot_geom(H, quant);
    const int64_t max_rows = (int64_t)S * (K < P ? K : P);
    const uint8_t *xb = static_cast<const uint8_t *>(x);
    uint8_t *wb = static_cast<uint8_t *>(window);
    if (quant == MOE_QUANT_NONE) {
        const int nvec = H / 8;
        const int nparts = (nvec + kDedupThreads - 1) / kDedupThreads;
        hipLaunchKernelGGL((pack_dedup_kernel<KMAX>), dim3((uint32_t)S * nparts), dim3(kDedupThreads),
                           0, stream, xb, rank_row_idx, topk_idx, K, E, E / P, nvec, nparts, g,
                           src_rank, max_rows, wb);
        return hipGetLastError();
    }
    const int ngroups = H / 16;
    const int threads = (ngroups + 63) & ~63;
    if (quant == MOE_QUANT_FP8_E4M3_DYN)
        hipLaunchKernelGGL((pack_dedup_quant_kernel<KMAX, MOE_QUANT_FP8_E4M3_DYN>), dim3(S),
                           dim3(threads), 0, stream, xb, rank_row_idx, topk_idx, K, E, E / P, ngroups,
                           g, src_rank, max_rows, wb);
    else
        hipLaunchKernelGGL((pack_dedup_quant_kernel<KMAX, MOE_QUANT_INT8_DYN>), dim3(S),
                           dim3(threads), 0, stream, xb, rank_row_idx, topk_idx, K, E, E / P, ngroups,
                           g, src_rank, max_rows, wb);
    return hipGetLastError();
}

hipError_t launch_pack_dedup(const void *x, const int32_t *rank_row_idx, const int32_t *topk_idx,
                             int32_t S, int32_t H, int32_t K, int32_t E, int32_t P, int32_t quant,
                             int32_t src_rank, void *window, hipStream_t stream) {
    if (K <= 2) return launch_dedup_k<2>(x, rank_row_idx, topk_idx, S, H, K, E, P, quant, src_rank, window, stream);
    if (K <= 4) return launch_dedup_k<4>(x, rank_row_idx, topk_idx, S, H, K, E, P, quant, src_rank, window, stream);
    if (K <= 8) return launch_dedup_k<8>(x, rank_row_idx, topk_idx, S, H, K, E, P, quant, src_rank, window, stream);
    return launch_dedup_k<16>(x, rank_row_idx, topk_idx, S, H, K, E, P, quant, src_rank, window, stream);
}

}  // namespace moe
