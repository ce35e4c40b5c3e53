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
// LDS reduction across waves, then codes are written to the K slots.
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

#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPartThreads = 32;    // bf16: lanes (= 16-byte vectors) per (token, part) workgroup
constexpr int kPolicyDefault = 0;
constexpr int kPolicyStream = 1 | 16 | 2;  // sc0 sc1 nt

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *base, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, int32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolicyDefault);
}

__device__ inline void store16(u32x4 v, __amdgpu_buffer_rsrc_t r, int32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kPolicyStream);
}

// Tail of one slot, lane `lane` < ntail: 16-byte vectors from payload_bytes to tail_end, all zero
// except the scale vector (fp32 scale in its first word) and the triple vector (src_rank, t, k, 0).
__device__ inline void store_tail(__amdgpu_buffer_rsrc_t slot, const SlotGeom &g, int lane,
                                  uint32_t scale_bits, int src_rank, int t, int k) {
    const int off = g.payload_bytes + (lane << 4);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (off == g.scale_off) v.x = scale_bits;
    if (off == g.triple_off) v = u32x4{(uint32_t)src_rank, (uint32_t)t, (uint32_t)k, 0u};
    store16(v, slot, off);
}

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
// grid = S * nparts; workgroup (t, q) as in pack_bf16_kernel. The token's K rows (and, for the
// tail lanes, its K ids) are loaded up front into registers: KMAX >= K.
template <int KMAX>
__global__ __launch_bounds__(kPartThreads) void pack_dedup_kernel(
    const uint8_t *__restrict__ x, const int32_t *__restrict__ rank_row_idx,
    const int32_t *__restrict__ topk, int K, int E, int epr, int nvec, int nparts, SlotGeom g,
    int src_rank, int64_t max_rows, uint8_t *__restrict__ window) {
    const int t = blockIdx.x / nparts;
    const int q = blockIdx.x - t * nparts;
    const int lane = threadIdx.x;
    const int v = q * kPartThreads + lane;
    const int row_bytes = nvec << 4;
    int64_t j[KMAX];
    int e[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        j[k] = k < K ? rank_row_idx[(int64_t)t * K + k] : -1;
        e[k] = k < K ? topk[(int64_t)t * K + k] : -1;
    }
    const u32x4 r = load16(rsrc(x + (int64_t)t * row_bytes, row_bytes), v << 4);
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

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> INT8 code (two's complement byte): round half to even, clamp to [-127, 127].
__device__ inline uint32_t int8_code(float q) {
    const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(q), -127.0f, 127.0f);
    return (uint32_t)((int32_t)r) & 0xFFu;
}

// Largest code magnitude: the row's amax maps onto it.
template <int QUANT>
constexpr float code_max() { return QUANT == MOE_QUANT_FP8_E4M3_DYN ? 448.0f : 127.0f; }

// Smallest scale the reciprocal division below handles; rows with a smaller (or a non-finite)
// scale divide with the IEEE division itself.
constexpr float kFastDivMinScale = 0x1p-90f;

// RN(x / scale) for scale in [2^-90, FLT_MAX], with y = RN(1 / scale): two FMA corrections of
// q = x * y (Markstein's correction step; the first brings q within one ulp of x / scale, the
// second rounds it correctly because y is the correctly rounded reciprocal). The exact remainder
// needs |x| above 2^-103, which every quotient that can change a code has (|x / scale| >= 2^-11
// with scale >= 2^-90); copysign keeps the sign of a zero x, which the corrections would turn
// into +0. Compared on MI355X with the IEEE division for every finite bf16 x and 90,600 scales
// (random, power-of-two neighbours, and every amax / 448 and amax / 127 of a bf16 amax): the
// quotients agree for every |x / scale| in [2^-11, 449], and the codes for every x.
__device__ inline float div_by_scale(float x, float scale, float y) {
    const float q0 = x * y;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, scale, x), y, q0);
    const float q2 = __builtin_fmaf(__builtin_fmaf(-q1, scale, x), y, q1);
    return __builtin_copysignf(q2, x);
}

template <bool FAST>
__device__ inline float quotient(float x, float scale, float y) {
    if constexpr (FAST) return div_by_scale(x, scale, y);
    else return x / scale;  // IEEE round-to-nearest division
}

// Four bf16 pairs (two input words) -> four codes in one word, element order kept. E4M3FN codes
// come from gfx950's packed fp8 convert (round to nearest even) after a clamp to +-448, which
// gives the saturating form; the pair compared equal to a bit-level RNE encoder on MI355X for
// every finite fp32 input of either sign.
template <int QUANT, bool FAST>
__device__ inline uint32_t quant4(uint32_t w0, uint32_t w1, float scale, float y) {
    const float q0 = quotient<FAST>(bf16_lo(w0), scale, y), q1 = quotient<FAST>(bf16_hi(w0), scale, y);
    const float q2 = quotient<FAST>(bf16_lo(w1), scale, y), q3 = quotient<FAST>(bf16_hi(w1), scale, y);
    if constexpr (QUANT == MOE_QUANT_FP8_E4M3_DYN) {
        const float lim = code_max<QUANT>();
        int packed = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q0, -lim, lim),
                                                     __builtin_amdgcn_fmed3f(q1, -lim, lim), 0, false);
        packed = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q2, -lim, lim),
                                                 __builtin_amdgcn_fmed3f(q3, -lim, lim), packed, true);
        return (uint32_t)packed;
    } else {
        return int8_code(q0) | (int8_code(q1) << 8) | (int8_code(q2) << 16) | (int8_code(q3) << 24);
    }
}

template <int QUANT, bool FAST>
__device__ inline u32x4 quant16(const u32x4 &a, const u32x4 &b, float scale, float y) {
    return u32x4{quant4<QUANT, FAST>(a[0], a[1], scale, y), quant4<QUANT, FAST>(a[2], a[3], scale, y),
                 quant4<QUANT, FAST>(b[0], b[1], scale, y), quant4<QUANT, FAST>(b[2], b[3], scale, y)};
}

// Quantises row t of x in one workgroup (blockDim.x >= ngroups, whole waves): lane u gets the 16
// codes of elements [16u, 16u + 16) (zero past the row) and every lane the row's fp32 scale. The
// row max is a wave shuffle reduction followed by an LDS reduction across waves (wave_max holds
// one value per wave); scale = amax / top by IEEE division, and every code from the correctly
// rounded quotient x / scale (div_by_scale, or the IEEE division for extreme scales).
template <int QUANT>
__device__ inline void quantise_row(const uint8_t *__restrict__ x, int t, int ngroups,
                                    float *wave_max, u32x4 &codes, uint32_t &scale_bits) {
    const int u = threadIdx.x, lane = u & 63, wave = u >> 6;
    const int row_bytes = ngroups << 5;
    const __amdgpu_buffer_rsrc_t src = rsrc(x + (int64_t)t * row_bytes, row_bytes);
    const u32x4 a = load16(src, u << 5);        // elements 16u .. 16u+7 (zero past the row)
    const u32x4 b = load16(src, (u << 5) + 16);  // elements 16u+8 .. 16u+15
    float amax = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(a[w])), fabsf(bf16_hi(a[w]))));
        amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(b[w])), fabsf(bf16_hi(b[w]))));
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    if (lane == 0) wave_max[wave] = amax;
    __syncthreads();
    const int nwaves = blockDim.x >> 6;
    for (int w = 0; w < nwaves; ++w) amax = fmaxf(amax, wave_max[w]);

    const float scale = amax / code_max<QUANT>();  // IEEE round-to-nearest division
    codes = u32x4{0u, 0u, 0u, 0u};
    if (u < ngroups && amax > 0.0f) {
        if (scale >= kFastDivMinScale && scale <= 0x1.fffffep127f)  // the same for the whole row
            codes = quant16<QUANT, true>(a, b, scale, 1.0f / scale);
        else
            codes = quant16<QUANT, false>(a, b, scale, 0.0f);
    }
    scale_bits = __float_as_uint(scale);
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
        const int nparts = (nvec + kPartThreads - 1) / kPartThreads;
        hipLaunchKernelGGL((pack_dedup_kernel<KMAX>), dim3((uint32_t)S * nparts), dim3(kPartThreads),
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
