// Dispatch pack kernels for gfx950: K-fold expanded copy of token rows into window slots.
//
// The CAM pack ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.6 InputToShare) walks the
// (token, k) pairs and re-reads the token row for every copy. Here one workgroup owns one token:
// the row is read from HBM once into registers (16-byte loads, consecutive lanes on consecutive
// 16-byte vectors) and stored K times with 16-byte non-temporal stores, since the window is written
// once and not read back by this kernel. Slot addresses come from the layout's slot_idx, so the
// kernel is a pure scatter with no atomics. Each store stream covers whole 128-byte lines: the slot
// pitch is a multiple of 512 bytes and the written region ends on a 128-byte boundary.
//
// fp8 variant: the DynamicQuant branch of the same section (bf16 -> fp32 -> abs -> row max ->
// scale -> narrow), with E4M3FN codes and scale = amax / 448. The row max is a wave shuffle
// reduction followed by an LDS reduction across the workgroup's waves.

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline void store_stream(void *p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// Writes the tail of one slot: 16-byte vectors from payload_bytes to tail_end, all zero except
// the scale vector (fp32 scale in its first word) and the triple vector (src_rank, t, k, 0).
__device__ inline void store_tail(uint8_t *slot, const SlotGeom &g, int tid, uint32_t scale_bits,
                                  int src_rank, int t, int k) {
    const int ntail = (g.tail_end - g.payload_bytes) >> 4;
    if (tid < ntail) {
        const int off = g.payload_bytes + (tid << 4);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (off == g.scale_off) v.x = scale_bits;
        if (off == g.triple_off) v = u32x4{(uint32_t)src_rank, (uint32_t)t, (uint32_t)k, 0u};
        store_stream(slot + off, v);
    }
}

// grid = S workgroups; workgroup t copies x[t] (nvec 16-byte vectors) into its K slots.
template <int MAXV>
__global__ __launch_bounds__(kThreads) void pack_bf16_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ slot_idx, int K, int nvec,
    SlotGeom g, int src_rank, int64_t max_slots, uint8_t *__restrict__ window) {
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const u32x4 *src = x + (int64_t)t * nvec;
    u32x4 row[MAXV];
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
        const int v = tid + j * kThreads;
        if (v < nvec) row[j] = src[v];
    }
    const int32_t *slots = slot_idx + (int64_t)t * K;
    for (int k = 0; k < K; ++k) {
        const int64_t s = slots[k];
        if (s < 0 || s >= max_slots) continue;
        uint8_t *slot = window + s * g.slot_bytes;
#pragma unroll
        for (int j = 0; j < MAXV; ++j) {
            const int v = tid + j * kThreads;
            if (v < nvec) store_stream(slot + ((int64_t)v << 4), row[j]);
        }
        store_tail(slot, g, tid, 0u, src_rank, t, k);
    }
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> OCP E4M3FN code, round to nearest even, saturating to +-448. q must not be NaN.
__device__ inline uint32_t e4m3fn_code(float q) {
    const uint32_t u = __float_as_uint(q);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x43E00000u) {  // |q| >= 448: largest finite code
        code = 0x7Eu;
    } else if (a < 0x3C800000u) {  // |q| < 2^-6: subnormal spacing 2^-9
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scale, RNE
    } else {
        // keep 3 mantissa bits: add just under half an ulp plus the kept lsb, then truncate;
        // a carry into the exponent is the correct round-up to the next binade
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        code = r - (120u << 3);  // rebias exponent 127 -> 7 in the 4.3 layout
    }
    return code | sign;
}

// grid = S workgroups. Thread owns 16-element groups u = tid + j*kThreads (two 16-byte input
// vectors each), producing one 16-byte output vector of codes per group.
template <int MAXU>
__global__ __launch_bounds__(kThreads) void pack_fp8_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ slot_idx, int K, int ngroups,
    SlotGeom g, int src_rank, int64_t max_slots, uint8_t *__restrict__ window) {
    __shared__ float wave_max[kWaves];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const u32x4 *src = x + (int64_t)t * ngroups * 2;
    u32x4 in0[MAXU], in1[MAXU];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXU; ++j) {
        const int u = tid + j * kThreads;
        if (u < ngroups) {
            in0[j] = src[2 * u];
            in1[j] = src[2 * u + 1];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                amax = fmaxf(amax, fabsf(bf16_lo(in0[j][w])));
                amax = fmaxf(amax, fabsf(bf16_hi(in0[j][w])));
                amax = fmaxf(amax, fabsf(bf16_lo(in1[j][w])));
                amax = fmaxf(amax, fabsf(bf16_hi(in1[j][w])));
            }
        }
    }
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    if (lane == 0) wave_max[wave] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, wave_max[w]);

    const float scale = amax / 448.0f;  // IEEE round-to-nearest division
    u32x4 codes[MAXU];
#pragma unroll
    for (int j = 0; j < MAXU; ++j) {
        codes[j] = u32x4{0u, 0u, 0u, 0u};
        const int u = tid + j * kThreads;
        if (u < ngroups && amax > 0.0f) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t src_w = w < 2 ? in0[j][2 * w] : in1[j][2 * (w - 2)];
                const uint32_t src_w2 = w < 2 ? in0[j][2 * w + 1] : in1[j][2 * (w - 2) + 1];
                const uint32_t c0 = e4m3fn_code(bf16_lo(src_w) / scale);
                const uint32_t c1 = e4m3fn_code(bf16_hi(src_w) / scale);
                const uint32_t c2 = e4m3fn_code(bf16_lo(src_w2) / scale);
                const uint32_t c3 = e4m3fn_code(bf16_hi(src_w2) / scale);
                codes[j][w] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
            }
        }
    }
    const uint32_t scale_bits = __float_as_uint(scale);
    const int32_t *slots = slot_idx + (int64_t)t * K;
    for (int k = 0; k < K; ++k) {
        const int64_t s = slots[k];
        if (s < 0 || s >= max_slots) continue;
        uint8_t *slot = window + s * g.slot_bytes;
#pragma unroll
        for (int j = 0; j < MAXU; ++j) {
            const int u = tid + j * kThreads;
            if (u < ngroups) store_stream(slot + ((int64_t)u << 4), codes[j]);
        }
        store_tail(slot, g, tid, scale_bits, src_rank, t, k);
    }
}

template <int MAXV>
hipError_t launch_bf16(const void *x, const int32_t *slot_idx, int S, int K, int nvec,
                       const SlotGeom &g, int src_rank, int64_t max_slots, void *window,
                       hipStream_t stream) {
    hipLaunchKernelGGL(pack_bf16_kernel<MAXV>, dim3(S), dim3(kThreads), 0, stream,
                       static_cast<const u32x4 *>(x), slot_idx, K, nvec, g, src_rank, max_slots,
                       static_cast<uint8_t *>(window));
    return hipGetLastError();
}

template <int MAXU>
hipError_t launch_fp8(const void *x, const int32_t *slot_idx, int S, int K, int ngroups,
                      const SlotGeom &g, int src_rank, int64_t max_slots, void *window,
                      hipStream_t stream) {
    hipLaunchKernelGGL(pack_fp8_kernel<MAXU>, dim3(S), dim3(kThreads), 0, stream,
                       static_cast<const u32x4 *>(x), slot_idx, K, ngroups, g, src_rank,
                       max_slots, static_cast<uint8_t *>(window));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                       int32_t quant, int32_t src_rank, void *window, hipStream_t stream) {
    const SlotGeom g = slot_geom(H, quant);
    const int64_t max_slots = (int64_t)S * K;
    if (quant == MOE_QUANT_NONE) {
        const int nvec = H / 8;  // 16-byte vectors of bf16
        const int per = (nvec + kThreads - 1) / kThreads;
        if (per <= 1) return launch_bf16<1>(x, slot_idx, S, K, nvec, g, src_rank, max_slots, window, stream);
        if (per <= 2) return launch_bf16<2>(x, slot_idx, S, K, nvec, g, src_rank, max_slots, window, stream);
        if (per <= 4) return launch_bf16<4>(x, slot_idx, S, K, nvec, g, src_rank, max_slots, window, stream);
        return launch_bf16<8>(x, slot_idx, S, K, nvec, g, src_rank, max_slots, window, stream);
    }
    const int ngroups = H / 16;  // 16 elements -> one 16-byte vector of codes
    const int per = (ngroups + kThreads - 1) / kThreads;
    if (per <= 1) return launch_fp8<1>(x, slot_idx, S, K, ngroups, g, src_rank, max_slots, window, stream);
    if (per <= 2) return launch_fp8<2>(x, slot_idx, S, K, ngroups, g, src_rank, max_slots, window, stream);
    return launch_fp8<4>(x, slot_idx, S, K, ngroups, g, src_rank, max_slots, window, stream);
}

}  // namespace moe
