// Device helpers shared by the pack kernels and the fused small-table layout + pack: buffer
// descriptors and streaming stores for window slots, the slot tail, and the per-token dynamic
// quantisation of one bf16 row ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.6, the
// DynamicQuant branch of InputToShare).
#pragma once

#include "moe_internal.h"

namespace moe {
namespace rows {


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Four fp32 values -> four E4M3FN codes in one word (element order kept): gfx950's packed fp8
// convert (round to nearest even) after a clamp to +-448, which gives the saturating form. It
// equals a bit-level RNE encoder for every finite fp32 input of either sign (tests/c_abi/quant_gpu.cpp
// checks every non-negative finite input against the oracle's code boundaries).
__device__ inline uint32_t e4m3fn_pack4(float q0, float q1, float q2, float q3) {
    constexpr float lim = 448.0f;
    int packed = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q0, -lim, lim),
                                                 __builtin_amdgcn_fmed3f(q1, -lim, lim), 0, false);
    packed = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q2, -lim, lim),
                                             __builtin_amdgcn_fmed3f(q3, -lim, lim), packed, true);
    return (uint32_t)packed;
}

// Four bf16 pairs (two input words) -> four codes in one word, element order kept.
template <int QUANT, bool FAST>
__device__ inline uint32_t quant4(uint32_t w0, uint32_t w1, float scale, float y) {
    const float q0 = quotient<FAST>(bf16_lo(w0), scale, y), q1 = quotient<FAST>(bf16_hi(w0), scale, y);
    const float q2 = quotient<FAST>(bf16_lo(w1), scale, y), q3 = quotient<FAST>(bf16_hi(w1), scale, y);
    if constexpr (QUANT == MOE_QUANT_FP8_E4M3_DYN)
        return e4m3fn_pack4(q0, q1, q2, q3);
    else
        return int8_code(q0) | (int8_code(q1) << 8) | (int8_code(q2) << 16) | (int8_code(q3) << 24);
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

}  // namespace rows
}  // namespace moe
