// Single-launch routing layout for small routing tables (decode-sized batches) on gfx950.
//
// Computes exactly what the three-launch layout computes (the dispatch handle of "Ascend DeepEP MoE
// Dispatch Optimization", section "Dispatch handle 六项分别保存什么", plus the slot of every
// (token, k) following the per-expert offset + running count of "HCCL Window 模式 (Non-SHMEM)
// 代码深度剖析", section 3.6 InputToShare) in one launch. For a batch of a few hundred tokens the
// three launches are pure latency; here every workgroup reads the whole routing table (at most
// kSmallLayoutEntries ids, a few KB that stay in L2) and derives its share of the outputs on its
// own, so no workgroup waits for another. Workgroups take one of four roles by blockIdx.x:
//
//   slots    (workgroup 0) entries in (t, k) order, 1024 per batch: per-wave LDS lane masks +
//            popcount give each valid entry its rank among all earlier entries of its expert
//            (deterministic: atomics only build masks and counts); then an exclusive scan of the
//            per-expert totals gives the bases, slot = base[e] + rank, the count vectors and the
//            status word.
//   experts  16 rows of expert_prefix per workgroup, one per wave: the row's entries are binned by
//            channel in LDS, then an inclusive wave scan along the channels writes the row.
//   ranks    16 rows of rank_prefix per workgroup: a bitset over tokens per rank (OR is idempotent,
//            so a rank hit twice by one token counts once), word popcount prefixes, then
//            rank_prefix[r][c] = tokens of rank r below the end of channel c; the row total is
//            num_tokens_per_rank[r].
//   tokens   64 rows of is_token_in_rank per workgroup: the group's ids are loaded once (one per
//            lane) into LDS, then one wave per token sets byte r iff one of its K ids belongs to
//            rank r.
//
// Channel c ends at (c+1)*floor(S/C) + min(c+1, S mod C): the floor share plus one extra token for
// each of the first S mod C channels ("HCCL Window 模式", section 8.3 分片策略). The host picks this
// path only when layout_small_fits() holds, so every LDS table below is large enough.
//
// The fused layout + pack kernel adds a fifth role after the four above:
//
//   pack     one (token, part of the row) per work item. The slot of (t, k) is the number of valid
//            entries that come before it in (expert id, flat index t*K + k) order, which is the
//            slot order of the layout (expert-major, then source token, then k); each workgroup
//            holds the table as such sort keys in registers and counts with wave ballots. Then the
//            row, or its per-token quantisation, is stored to the K slots exactly as the pack
//            kernels store it. The layout workgroups write slot_idx from their own counts, so no
//            workgroup waits for another and the dispatch needs no second launch.

#include <atomic>

#include "pack_rows.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerGroup = kWaves;  // matrix rows per expert / rank workgroup
constexpr int kTokensPerGroup = 64;    // is_token_in_rank rows per token workgroup
constexpr int kMaxWords = (kSmallLayoutEntries + 63) / 64;  // bitset words per rank row (S <= N)

// LDS of each role, carved from one buffer.
// Entries per lane in the slots role: entry i belongs to lane i % kThreads, batch i / kThreads.
constexpr int kBatches = kSmallLayoutEntries / kThreads;
static_assert(kBatches * kThreads == kSmallLayoutEntries, "whole batches");

struct SlotLds {
    unsigned long long lane_mask[kWaves][MOE_MAX_EXPERTS];
    int32_t expert_run[MOE_MAX_EXPERTS];
    int32_t ebase[MOE_MAX_EXPERTS + 1];
    int32_t wave_sum[kWaves];
    int32_t any_bad;
};
struct ExpertLds {
    int32_t hist[kRowsPerGroup][kSmallLayoutChannels];
};
struct RankLds {
    unsigned long long bits[kRowsPerGroup][kMaxWords];
    int32_t pre[kRowsPerGroup][kMaxWords + 1];
};
struct TokenLds {
    int16_t rank[kTokensPerGroup * MOE_MAX_K];  // rank of each of the group's entries, -1 if masked
};
static_assert(kTokensPerGroup * MOE_MAX_K <= kThreads, "one id per lane in the token role");
struct PackLds {
    float wave_max[kWaves];                // row maximum per wave (quantised modes)
    int32_t count[2][kWaves][MOE_MAX_K];   // per-wave counts of entries before (t, k), by item parity
};
static_assert(MOE_MAX_K <= 64, "one k per lane of a wave");
constexpr int kKeysPerLane = kSmallLayoutEntries / kThreads;
static_assert(kKeysPerLane * kThreads == kSmallLayoutEntries, "whole keys per lane");
constexpr size_t max2(size_t a, size_t b) { return a > b ? a : b; }
constexpr size_t kLdsBytes =
    max2(max2(max2(sizeof(SlotLds), sizeof(ExpertLds)), max2(sizeof(RankLds), sizeof(TokenLds))),
         sizeof(PackLds));
static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup on gfx950");

// Inclusive prefix sum over the 64 lanes of a wave with DPP: row_shr 1, 2, 4, 8 within each row of
// 16 lanes, then row_bcast:15 and row_bcast:31 carry row totals upward. Lanes with no source lane
// add the `old` operand, 0.
__device__ inline int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return v;
}

__device__ inline int lane_value(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

__device__ void slots_role(SlotLds &L, const int32_t *__restrict__ topk, int S, int K, int E, int P,
                           int epr, int32_t *__restrict__ num_tokens_per_expert,
                           int32_t *__restrict__ rank_slot_base,
                           int32_t *__restrict__ expert_slot_base, int32_t *__restrict__ slot_idx,
                           int32_t *__restrict__ status) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = S * K;
    const unsigned long long lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int next = tid < N ? topk[tid] : -1;
    for (int i = tid; i < E; i += kThreads) {
        L.expert_run[i] = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) L.lane_mask[w][i] = 0ull;
    }
    if (tid == 0) L.any_bad = 0;
    bool bad = false;
    __syncthreads();

    // expert and rank of this lane's entries, one per batch, kept in registers
    int eid[kBatches], rank_of[kBatches];
#pragma unroll
    for (int bt = 0; bt < kBatches; ++bt) {
        eid[bt] = -1;
        rank_of[bt] = 0;
        const int i0 = bt * kThreads;
        if (i0 >= N) continue;  // uniform: N is the same for the whole workgroup
        const int i = i0 + tid;
        const int v = next;
        next = i + kThreads < N ? topk[i + kThreads] : -1;  // prefetch the next batch
        const bool in = i < N;
        const int e = (in && v >= 0 && v < E) ? v : -1;
        bad = bad || (in && v != -1 && e < 0);
        eid[bt] = e;
        if (e >= 0) atomicOr(&L.lane_mask[wave][e], 1ull << lane);
        __syncthreads();
        bool leader = false;
        int count = 0;
        if (e >= 0) {
            int earlier = 0;
            for (int w = 0; w < wave; ++w) earlier += __popcll(L.lane_mask[w][e]);
            const int below = __popcll(L.lane_mask[wave][e] & lt_mask);
            rank_of[bt] = L.expert_run[e] + earlier + below;
            leader = earlier == 0 && below == 0;  // first entry of expert e in this batch
            if (leader)
                for (int w = 0; w < kWaves; ++w) count += __popcll(L.lane_mask[w][e]);
        }
        __syncthreads();
        if (e >= 0) {
            if (leader) L.expert_run[e] += count;
            L.lane_mask[wave][e] = 0ull;
        }
        __syncthreads();
    }

    // bases: exclusive scan of the per-expert totals (E <= 512 < kThreads)
    const int n = tid < E ? L.expert_run[tid] : 0;
    const int incl = wave_inclusive_scan(n);
    if (lane == 63) L.wave_sum[wave] = incl;
    if (bad) L.any_bad = 1;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        before += w < wave ? L.wave_sum[w] : 0;
        total += L.wave_sum[w];
    }
    if (tid < E) {
        const int b = before + incl - n;
        L.ebase[tid] = b;
        expert_slot_base[tid] = b;
        num_tokens_per_expert[tid] = n;
        if (tid % epr == 0) rank_slot_base[tid / epr] = b;
    }
    if (tid == 0) {
        expert_slot_base[E] = total;
        rank_slot_base[P] = total;
        *status = L.any_bad;
    }
    __syncthreads();
#pragma unroll
    for (int bt = 0; bt < kBatches; ++bt) {
        const int i = bt * kThreads + tid;
        if (i < N) slot_idx[i] = eid[bt] >= 0 ? L.ebase[eid[bt]] + rank_of[bt] : -1;
    }
}

__device__ void experts_role(ExpertLds &L, int e0, const int32_t *__restrict__ topk, int S, int K,
                             int E, int C, int32_t *__restrict__ expert_prefix) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = S * K;
    const int rows = min(kRowsPerGroup, E - e0);
    const int per = S / C, rem = S % C, big = rem * (per + 1);
    for (int j = tid; j < rows * C; j += kThreads) L.hist[j / C][j % C] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += kThreads) {
        const int v = topk[i];
        if (v >= e0 && v < e0 + rows) {  // implies a valid id of this workgroup's rows
            const int t = i / K;
            const int c = t < big ? t / (per + 1) : rem + (t - big) / per;
            atomicAdd(&L.hist[v - e0][c], 1);
        }
    }
    __syncthreads();
    if (wave < rows) {
        int32_t *row = expert_prefix + (int64_t)(e0 + wave) * C;
        int carry = 0;
        for (int c0 = 0; c0 < C; c0 += 64) {
            const int c = c0 + lane;
            const int incl = wave_inclusive_scan(c < C ? L.hist[wave][c] : 0);
            if (c < C) row[c] = carry + incl;
            carry += lane_value(incl, 63);
        }
    }
}

__device__ void ranks_role(RankLds &L, int r0, const int32_t *__restrict__ topk, int S, int K,
                           int E, int P, int epr, int C, int32_t *__restrict__ rank_prefix,
                           int32_t *__restrict__ num_tokens_per_rank) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = S * K;
    const int W = (S + 63) >> 6;
    const int rows = min(kRowsPerGroup, P - r0);
    for (int j = tid; j < rows * W; j += kThreads) L.bits[j / W][j % W] = 0ull;
    __syncthreads();
    for (int i = tid; i < N; i += kThreads) {
        const int v = topk[i];
        if (v >= 0 && v < E) {
            const int r = v / epr - r0;
            if (r >= 0 && r < rows) {
                const int t = i / K;
                atomicOr(&L.bits[r][t >> 6], 1ull << (t & 63));
            }
        }
    }
    __syncthreads();
    if (wave < rows) {
        // exclusive popcount prefix over the row's words, 64 words per step; pre[W] is the total
        int carry = 0;
        for (int w0 = 0; w0 <= W; w0 += 64) {
            const int w = w0 + lane;
            const int pc = w < W ? __popcll(L.bits[wave][w]) : 0;
            const int incl = wave_inclusive_scan(pc);
            if (w <= W) L.pre[wave][w] = carry + incl - pc;
            carry += lane_value(incl, 63);
        }
        const int per = S / C, rem = S % C;
        int32_t *row = rank_prefix + (int64_t)(r0 + wave) * C;
        for (int c = lane; c < C; c += 64) {
            const int end = (c + 1) * per + min(c + 1, rem);
            const int w = end >> 6, b = end & 63;
            int val = L.pre[wave][w];
            if (b) val += __popcll(L.bits[wave][w] & ((1ull << b) - 1ull));
            row[c] = val;
        }
        if (lane == 0) num_tokens_per_rank[r0 + wave] = carry;
    }
}

__device__ void tokens_role(TokenLds &L, int t0, const int32_t *__restrict__ topk, int S, int K,
                            int E, int P, int epr, uint8_t *__restrict__ is_in) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t1 = min(t0 + kTokensPerGroup, S);
    // the group's K ids per token, one coalesced load per lane (kTokensPerGroup * K <= kThreads)
    const int n = (t1 - t0) * K;
    if (tid < n) {
        const int v = topk[(int64_t)t0 * K + tid];
        L.rank[tid] = (int16_t)((v >= 0 && v < E) ? v / epr : -1);
    }
    __syncthreads();
    const bool words = (P & 3) == 0 && (((uintptr_t)is_in) & 3) == 0;
    for (int t = t0 + wave; t < t1; t += kWaves) {
        const int16_t *rk = L.rank + (t - t0) * K;
        if (words) {
            uint32_t *dst = reinterpret_cast<uint32_t *>(is_in + (int64_t)t * P);
            for (int wd = lane; wd < (P >> 2); wd += 64) {
                uint32_t val = 0;
                for (int k = 0; k < K; ++k) {
                    const int r = rk[k];
                    if (r >= 0 && (r >> 2) == wd) val |= 1u << (8 * (r & 3));
                }
                dst[wd] = val;
            }
        } else {
            for (int r = lane; r < P; r += 64) {
                bool hit = false;
                for (int k = 0; k < K; ++k) hit = hit || rk[k] == r;
                is_in[(int64_t)t * P + r] = hit ? 1 : 0;
            }
        }
    }
}

// Workgroups taking the four layout roles, for S tokens, E experts and P ranks.
inline int layout_groups(int S, int E, int P) {
    return 1 + (E + kRowsPerGroup - 1) / kRowsPerGroup + (P + kRowsPerGroup - 1) / kRowsPerGroup +
           (S + kTokensPerGroup - 1) / kTokensPerGroup;
}

__device__ __forceinline__ void layout_roles(
    unsigned char *lds, int b, const int32_t *__restrict__ topk, int S, int K, int E, int P, int epr,
    int C, uint8_t *__restrict__ is_in, int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ num_tokens_per_expert, int32_t *__restrict__ rank_prefix,
    int32_t *__restrict__ expert_prefix, int32_t *__restrict__ rank_slot_base,
    int32_t *__restrict__ expert_slot_base, int32_t *__restrict__ slot_idx,
    int32_t *__restrict__ status) {
    const int nE = (E + kRowsPerGroup - 1) / kRowsPerGroup;
    const int nR = (P + kRowsPerGroup - 1) / kRowsPerGroup;
    if (b == 0)
        slots_role(*reinterpret_cast<SlotLds *>(lds), topk, S, K, E, P, epr,
                   num_tokens_per_expert, rank_slot_base, expert_slot_base, slot_idx, status);
    else if (b <= nE)
        experts_role(*reinterpret_cast<ExpertLds *>(lds), (b - 1) * kRowsPerGroup, topk, S, K, E, C,
                     expert_prefix);
    else if (b <= nE + nR)
        ranks_role(*reinterpret_cast<RankLds *>(lds), (b - 1 - nE) * kRowsPerGroup, topk, S, K, E,
                   P, epr, C, rank_prefix, num_tokens_per_rank);
    else
        tokens_role(*reinterpret_cast<TokenLds *>(lds), (b - 1 - nE - nR) * kTokensPerGroup, topk, S,
                    K, E, P, epr, is_in);
}

__global__ __launch_bounds__(kThreads) void layout_small_kernel(
    const int32_t *__restrict__ topk, int S, int K, int E, int P, int epr, int C,
    uint8_t *__restrict__ is_in, int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ num_tokens_per_expert, int32_t *__restrict__ rank_prefix,
    int32_t *__restrict__ expert_prefix, int32_t *__restrict__ rank_slot_base,
    int32_t *__restrict__ expert_slot_base, int32_t *__restrict__ slot_idx,
    int32_t *__restrict__ status) {
    __shared__ __align__(16) unsigned char lds[kLdsBytes];
    layout_roles(lds, blockIdx.x, topk, S, K, E, P, epr, C, is_in, num_tokens_per_rank,
                 num_tokens_per_expert, rank_prefix, expert_prefix, rank_slot_base, expert_slot_base,
                 slot_idx, status);
}

// Pack role: workgroup g of ngroups takes work items g, g + ngroups, ... of S * nparts, item
// (t, q) = part q of token t's row. nvec: 16-byte vectors per bf16 row (split into nparts parts);
// ngroups_q: 16-element code groups per row for the quantised modes (nparts = 1, one group per
// lane). Every lane of the workgroup runs every item, so the barriers are uniform.
//
// Per item the loads (the token's K ids, one per lane, and its row) are issued together; the
// slot count then needs one barrier: each wave ballots its lanes' keys against the K entries,
// lane 0 writes the wave's K counts, and after the barrier lane k of every wave sums the counts of
// entry k over the waves and the slots reach the other lanes by readlane. The counts alternate
// between two buffers, so the next item can write its counts while a slower wave still reads
// these (it cannot pass the next barrier before that wave arrives there).
template <int QUANT>
__device__ __forceinline__ void pack_role(PackLds &L, int g, int ngroups, const int32_t *__restrict__ topk,
                                          int S, int K, int E, const uint8_t *__restrict__ x,
                                          int nvec, int nparts, int ngroups_q, const SlotGeom &geom,
                                          int src_rank, uint8_t *__restrict__ window) {
    using namespace rows;
    const int u = threadIdx.x, lane = u & 63, wave = u >> 6;
    const int n = S * K;
    // The table as sort keys: id * n + flat index for a valid id, above every valid key otherwise.
    int key[kKeysPerLane];
#pragma unroll
    for (int m = 0; m < kKeysPerLane; ++m) {
        const int j = u + m * kThreads;
        const int e = j < n ? topk[j] : -1;
        key[m] = (j < n && e >= 0 && e < E) ? e * n + j : INT32_MAX;
    }
    const int ntail = (geom.tail_end - geom.payload_bytes) >> 4;
    const int per = (nvec + nparts - 1) / nparts;
    int parity = 0;
    for (int item = g; item < S * nparts; item += ngroups, parity ^= 1) {
        const int t = item / nparts, q = item - t * nparts;
        // lane k of every wave holds id k of the token
        const int my_id = lane < K ? topk[(int64_t)t * K + lane] : -1;
        const int row_bytes = nvec << 4;
        const __amdgpu_buffer_rsrc_t src = rsrc(x + (int64_t)t * row_bytes, row_bytes);
        const int v0 = q * per + u, v1 = min(nvec, (q + 1) * per);
        u32x4 r = {0u, 0u, 0u, 0u};
        u32x4 codes = {0u, 0u, 0u, 0u};
        uint32_t scale_bits = 0u;
        if constexpr (QUANT == MOE_QUANT_NONE) {
            if (v0 < v1) r = load16(src, v0 << 4);
        } else {
            quantise_row<QUANT>(x, t, ngroups_q, L.wave_max, codes, scale_bits);
        }
        const bool my_valid = my_id >= 0 && my_id < E;
        const int my_key = my_valid ? my_id * n + t * K + lane : -1;
        for (int k = 0; k < K; ++k) {
            const int mine = __builtin_amdgcn_readlane(my_key, k);
            int c = 0;
#pragma unroll
            for (int m = 0; m < kKeysPerLane; ++m) c += __popcll(__ballot(key[m] < mine));
            if (lane == 0) L.count[parity][wave][k] = c;
        }
        __syncthreads();
        int my_slot = -1;
        if (lane < K && my_valid) {
            int c = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) c += L.count[parity][w][lane];
            my_slot = c;
        }
        if constexpr (QUANT == MOE_QUANT_NONE) {
            for (int v = v0; v < v1; v += kThreads) {
                if (v != v0) r = load16(src, v << 4);
                for (int k = 0; k < K; ++k) {
                    const int64_t s = __builtin_amdgcn_readlane(my_slot, k);
                    if (s >= 0) store16(r, rsrc(window + s * geom.slot_bytes, geom.tail_end), v << 4);
                }
            }
            if (q == nparts - 1 && u < ntail)
                for (int k = 0; k < K; ++k) {
                    const int64_t s = __builtin_amdgcn_readlane(my_slot, k);
                    if (s >= 0)
                        store_tail(rsrc(window + s * geom.slot_bytes, geom.tail_end), geom, u, 0u,
                                   src_rank, t, k);
                }
        } else {
            for (int k = 0; k < K; ++k) {
                const int64_t s = __builtin_amdgcn_readlane(my_slot, k);
                if (s < 0) continue;
                const __amdgpu_buffer_rsrc_t dst = rsrc(window + s * geom.slot_bytes, geom.tail_end);
                if (u < ngroups_q) store16(codes, dst, u << 4);
                if (u < ntail) store_tail(dst, geom, u, scale_bits, src_rank, t, k);
            }
        }
    }
}

// Layout (workgroups [0, nlayout)) and pack (the rest) of a small routing table in one launch.
template <int QUANT>
__global__ __launch_bounds__(kThreads) void layout_pack_small_kernel(
    const int32_t *__restrict__ topk, int S, int K, int E, int P, int epr, int C,
    uint8_t *__restrict__ is_in, int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ num_tokens_per_expert, int32_t *__restrict__ rank_prefix,
    int32_t *__restrict__ expert_prefix, int32_t *__restrict__ rank_slot_base,
    int32_t *__restrict__ expert_slot_base, int32_t *__restrict__ slot_idx,
    int32_t *__restrict__ status, int nlayout, const uint8_t *__restrict__ x, int nvec, int nparts,
    int ngroups_q, SlotGeom geom, int src_rank, uint8_t *__restrict__ window) {
    __shared__ __align__(16) unsigned char lds[kLdsBytes];
    const int b = blockIdx.x;
    if (b < nlayout)
        layout_roles(lds, b, topk, S, K, E, P, epr, C, is_in, num_tokens_per_rank,
                     num_tokens_per_expert, rank_prefix, expert_prefix, rank_slot_base,
                     expert_slot_base, slot_idx, status);
    else
        pack_role<QUANT>(*reinterpret_cast<PackLds *>(lds), b - nlayout, gridDim.x - nlayout, topk, S,
                         K, E, x, nvec, nparts, ngroups_q, geom, src_rank, window);
}

// Compute units of the device that runs `stream` (cached per device). The fused grid is capped
// there: measured on MI355X, a grid larger than one workgroup per compute unit runs as a second
// round (at 384 workgroups the kernel took twice as long as at 256), although HIP's occupancy
// calculator reports room for two of these workgroups per unit.
int compute_units(hipStream_t stream) {
    // Racing first calls on several host threads all store the same value; relaxed atomics make
    // that race well defined. A device id of 64 or more is queried on every call.
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        n = 256;
    if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <int QUANT>
hipError_t launch_fused(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                        int32_t C, uint8_t *is_in, int32_t *ntpr, int32_t *ntpe, int32_t *rpm,
                        int32_t *epm, int32_t *rsb, int32_t *esb, int32_t *slot_idx,
                        int32_t *status, const void *x, int32_t H, int32_t src_rank, void *window,
                        hipStream_t stream) {
    const SlotGeom geom = slot_geom(H, QUANT);
    const int nlayout = layout_groups(S, E, P);
    const int nvec = H / 8;
    const int ngroups_q = H / 16;
    // the pack workgroups take the compute units the layout roles leave free; a bf16 row is split
    // into up to 4 parts when that spreads a small batch over more of them
    const int room = compute_units(stream) - nlayout;
    const int slots = room > 1 ? room : 1;
    int nparts = 1;
    if (QUANT == MOE_QUANT_NONE) {
        nparts = slots / S;
        nparts = nparts < 1 ? 1 : (nparts > 4 ? 4 : nparts);
    }
    const int items = S * nparts;
    const int npack = items < slots ? items : slots;
    hipLaunchKernelGGL((layout_pack_small_kernel<QUANT>), dim3(nlayout + npack), dim3(kThreads), 0,
                       stream, topk_idx, S, K, E, P, E / P, C, is_in, ntpr, ntpe, rpm, epm, rsb,
                       esb, slot_idx, status, nlayout, static_cast<const uint8_t *>(x), nvec,
                       nparts, ngroups_q, geom, src_rank, static_cast<uint8_t *>(window));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_layout_small(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                               int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                               int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                               int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                               int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                               hipStream_t stream) {
    hipLaunchKernelGGL(layout_small_kernel, dim3(layout_groups(S, E, P)), dim3(kThreads), 0, stream, topk_idx, S, K,
                       E, P, E / P, C, is_token_in_rank, num_tokens_per_rank, num_tokens_per_expert,
                       rank_prefix_matrix, expert_prefix_matrix, rank_slot_base, expert_slot_base,
                       slot_idx, status);
    return hipGetLastError();
}

hipError_t launch_layout_dispatch_small(
    const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
    uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
    int32_t *rank_prefix_matrix, int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
    int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status, const void *x, int32_t H,
    int32_t quant, int32_t src_rank, void *window, hipStream_t stream) {
    if (quant == MOE_QUANT_FP8_E4M3_DYN)
        return launch_fused<MOE_QUANT_FP8_E4M3_DYN>(
            topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank, num_tokens_per_expert,
            rank_prefix_matrix, expert_prefix_matrix, rank_slot_base, expert_slot_base, slot_idx,
            status, x, H, src_rank, window, stream);
    if (quant == MOE_QUANT_INT8_DYN)
        return launch_fused<MOE_QUANT_INT8_DYN>(
            topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank, num_tokens_per_expert,
            rank_prefix_matrix, expert_prefix_matrix, rank_slot_base, expert_slot_base, slot_idx,
            status, x, H, src_rank, window, stream);
    return launch_fused<MOE_QUANT_NONE>(
        topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank, num_tokens_per_expert,
        rank_prefix_matrix, expert_prefix_matrix, rank_slot_base, expert_slot_base, slot_idx,
        status, x, H, src_rank, window, stream);
}

}  // namespace moe
