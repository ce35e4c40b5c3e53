// Routing layout kernels for gfx950 (wave64).
//
// The layout turns topk_idx[S,K] into the dispatch handle of "Ascend DeepEP MoE Dispatch
// Optimization" (section "Dispatch handle 六项分别保存什么": is_token_in_rank, rank / channel prefix
// matrices) plus the slot of every (token, k): the per-expert offset + running count of the CAM
// pack ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.6 InputToShare), resolved before any
// byte moves so the pack is a pure scatter.
//
// Three launches on one stream:
//   count  one workgroup per channel. LDS histograms of ranks (a rank counted once per token) and
//          experts, the token rows of is_token_in_rank, and for each valid entry its rank among the
//          channel's entries of the same expert in (t, k) order. That rank comes from per-wave LDS
//          lane masks + popcount, so atomics only build masks and counts and never decide an order.
//          Raw counts go to column c of both prefix matrices.
//   scan   one wave per matrix row: in-place inclusive scan along the channels.
//   assign one workgroup per channel: exclusive scan of the per-expert totals (the slot bases), then
//          slot = base[e] + prefix[e][c-1] + local rank. Workgroup 0 also writes the count vectors.
// Everything is derived from the K ids of each token, so no pass scans the [S, P] matrix.

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRankWords = (MOE_MAX_RANKS + 31) / 32;

__device__ inline void channel_range(int S, int C, int c, int &begin, int &end) {
    // floor share + remainder to the first channels ("HCCL Window 模式", section 8.3 分片策略)
    const int per = S / C, rem = S % C;
    begin = c * per + (c < rem ? c : rem);
    end = begin + per + (c < rem ? 1 : 0);
}

__device__ inline int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

__global__ __launch_bounds__(kThreads) void layout_count_kernel(
    const int32_t *__restrict__ topk, int S, int K, int E, int P, int epr, int C,
    uint8_t *__restrict__ is_in, int32_t *__restrict__ rank_prefix,
    int32_t *__restrict__ expert_prefix, int32_t *__restrict__ slot_local) {
    __shared__ uint32_t rank_bits[kThreads][kRankWords];
    __shared__ int32_t rank_cnt[MOE_MAX_RANKS];
    __shared__ int32_t expert_run[MOE_MAX_EXPERTS];
    __shared__ unsigned long long lane_mask[kWaves][MOE_MAX_EXPERTS];

    const int c = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int tb, te;
    channel_range(S, C, c, tb, te);

    for (int i = tid; i < P; i += kThreads) rank_cnt[i] = 0;
    for (int i = tid; i < E; i += kThreads) {
        expert_run[i] = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) lane_mask[w][i] = 0ull;
    }
    __syncthreads();

    // Phase A: one thread per token. Distinct ranks of the token -> rank histogram + row bits.
    const int nwords = (P + 31) >> 5;
    for (int t0 = tb; t0 < te; t0 += kThreads) {
        const int ntok = min(kThreads, te - t0);
        for (int w = 0; w < nwords; ++w) rank_bits[tid][w] = 0u;
        if (tid < ntok) {
            const int32_t *row = topk + (int64_t)(t0 + tid) * K;
            int rr[MOE_MAX_K];
#pragma unroll
            for (int k = 0; k < MOE_MAX_K; ++k) {
                rr[k] = -1;
                if (k < K) {
                    const int e = row[k];
                    if (e >= 0 && e < E) rr[k] = e / epr;
                }
            }
#pragma unroll
            for (int k = 0; k < MOE_MAX_K; ++k) {
                bool first = rr[k] >= 0;
#pragma unroll
                for (int j = 0; j < k; ++j) first = first && (rr[j] != rr[k]);
                if (first) {
                    atomicAdd(&rank_cnt[rr[k]], 1);
                    rank_bits[tid][rr[k] >> 5] |= 1u << (rr[k] & 31);
                }
            }
        }
        __syncthreads();
        // rows [t0, t0 + ntok) are the contiguous bytes [t0 * P, (t0 + ntok) * P)
        uint8_t *dst = is_in + (int64_t)t0 * P;
        const int nbytes = ntok * P;
        if ((((uintptr_t)dst) & 3) == 0 && (nbytes & 3) == 0) {
            uint32_t *dst32 = reinterpret_cast<uint32_t *>(dst);
            for (int wd = tid; wd < (nbytes >> 2); wd += kThreads) {
                uint32_t v = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int i = 4 * wd + b;
                    const int tl = i / P, r = i - tl * P;
                    v |= ((rank_bits[tl][r >> 5] >> (r & 31)) & 1u) << (8 * b);
                }
                dst32[wd] = v;
            }
        } else {
            for (int i = tid; i < nbytes; i += kThreads) {
                const int tl = i / P, r = i - tl * P;
                dst[i] = (uint8_t)((rank_bits[tl][r >> 5] >> (r & 31)) & 1u);
            }
        }
        __syncthreads();
    }

    // Phase B: the channel's entries [tb*K, te*K) in (t, k) order, kThreads at a time.
    const int64_t eb = (int64_t)tb * K, ee = (int64_t)te * K;
    const unsigned long long lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int64_t i0 = eb; i0 < ee; i0 += kThreads) {
        const int64_t i = i0 + tid;
        int e = -1;
        if (i < ee) {
            const int v = topk[i];
            if (v >= 0 && v < E) e = v;
        }
        if (e >= 0) atomicOr(&lane_mask[wave][e], 1ull << lane);
        __syncthreads();
        bool leader = false;
        int total = 0;
        if (e >= 0) {
            const unsigned long long mine = lane_mask[wave][e];
            int before = 0;
            for (int w = 0; w < wave; ++w) before += __popcll(lane_mask[w][e]);
            const int below = __popcll(mine & lt_mask);
            slot_local[i] = expert_run[e] + before + below;
            leader = before == 0 && below == 0;  // first entry of expert e in this batch
            if (leader)
                for (int w = 0; w < kWaves; ++w) total += __popcll(lane_mask[w][e]);
        }
        __syncthreads();
        if (e >= 0) {
            if (leader) expert_run[e] += total;
            lane_mask[wave][e] = 0ull;
        }
        __syncthreads();
    }

    // Phase C: raw per-channel counts into column c.
    for (int e = tid; e < E; e += kThreads) expert_prefix[(int64_t)e * C + c] = expert_run[e];
    for (int r = tid; r < P; r += kThreads) rank_prefix[(int64_t)r * C + c] = rank_cnt[r];
}

__global__ __launch_bounds__(kThreads) void layout_scan_kernel(int32_t *__restrict__ expert_prefix,
                                                               int32_t *__restrict__ rank_prefix,
                                                               int E, int P, int C,
                                                               int32_t *__restrict__ status) {
    const int row_id = (blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (blockIdx.x == 0 && threadIdx.x == 0) *status = 0;
    if (row_id >= E + P) return;  // whole waves only
    int32_t *row = row_id < E ? expert_prefix + (int64_t)row_id * C
                              : rank_prefix + (int64_t)(row_id - E) * C;
    int carry = 0;
    for (int j = 0; j < C; j += 64) {
        const bool in = j + lane < C;
        int v = in ? row[j + lane] : 0;
        v = wave_inclusive_scan(v, lane);
        if (in) row[j + lane] = v + carry;
        carry += __shfl(v, 63, 64);
    }
}

__global__ __launch_bounds__(kThreads) void layout_assign_kernel(
    const int32_t *__restrict__ topk, int S, int K, int E, int P, int epr, int C,
    const int32_t *__restrict__ expert_prefix, const int32_t *__restrict__ rank_prefix,
    int32_t *__restrict__ slot_idx, int32_t *__restrict__ expert_slot_base,
    int32_t *__restrict__ rank_slot_base, int32_t *__restrict__ num_tokens_per_expert,
    int32_t *__restrict__ num_tokens_per_rank, int32_t *__restrict__ status) {
    __shared__ int32_t off[MOE_MAX_EXPERTS];
    __shared__ int32_t wave_sum[kWaves];

    const int c = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Exclusive scan of the per-expert totals (last column); thread tid owns experts 2tid, 2tid+1.
    const int e0 = 2 * tid, e1 = 2 * tid + 1;
    const int n0 = e0 < E ? expert_prefix[(int64_t)e0 * C + C - 1] : 0;
    const int n1 = e1 < E ? expert_prefix[(int64_t)e1 * C + C - 1] : 0;
    const int p0 = (c > 0 && e0 < E) ? expert_prefix[(int64_t)e0 * C + c - 1] : 0;
    const int p1 = (c > 0 && e1 < E) ? expert_prefix[(int64_t)e1 * C + c - 1] : 0;
    const int pair = n0 + n1;
    const int incl = wave_inclusive_scan(pair, lane);
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        before += w < wave ? wave_sum[w] : 0;
        total += wave_sum[w];
    }
    const int base0 = before + incl - pair, base1 = base0 + n0;
    if (e0 < E) off[e0] = base0 + p0;
    if (e1 < E) off[e1] = base1 + p1;
    if (c == 0) {
        if (e0 < E) {
            expert_slot_base[e0] = base0;
            num_tokens_per_expert[e0] = n0;
            if (e0 % epr == 0) rank_slot_base[e0 / epr] = base0;
        }
        if (e1 < E) {
            expert_slot_base[e1] = base1;
            num_tokens_per_expert[e1] = n1;
            if (e1 % epr == 0) rank_slot_base[e1 / epr] = base1;
        }
        if (tid == 0) {
            expert_slot_base[E] = total;
            rank_slot_base[P] = total;
        }
        for (int r = tid; r < P; r += kThreads)
            num_tokens_per_rank[r] = rank_prefix[(int64_t)r * C + C - 1];
    }
    __syncthreads();

    int tb, te;
    channel_range(S, C, c, tb, te);
    bool bad = false;
    for (int64_t i = (int64_t)tb * K + tid; i < (int64_t)te * K; i += kThreads) {
        const int e = topk[i];
        if (e >= 0 && e < E) {
            slot_idx[i] = off[e] + slot_idx[i];
        } else {
            slot_idx[i] = -1;
            bad = bad || e != -1;
        }
    }
    if (bad) atomicOr(status, 1);
}

}  // namespace

hipError_t launch_layout(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                         int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                         int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                         int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                         int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                         hipStream_t stream) {
    const int epr = E / P;
    hipLaunchKernelGGL(layout_count_kernel, dim3(C), dim3(kThreads), 0, stream, topk_idx, S, K, E,
                       P, epr, C, is_token_in_rank, rank_prefix_matrix, expert_prefix_matrix,
                       slot_idx);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int scan_blocks = (E + P + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(layout_scan_kernel, dim3(scan_blocks), dim3(kThreads), 0, stream,
                       expert_prefix_matrix, rank_prefix_matrix, E, P, C, status);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(layout_assign_kernel, dim3(C), dim3(kThreads), 0, stream, topk_idx, S, K, E,
                       P, epr, C, expert_prefix_matrix, rank_prefix_matrix, slot_idx,
                       expert_slot_base, rank_slot_base, num_tokens_per_expert,
                       num_tokens_per_rank, status);
    return hipGetLastError();
}

}  // namespace moe
