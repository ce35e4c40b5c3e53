// Routing layout kernels for gfx950 (wave64).
//
// The layout turns topk_idx[S,K] into the dispatch handle of "Ascend DeepEP MoE Dispatch
// Optimization" (section "Dispatch handle 六项分别保存什么": is_token_in_rank, rank / channel prefix
// matrices) plus the slot of every (token, k): the per-expert offset + running count of the CAM
// pack ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.6 InputToShare), resolved before any
// byte moves so the pack is a pure scatter. Counts and prefix sums follow the notify stage of the
// same DeepEP page ("Notify 先交换数量和前缀") and "internode.cu" section 1 notify_dispatch.
//
// Three launches on one stream, each built around a single round trip to memory:
//   count  one workgroup per channel. Lanes map to (token, k) with a power-of-two lane group per
//          token, in (t, k) order. Per batch: a rank is counted once per token (a lane counts it
//          only if no lower lane of its token has the same rank, compared with DPP row shifts);
//          per-wave LDS lane masks + popcount give each entry its rank among the channel's earlier
//          entries of the same expert (atomics build masks and counts, never an order, so the
//          result is deterministic); the token rows of is_token_in_rank are assembled in LDS and
//          written as words. Raw counts go to column c of both prefix matrices.
//   scan   one wave per matrix row: all of the row is loaded first, then scanned along the channels
//          in place (inclusive).
//   assign one workgroup per channel: exclusive scan of the per-expert totals (the slot bases), then
//          slot = base[e] + prefix[e][c-1] + local rank. Workgroup 0 also writes the count vectors.
// Nothing scans the [S, P] matrix: everything is derived from the K ids of each token.
// Small tables (decode-sized batches) take the single-launch path in layout_small.hip instead.
//
// The workspace form (moe_layout_ws) needs two launches:
//   count     as above, and besides: the channel's exclusive scan over experts of its counts
//             (colexcl[e][c]) and its entries grouped by expert in a per-channel bucket list.
//   finalize  workgroups per expert (8 slices of each when C <= 256, so that one hot expert of a
//             skewed routing is spread over several CUs): the expert's count in channel c is
//             colexcl[e+1][c] - colexcl[e][c], its slot base the sum of colexcl[e][.] over the
//             channels, and entry j of the expert sits in the bucket list of the channel c with
//             prefix[c-1] <= j < prefix[c]; so each slice writes its entries' slots with no further
//             scan. The same kernel scans the rank rows and, for the planned bf16 pack, writes each
//             entry's (slot, token, k) record at its place in the pack plan (groups of whole
//             channels, slot order inside a group), which the separate plan kernel would otherwise
//             build. Measured at S=4096, K=8, E=256, C=128: 4.8 + 6.1 us against 4.0 + 2.9 + 3.3 us
//             for the three launches and 4.0 us for the plan kernel; with Zipf routing at S=8192
//             (one expert holding about a fifth of the entries) 7.6 + 6.7 us.

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRankWords = (MOE_MAX_RANKS + 31) / 32;
constexpr int kScanRegs = 16;  // row chunks of 64 held in registers by the scan (C <= 1024 in one go)

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

// True iff rank r (>= 0) differs from the ranks held by the lk lanes just below this one, which
// are the lower lanes of the same token (a token's KP lanes never straddle a 16-lane DPP row).
// Every shifted value is computed on all lanes; only bitwise ops combine them.
template <int KP, int J = 1>
__device__ inline bool no_lower_match(int r, int lk) {
    if constexpr (J >= KP) {
        return true;
    } else {
        // row_shr:J -> value of lane (lane - J) within the 16-lane row; -2 where there is none
        const int rj = __builtin_amdgcn_update_dpp(-2, r, 0x110 + J, 0xF, 0xF, false);
        return !((J <= lk) & (rj == r)) & no_lower_match<KP, J + 1>(r, lk);
    }
}

template <int KP>
__device__ inline bool first_in_token(int r, int lk) {
    return (r >= 0) & no_lower_match<KP>(r, lk);
}

// WS: the workspace form (moe_layout_dispatch_ws). It writes the raw rank counts, but not the
// expert counts; instead, for the finalize kernel: -1 into slot_idx for every masked entry; the
// channel's exclusive scan over experts of its counts into colexcl[e][c] (entries of channel c routed
// to experts below e); the channel's valid entries grouped by expert into bucket[tb*K ..] (position
// colexcl[e][c] + rank of the entry among the channel's entries of expert e); and (valid count,
// bad-id flag) into chan[2c], chan[2c+1]. The count of expert e in channel c is then
// colexcl[e+1][c] - colexcl[e][c] (chan[2c] - colexcl[E-1][c] for the last expert).
constexpr int kEntCap = 4096;  // entries of a channel kept in LDS for the grouping (WS)

template <int KP, bool WS>
__global__ __launch_bounds__(kThreads) void layout_count_kernel(
    const int32_t *__restrict__ topk, int S, int K, int E, int P, int epr, int C,
    uint8_t *__restrict__ is_in, int32_t *__restrict__ rank_prefix,
    int32_t *__restrict__ expert_prefix, int32_t *__restrict__ slot_local,
    int32_t *__restrict__ colexcl, int32_t *__restrict__ bucket, int32_t *__restrict__ chan) {
    constexpr int kTokWave = 64 / KP;             // tokens per wave per batch
    constexpr int kTokBatch = kWaves * kTokWave;  // tokens per batch
    __shared__ uint32_t row_bits[kTokBatch][kRankWords];
    __shared__ int32_t rank_cnt[MOE_MAX_RANKS];
    __shared__ int32_t expert_run[MOE_MAX_EXPERTS];
    __shared__ unsigned long long lane_mask[kWaves][MOE_MAX_EXPERTS];
    __shared__ int32_t ent[WS ? kEntCap : 1];  // (local << 9 | e) or -1 per entry of the channel (WS)

    const int c = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tl = wave * kTokWave + lane / KP;  // token of this lane within the batch
    const int lk = lane % KP;                    // k of this lane
    int tb, te;
    channel_range(S, C, c, tb, te);

    const int nwords = (P + 31) >> 5;
    for (int i = tid; i < P; i += kThreads) rank_cnt[i] = 0;
    for (int i = tid; i < E; i += kThreads) {
        expert_run[i] = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) lane_mask[w][i] = 0ull;
    }
    for (int i = tid; i < kTokBatch * nwords; i += kThreads) row_bits[i / nwords][i % nwords] = 0u;

    const unsigned long long lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    auto fetch = [&](int t0) {
        const int t = t0 + tl;
        return (t < te && lk < K) ? topk[(int64_t)t * K + lk] : -1;
    };
    int next = fetch(tb);
    const int64_t b0 = (int64_t)tb * K;
    const bool in_lds = (int64_t)(te - tb) * K <= kEntCap;
    bool bad = false;
    __syncthreads();
    for (int t0 = tb; t0 < te; t0 += kTokBatch) {
        const int v = next;
        next = fetch(t0 + kTokBatch);  // prefetch the following batch
        const int t = t0 + tl;
        const int e = (v >= 0 && v < E) ? v : -1;
        if constexpr (WS) {
            bad = bad || (v != -1 && e < 0);
            if (e < 0 && t < te && lk < K) {
                slot_local[(int64_t)t * K + lk] = -1;
                if (in_lds) ent[(t - tb) * K + lk] = -1;
            }
        }
        const int r = e >= 0 ? e / epr : -1;
        if (first_in_token<KP>(r, lk)) {
            atomicAdd(&rank_cnt[r], 1);
            atomicOr(&row_bits[tl][r >> 5], 1u << (r & 31));
        }
        if (e >= 0) atomicOr(&lane_mask[wave][e], 1ull << lane);
        __syncthreads();

        // local rank among the channel's earlier entries of the same expert
        bool leader = false;
        int count = 0;
        if (e >= 0) {
            const unsigned long long mine = lane_mask[wave][e];
            int earlier = 0;
            for (int w = 0; w < wave; ++w) earlier += __popcll(lane_mask[w][e]);
            const int below = __popcll(mine & lt_mask);
            const int local = expert_run[e] + earlier + below;
            if constexpr (WS) {
                if (in_lds) ent[(t - tb) * K + lk] = (local << 9) | e;
                else slot_local[(int64_t)t * K + lk] = local;
            } else {
                slot_local[(int64_t)t * K + lk] = local;
            }
            leader = earlier == 0 && below == 0;  // first entry of expert e in this batch
            if (leader)
                for (int w = 0; w < kWaves; ++w) count += __popcll(lane_mask[w][e]);
        }

        // token rows [t0, t0 + ntok) are the contiguous bytes [t0 * P, (t0 + ntok) * P)
        const int ntok = min(kTokBatch, te - t0);
        uint8_t *dst = is_in + (int64_t)t0 * P;
        const int nbytes = ntok * P;
        if ((((uintptr_t)dst) & 3) == 0 && (nbytes & 3) == 0) {
            uint32_t *dst32 = reinterpret_cast<uint32_t *>(dst);
            for (int wd = tid; wd < (nbytes >> 2); wd += kThreads) {
                uint32_t val = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int i = 4 * wd + b;
                    const int tk = i / P, rr = i - tk * P;
                    val |= ((row_bits[tk][rr >> 5] >> (rr & 31)) & 1u) << (8 * b);
                }
                dst32[wd] = val;
            }
        } else {
            for (int i = tid; i < nbytes; i += kThreads) {
                const int tk = i / P, rr = i - tk * P;
                dst[i] = (uint8_t)((row_bits[tk][rr >> 5] >> (rr & 31)) & 1u);
            }
        }
        __syncthreads();
        if (e >= 0) {
            if (leader) expert_run[e] += count;
            lane_mask[wave][e] = 0ull;
        }
        for (int i = tid; i < ntok * nwords; i += kThreads) row_bits[i / nwords][i % nwords] = 0u;
        __syncthreads();
    }

    // raw per-channel counts into column c
    if constexpr (!WS)
        for (int e = tid; e < E; e += kThreads) expert_prefix[(int64_t)e * C + c] = expert_run[e];
    for (int rr = tid; rr < P; rr += kThreads) rank_prefix[(int64_t)rr * C + c] = rank_cnt[rr];
    if constexpr (WS) {
        // exclusive scan of the channel's per-expert counts (two experts per thread, E <= 512)
        __shared__ int32_t wave_sum[kWaves];
        int32_t *colex = reinterpret_cast<int32_t *>(lane_mask);  // free again: reused as [E]
        const int e0 = 2 * tid, e1 = 2 * tid + 1;
        const int n0 = e0 < E ? expert_run[e0] : 0, n1 = e1 < E ? expert_run[e1] : 0;
        const int pair = n0 + n1;
        const int incl = wave_inclusive_scan(pair, lane);
        if (lane == 63) wave_sum[wave] = incl;
        const int any_bad = __syncthreads_or(bad ? 1 : 0);
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            before += w < wave ? wave_sum[w] : 0;
            total += wave_sum[w];
        }
        const int x0 = before + incl - pair, x1 = x0 + n0;
        if (e0 < E) {
            colex[e0] = x0;
            colexcl[(int64_t)e0 * C + c] = x0;
        }
        if (e1 < E) {
            colex[e1] = x1;
            colexcl[(int64_t)e1 * C + c] = x1;
        }
        if (tid == 0) {
            chan[2 * c] = total;
            chan[2 * c + 1] = any_bad;
        }
        __syncthreads();  // also orders this workgroup's slot_local stores before the loads below
        const int n_ent = (te - tb) * K;
        if (in_lds) {
            for (int i = tid; i < n_ent; i += kThreads) {
                const int pk = ent[i];
                if (pk >= 0) bucket[b0 + colex[pk & 511] + (pk >> 9)] = (int32_t)(b0 + i);
            }
        } else {  // channels above kEntCap entries: read the ids and ranks back
            for (int i = tid; i < n_ent; i += kThreads) {
                const int v = topk[b0 + i];
                if (v < 0 || v >= E) continue;
                bucket[b0 + colex[v] + slot_local[b0 + i]] = (int32_t)(b0 + i);
            }
        }
    }
}

// Second launch of the workspace layout (moe_layout_dispatch_ws). Workgroups [0, E * ns): slice s of
// expert e = b / ns. Each builds the expert's inclusive prefix along the channels from the count
// kernel's column scans and its base (the sum over channels of colexcl[e][c], the entries routed to
// lower experts); slice 0 writes the prefix row, the total and the slot bases. Slice s then gives the
// s-th of ns equal stretches of the expert's entries their slots, taken from the channels' buckets in
// order (entry j of expert e is in the channel c with M[c-1] <= j < M[c]), and, with a plan, their
// records in the pack plan of the channel group that holds them (plan position: the group's entries
// of lower experts, then expert e's earlier entries of the group). Slices keep one hot expert of a
// skewed routing from serialising on one workgroup. Workgroups [E * ns, E * ns + nrank): one wave
// per rank row. The rest: one per plan list slot g (padding records after the group's valid entries;
// all of a slot past the last group); the first of them writes status; without a plan there is one
// such workgroup (status only). Dynamic LDS: 3 * C int32.
struct FinalizePlan {
    int2 *plan;  // null: no plan
    int cpc;     // channels per group
    int ngroups; // groups
    int nsx;     // group slots per XCD list
    int cap;     // records per group
};

constexpr int kFinUnroll = 4;  // entries per thread in flight in the slot loop

__global__ __launch_bounds__(kThreads) void layout_finalize_kernel(
    int S, int K, int E, int P, int epr, int C, int ns, int32_t *__restrict__ rank_prefix,
    int32_t *__restrict__ expert_prefix, int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ num_tokens_per_expert, int32_t *__restrict__ rank_slot_base,
    int32_t *__restrict__ expert_slot_base, int32_t *__restrict__ slot_idx,
    int32_t *__restrict__ status, const int32_t *__restrict__ colexcl,
    const int32_t *__restrict__ bucket, const int32_t *__restrict__ chan, FinalizePlan fp) {
    extern __shared__ int32_t fin_lds[];
    int32_t *M = fin_lds;          // inclusive prefix of the row
    int32_t *R = fin_lds + C;      // raw counts; then plan starts per group
    int32_t *X = fin_lds + 2 * C;  // colexcl row
    __shared__ int32_t red[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nrank = (P + kWaves - 1) / kWaves;
    const int b = blockIdx.x;
    if (b < E * ns) {
        const int e = b / ns, sl = b - e * ns;
        for (int c = tid; c < C; c += kThreads) {
            const int x = colexcl[(int64_t)e * C + c];
            const int nx = e + 1 < E ? colexcl[(int64_t)(e + 1) * C + c] : chan[2 * c];
            X[c] = x;
            R[c] = nx - x;
        }
        __syncthreads();
        // inclusive scan of R: thread tid owns the contiguous stretch [tid * per, (tid + 1) * per)
        const int per = (C + kThreads - 1) / kThreads;
        const int c0 = tid * per, c1 = min(C, c0 + per);
        int seg = 0, xs = 0;
        for (int c = c0; c < c1; ++c) {
            seg += R[c];
            xs += X[c];
        }
        const int incl = wave_inclusive_scan(seg, lane);
        if (lane == 63) red[wave] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            before += w < wave ? red[w] : 0;
            total += red[w];
        }
        int run = before + incl - seg;
        for (int c = c0; c < c1; ++c) {
            run += R[c];
            M[c] = run;
        }
        // base = sum of X over the row
        int xsum = xs;
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) xsum += __shfl_xor(xsum, d, 64);
        __syncthreads();  // red reused below; M complete
        if (lane == 0) red[wave] = xsum;
        __syncthreads();
        int base = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) base += red[w];
        if (sl == 0) {
            int32_t *row = expert_prefix + (int64_t)e * C;
            for (int c = tid; c < C; c += kThreads) row[c] = M[c];
            if (tid == 0) {
                num_tokens_per_expert[e] = total;
                expert_slot_base[e] = base;
                if (e % epr == 0) rank_slot_base[e / epr] = base;
                if (e == E - 1) {
                    expert_slot_base[E] = base + total;
                    rank_slot_base[P] = base + total;
                }
            }
        }
        if (fp.plan) {  // R[g] <- plan start of group g: entries of lower experts in the group
            for (int g = tid; g < fp.ngroups; g += kThreads) {
                int sum = 0;
                const int ga = g * fp.cpc, gb = min(C, ga + fp.cpc);
                for (int c = ga; c < gb; ++c) sum += X[c];
                R[g] = sum;  // R is free once M is built (barrier above); groups <= C
            }
        }
        __syncthreads();
        const int cper = S / C, crem = S % C;
        const int chunk = (total + ns - 1) / ns;
        const int j0 = sl * chunk, j1 = min(total, j0 + chunk);
        for (int jb = j0; jb < j1; jb += kThreads * kFinUnroll) {
            int entry[kFinUnroll], pos[kFinUnroll], grp[kFinUnroll];
#pragma unroll
            for (int u = 0; u < kFinUnroll; ++u) {  // every bucket load before any store
                const int j = jb + u * kThreads + tid;
                entry[u] = -1;
                if (j < j1) {
                    int lo = 0, hi = C - 1;  // first channel with M[c] > j
                    while (lo < hi) {
                        const int mid = (lo + hi) >> 1;
                        if (M[mid] > j) hi = mid;
                        else lo = mid + 1;
                    }
                    const int c = lo;
                    const int mbefore = c > 0 ? M[c - 1] : 0;
                    const int local = j - mbefore;
                    const int tb = c * cper + (c < crem ? c : crem);
                    entry[u] = bucket[(int64_t)tb * K + X[c] + local];
                    if (fp.plan) {
                        const int g = c / fp.cpc;
                        const int ga = g * fp.cpc;
                        grp[u] = g;
                        pos[u] = R[g] + (mbefore - (ga > 0 ? M[ga - 1] : 0)) + local;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kFinUnroll; ++u) {
                if (entry[u] < 0) continue;
                const int slot = base + jb + u * kThreads + tid;
                slot_idx[entry[u]] = slot;
                if (fp.plan) {
                    const int t = entry[u] / K;
                    fp.plan[((int64_t)(grp[u] & 7) * fp.nsx + (grp[u] >> 3)) * fp.cap + pos[u]] =
                        int2{slot, (t << 4) | (entry[u] - t * K)};
                }
            }
        }
        return;
    }
    if (b < E * ns + nrank) {  // one wave per rank row, scanned in place
        const int r = (b - E * ns) * kWaves + wave;
        if (r >= P) return;
        int32_t *row = rank_prefix + (int64_t)r * C;
        int carry = 0;
        for (int j0 = 0; j0 < C; j0 += 64 * kScanRegs) {
            int v[kScanRegs];
#pragma unroll
            for (int u = 0; u < kScanRegs; ++u) {
                const int j = j0 + 64 * u + lane;
                v[u] = j < C ? row[j] : 0;
            }
#pragma unroll
            for (int u = 0; u < kScanRegs; ++u) {
                if (j0 + 64 * u < C) {
                    const int j = j0 + 64 * u + lane;
                    const int sc = wave_inclusive_scan(v[u], lane);
                    if (j < C) row[j] = sc + carry;
                    carry += __shfl(sc, 63, 64);
                }
            }
        }
        if (lane == 0) num_tokens_per_rank[r] = carry;
        return;
    }
    const int g = b - E * ns - nrank;
    if (g == 0) {
        int any = 0;
        for (int c = tid; c < C; c += kThreads) any |= chan[2 * c + 1];
        any = __syncthreads_or(any);
        if (tid == 0) *status = any ? 1 : 0;
    }
    if (!fp.plan) return;
    int count = 0;
    if (g < fp.ngroups) {
        const int ga = g * fp.cpc, gb = min(C, ga + fp.cpc);
        for (int c = ga + tid; c < gb; c += kThreads) count += chan[2 * c];
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) count += __shfl_xor(count, d, 64);
        if (lane == 0) red[wave] = count;
        __syncthreads();
        count = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) count += red[w];
    }
    int2 *out = fp.plan + ((int64_t)(g & 7) * fp.nsx + (g >> 3)) * fp.cap;
    for (int pidx = count + tid; pidx < fp.cap; pidx += kThreads) out[pidx] = int2{-1, 0};
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
    for (int j0 = 0; j0 < C; j0 += 64 * kScanRegs) {
        int v[kScanRegs];
#pragma unroll
        for (int u = 0; u < kScanRegs; ++u) {  // all loads of this stretch before any scan step
            const int j = j0 + 64 * u + lane;
            v[u] = j < C ? row[j] : 0;
        }
#pragma unroll
        for (int u = 0; u < kScanRegs; ++u) {
            if (j0 + 64 * u < C) {  // wave-uniform
                const int j = j0 + 64 * u + lane;
                const int s = wave_inclusive_scan(v[u], lane);
                if (j < C) row[j] = s + carry;
                carry += __shfl(s, 63, 64);
            }
        }
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
    int tb, te;
    channel_range(S, C, c, tb, te);
    const int64_t eb = (int64_t)tb * K, ee = (int64_t)te * K;

    // first batch of the channel's entries and their local ranks, loaded up front
    int e_cur = -1, local_cur = 0;
    if (eb + tid < ee) {
        e_cur = topk[eb + tid];
        local_cur = slot_idx[eb + tid];
    }

    // exclusive scan of the per-expert totals (last column); thread tid owns experts 2tid, 2tid+1
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

    bool bad = false;
    for (int64_t i = eb + tid; i < ee; i += kThreads) {
        const int e = e_cur, local = local_cur;
        if (i + kThreads < ee) {  // prefetch the next batch
            e_cur = topk[i + kThreads];
            local_cur = slot_idx[i + kThreads];
        }
        if (e >= 0 && e < E) {
            slot_idx[i] = off[e] + local;
        } else {
            slot_idx[i] = -1;
            bad = bad || e != -1;
        }
    }
    if (bad) atomicOr(status, 1);
}

// Value of v held by the first lane of this token whose rank equals r (lanes lk - J for J = 1..KP-1
// are the lower lanes of the same token; DPP reads them within the 16-lane row). Lanes that are
// themselves the first keep v. Called with every lane of the wave active.
template <int KP, int J = 1>
__device__ inline int first_lane_value(int v, int r, bool first, int lk, int found) {
    if constexpr (J >= KP) {
        return first ? v : found;
    } else {
        const int rj = __builtin_amdgcn_update_dpp(-2, r, 0x110 + J, 0xF, 0xF, false);
        const int vj = __builtin_amdgcn_update_dpp(0, v, 0x110 + J, 0xF, 0xF, false);
        const int fj = __builtin_amdgcn_update_dpp(0, first ? 1 : 0, 0x110 + J, 0xF, 0xF, false);
        const bool hit = (J <= lk) & (rj == r) & (fj != 0);
        return first_lane_value<KP, J + 1>(v, r, first, lk, hit ? vj : found);
    }
}

// Per-rank deduplicated rows ("Ascend DeepEP MoE Dispatch Optimization", sections "一条 token 如何走完
// MoE" and "所谓 compact plan 到底压缩了什么": one copy of a token per destination rank, grouped into
// one segment per rank). Rank r's segment starts at rank_token_base[r] (exclusive prefix of
// num_tokens_per_rank) and lists its tokens in ascending order, so token t's row on rank r is
//   rank_token_base[r] + rank_prefix[r][c-1] (tokens of r in earlier channels)
//                      + tokens of r earlier in channel c.
// One workgroup per channel, lanes over (token, k) as in the count kernel; the first lane of each
// (token, rank) gets its order from per-wave lane masks + popcount, and the token's other lanes on
// the same rank copy it with DPP. Workgroup 0 also writes rank_token_base.
template <int KP>
__global__ __launch_bounds__(kThreads) void rank_rows_kernel(
    const int32_t *__restrict__ topk, int S, int K, int E, int P, int epr, int C,
    const int32_t *__restrict__ rank_prefix, const int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ rank_row_idx, int32_t *__restrict__ rank_token_base) {
    constexpr int kTokWave = 64 / KP;
    constexpr int kTokBatch = kWaves * kTokWave;
    __shared__ int32_t rbase[MOE_MAX_RANKS];
    __shared__ int32_t rank_run[MOE_MAX_RANKS];
    __shared__ int32_t wave_sum[kWaves];
    __shared__ unsigned long long lane_mask[kWaves][MOE_MAX_RANKS];

    const int c = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tl = wave * kTokWave + lane / KP;
    const int lk = lane % KP;
    int tb, te;
    channel_range(S, C, c, tb, te);

    // segment starts: exclusive scan of num_tokens_per_rank, two ranks per lane (P <= 512)
    const int r0 = 2 * tid, r1 = 2 * tid + 1;
    const int n0 = r0 < P ? num_tokens_per_rank[r0] : 0;
    const int n1 = r1 < P ? num_tokens_per_rank[r1] : 0;
    const int pair = n0 + n1;
    const int incl = wave_inclusive_scan(pair, lane);
    if (lane == 63) wave_sum[wave] = incl;
    for (int r = tid; r < P; r += kThreads) {
        rank_run[r] = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) lane_mask[w][r] = 0ull;
    }
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        before += w < wave ? wave_sum[w] : 0;
        total += wave_sum[w];
    }
    const int b0 = before + incl - pair, b1 = b0 + n0;
    if (r0 < P) rbase[r0] = b0 + (c > 0 ? rank_prefix[(int64_t)r0 * C + c - 1] : 0);
    if (r1 < P) rbase[r1] = b1 + (c > 0 ? rank_prefix[(int64_t)r1 * C + c - 1] : 0);
    if (c == 0) {
        if (r0 < P) rank_token_base[r0] = b0;
        if (r1 < P) rank_token_base[r1] = b1;
        if (tid == 0) rank_token_base[P] = total;
    }

    const unsigned long long lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    auto fetch = [&](int t0) {
        const int t = t0 + tl;
        return (t < te && lk < K) ? topk[(int64_t)t * K + lk] : -1;
    };
    int next = fetch(tb);
    __syncthreads();
    for (int t0 = tb; t0 < te; t0 += kTokBatch) {
        const int v = next;
        next = fetch(t0 + kTokBatch);
        const int t = t0 + tl;
        const int r = (v >= 0 && v < E) ? v / epr : -1;
        const bool first = first_in_token<KP>(r, lk);
        if (first) atomicOr(&lane_mask[wave][r], 1ull << lane);
        __syncthreads();
        int order = 0, count = 0;
        bool leader = false;
        if (first) {
            int earlier = 0;
            for (int w = 0; w < wave; ++w) earlier += __popcll(lane_mask[w][r]);
            const int below = __popcll(lane_mask[wave][r] & lt_mask);
            order = rank_run[r] + earlier + below;
            leader = earlier == 0 && below == 0;  // first token of rank r in this batch
            if (leader)
                for (int w = 0; w < kWaves; ++w) count += __popcll(lane_mask[w][r]);
        }
        const int row = (r >= 0 ? rbase[r] : 0) + order;
        const int mine = first_lane_value<KP>(row, r, first, lk, 0);
        if (t < te && lk < K) rank_row_idx[(int64_t)t * K + lk] = r >= 0 ? mine : -1;
        __syncthreads();
        if (first) {
            if (leader) rank_run[r] += count;
            lane_mask[wave][r] = 0ull;
        }
        __syncthreads();
    }
}

template <int KP>
hipError_t launch_rank_rows_kp(const int32_t *topk_idx, int S, int K, int E, int P, int C,
                               const int32_t *rank_prefix, const int32_t *num_tokens_per_rank,
                               int32_t *rank_row_idx, int32_t *rank_token_base,
                               hipStream_t stream) {
    hipLaunchKernelGGL(rank_rows_kernel<KP>, dim3(C), dim3(kThreads), 0, stream, topk_idx, S, K, E,
                       P, E / P, C, rank_prefix, num_tokens_per_rank, rank_row_idx,
                       rank_token_base);
    return hipGetLastError();
}

template <int KP, bool WS>
hipError_t launch_count(const int32_t *topk_idx, int S, int K, int E, int P, int C,
                        uint8_t *is_in, int32_t *rank_prefix, int32_t *expert_prefix,
                        int32_t *slot_idx, int32_t *colexcl, int32_t *bucket, int32_t *chan,
                        hipStream_t stream) {
    hipLaunchKernelGGL((layout_count_kernel<KP, WS>), dim3(C), dim3(kThreads), 0, stream, topk_idx,
                       S, K, E, P, E / P, C, is_in, rank_prefix, expert_prefix, slot_idx, colexcl,
                       bucket, chan);
    return hipGetLastError();
}

template <bool WS>
hipError_t launch_count_k(const int32_t *topk_idx, int S, int K, int E, int P, int C,
                          uint8_t *is_in, int32_t *rank_prefix, int32_t *expert_prefix,
                          int32_t *slot_idx, int32_t *colexcl, int32_t *bucket, int32_t *chan,
                          hipStream_t stream) {
    if (K <= 1)
        return launch_count<1, WS>(topk_idx, S, K, E, P, C, is_in, rank_prefix, expert_prefix, slot_idx, colexcl, bucket, chan, stream);
    if (K <= 2)
        return launch_count<2, WS>(topk_idx, S, K, E, P, C, is_in, rank_prefix, expert_prefix, slot_idx, colexcl, bucket, chan, stream);
    if (K <= 4)
        return launch_count<4, WS>(topk_idx, S, K, E, P, C, is_in, rank_prefix, expert_prefix, slot_idx, colexcl, bucket, chan, stream);
    if (K <= 8)
        return launch_count<8, WS>(topk_idx, S, K, E, P, C, is_in, rank_prefix, expert_prefix, slot_idx, colexcl, bucket, chan, stream);
    return launch_count<16, WS>(topk_idx, S, K, E, P, C, is_in, rank_prefix, expert_prefix, slot_idx, colexcl, bucket, chan, stream);
}

}  // namespace


hipError_t launch_layout(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                         int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                         int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                         int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                         int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                         hipStream_t stream) {
    hipError_t err = launch_count_k<false>(topk_idx, S, K, E, P, C, is_token_in_rank,
                                           rank_prefix_matrix, expert_prefix_matrix, slot_idx,
                                           nullptr, nullptr, nullptr, stream);
    if (err != hipSuccess) return err;
    const int scan_blocks = (E + P + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(layout_scan_kernel, dim3(scan_blocks), dim3(kThreads), 0, stream,
                       expert_prefix_matrix, rank_prefix_matrix, E, P, C, status);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(layout_assign_kernel, dim3(C), dim3(kThreads), 0, stream, topk_idx, S, K, E,
                       P, E / P, C, expert_prefix_matrix, rank_prefix_matrix, slot_idx,
                       expert_slot_base, rank_slot_base, num_tokens_per_expert,
                       num_tokens_per_rank, status);
    return hipGetLastError();
}

hipError_t launch_layout_ws(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                            int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                            int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                            int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                            int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                            const LayoutWorkspace &ws, hipStream_t stream) {
    hipError_t err = launch_count_k<true>(topk_idx, S, K, E, P, C, is_token_in_rank,
                                          rank_prefix_matrix, expert_prefix_matrix, slot_idx,
                                          ws.colexcl, ws.bucket, ws.chan, stream);
    if (err != hipSuccess) return err;
    FinalizePlan fp{ws.plan, ws.chunks.cpc, ws.chunks.nsub, ws.chunks.nsx, ws.chunks.cap};
    const int nrank = (P + kWaves - 1) / kWaves;
    const int nextra = ws.plan ? 8 * ws.chunks.nsx : 1;
    // slices per expert: each re-reads two rows of C counts, so fewer when rows are long
    const int ns = C <= 256 ? 8 : (C <= 1024 ? 2 : 1);
    const size_t lds = (size_t)3 * C * sizeof(int32_t);
    hipLaunchKernelGGL(layout_finalize_kernel, dim3(E * ns + nrank + nextra), dim3(kThreads), lds, stream,
                       S, K, E, P, E / P, C, ns, rank_prefix_matrix, expert_prefix_matrix,
                       num_tokens_per_rank, num_tokens_per_expert, rank_slot_base, expert_slot_base,
                       slot_idx, status, ws.colexcl, ws.bucket, ws.chan, fp);
    return hipGetLastError();
}

hipError_t launch_rank_rows(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                            int32_t C, const int32_t *rank_prefix_matrix,
                            const int32_t *num_tokens_per_rank, int32_t *rank_row_idx,
                            int32_t *rank_token_base, hipStream_t stream) {
    if (K <= 1)
        return launch_rank_rows_kp<1>(topk_idx, S, K, E, P, C, rank_prefix_matrix, num_tokens_per_rank, rank_row_idx, rank_token_base, stream);
    if (K <= 2)
        return launch_rank_rows_kp<2>(topk_idx, S, K, E, P, C, rank_prefix_matrix, num_tokens_per_rank, rank_row_idx, rank_token_base, stream);
    if (K <= 4)
        return launch_rank_rows_kp<4>(topk_idx, S, K, E, P, C, rank_prefix_matrix, num_tokens_per_rank, rank_row_idx, rank_token_base, stream);
    if (K <= 8)
        return launch_rank_rows_kp<8>(topk_idx, S, K, E, P, C, rank_prefix_matrix, num_tokens_per_rank, rank_row_idx, rank_token_base, stream);
    return launch_rank_rows_kp<16>(topk_idx, S, K, E, P, C, rank_prefix_matrix, num_tokens_per_rank, rank_row_idx, rank_token_base, stream);
}

}  // namespace moe
