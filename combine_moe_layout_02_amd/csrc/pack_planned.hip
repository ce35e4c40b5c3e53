// Planned bf16 dispatch pack for gfx950: the same window bytes as pack_bf16_kernel, written in an
// order that HBM absorbs faster.
//
// The CAM pack ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.6 InputToShare) and the
// token-order pack in pack.hip write each token's K copies as soon as its row is read, so at any
// moment the writes in flight are spread over every expert's slot range of the window. Measured on
// MI355X at S=4096, H=7168, K=8, that scatter writes about 5 TB/s even with no reads at all.
// Here the window is written in slot order inside token chunks, with every row read by the XCD
// that later re-reads it:
//
//   plan  one workgroup per chunk of Tc = 2^lt tokens (Tc * K <= 1024 entries): the chunk's slot
//         numbers are bucketed by slot >> shift (at most 1024 buckets) with an LDS histogram and a
//         workgroup scan, and the (slot, token, k) records are written in bucket order to the
//         chunk's position in the list of the XCD that owns it (chunk c belongs to XCD c % 8).
//   pack  one 128-lane workgroup per (record, 2 KB part of the row), preceded by one workgroup per
//         2 KB part of each row of the XCD's chunks that only reads it. Workgroup b runs on XCD b % 8 (the
//         dispatcher hands out workgroups to the eight XCDs in turn), so each XCD first brings its
//         rows into its L2 and the memory-side cache, then stores its records in slot order:
//         consecutive workgroups write neighbouring slots, and the K re-reads of a row hit cache.
//
// moe_layout_ws can write the record lists itself (groups of whole channels instead of token chunks;
// the PackChunks argument says which), and the pack kernel then runs alone (moe_dispatch_planned).
//
// Measured at S=4096, H=7168, K=8 with x in HBM: 83 us for the pack kernel (and 3.4 us for the plan
// kernel when the layout does not write the lists), against 98 us for the token-order pack; at
// S=8192, P=128 with Zipf routing 170-187 us against 193 us. The pack kernel's prologue holds no runtime integer division (a 32-bit multiply-high
// replaces the division by the part count): with divisions the same kernel took 117 us, because
// the pack is bound by how fast workgroups turn over.
//
// The order inside a bucket depends on LDS atomics and is not deterministic, but every record
// carries its own slot and source, so the window bytes are: each (slot, part) is written exactly
// once, by one workgroup, with the same bytes as the token-order pack.

#include "pack_rows.h"

namespace moe {
namespace {

using namespace rows;

constexpr int kPlanThreads = 1024;  // plan entries per chunk (Tc * K) at most
constexpr int kPartLanes = 128;     // 16-byte vectors per pack workgroup (2 KB of a bf16 row)

// grid = 8 * nsx workgroups of kPlanThreads: chunk c = blockIdx.x (chunks past nsub write padding
// only). Record of entry e = t*K + k with slot s: (s, t << 4 | k); list position of chunk c:
// plan + (x * nsx + i) * Tc * K with x = c % 8, i = c / 8. After the chunk's valid records come
// (-1, 0) records up to Tc * K.
__global__ __launch_bounds__(kPlanThreads) void pack_plan_kernel(const int32_t *__restrict__ slot_idx,
                                                                 int S, int K, int lt, int nsx,
                                                                 int shift, int2 *__restrict__ plan) {
    __shared__ int32_t hist[kPlanThreads];
    __shared__ int32_t wave_sum[kPlanThreads / 64];
    const int c = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int TcK = K << lt;
    const int64_t t0 = (int64_t)c << lt;
    const int64_t t1 = t0 + (1 << lt) < S ? t0 + (1 << lt) : S;
    const int64_t n_ent = t1 > t0 ? (t1 - t0) * K : 0;
    const int64_t max_slots = (int64_t)S * K;
    const int64_t e0 = t0 * K;
    int s = -1;
    if (tid < n_ent) s = slot_idx[e0 + tid];
    const bool valid = s >= 0 && s < max_slots;
    hist[tid] = 0;
    __syncthreads();
    const int bucket = valid ? (s >> shift) : 0;  // < 1024: s < S*K <= 2^(shift + 10)
    int within = 0;
    if (valid) within = atomicAdd(&hist[bucket], 1);
    __syncthreads();
    // exclusive scan of the 1024 bucket counts: wave scans, then the wave totals
    const int h = hist[tid];
    int incl = h;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d, 64);
        if (lane >= d) incl += u;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / 64; ++w) {
        const int v = wave_sum[w];
        before += w < wave ? v : 0;
        total += v;
    }
    hist[tid] = before + incl - h;  // each thread rewrites only its own bucket
    __syncthreads();
    int2 *out = plan + ((int64_t)(c & 7) * nsx + (c >> 3)) * TcK;
    if (valid) {
        const int e = (int)(e0 + tid);
        const int t = e / K;
        out[hist[bucket] + within] = int2{s, (t << 4) | (e - t * K)};
    }
    if (tid >= total && tid < TcK) out[tid] = int2{-1, 0};
}

// grid = 8 * (nsx * 2^lt * nparts + nsx * cap * nparts) workgroups of kPartLanes. Workgroup b: XCD
// x = b % 8, index m = b / 8 in that XCD's sequence. m < nsx * 2^lt * nparts: with i = m / nparts
// and r = nsx * 2^lt - 1 - i, reads part m % nparts of token r & (2^lt - 1) of group 8(r >> lt) + x
// (if the group has that many) and stores nothing. Otherwise record (m - npf) / nparts of list x,
// part (m - npf) % nparts. The quotients are a multiply-high with np_magic = ceil(2^32 / nparts),
// exact for nparts in [2, 32] and indices below 2^24; nparts = 1 needs no division (its magic,
// 2^32, would not fit in 32 bits).
__global__ __launch_bounds__(kPartLanes) void pack_planned_kernel(
    const uint8_t *__restrict__ x, const int2 *__restrict__ plan, int S, int K, int nvec,
    int nparts, uint32_t np_magic, PackChunks pc, SlotGeom g, int src_rank,
    uint8_t *__restrict__ window) {
    const int b = blockIdx.x;
    const int xcd = b & 7;
    const int m = b >> 3;
    const int nrows = pc.nsx << pc.lt;
    const int npf = nrows * nparts;
    const int lane = threadIdx.x;
    const int row_bytes = nvec << 4;
    if (m < npf) {
        // one workgroup per (row, part); last group first, so that the first groups stored are the
        // ones fetched last (still in L2)
        const uint32_t row = nparts == 1 ? (uint32_t)m : __umulhi((uint32_t)m, np_magic);
        const int q = m - (int)row * nparts;
        const int mr = nrows - 1 - (int)row;
        const int c = ((mr >> pc.lt) << 3) + xcd;  // group
        const int tc0 = c * pc.a + min(c * pc.d, pc.b);
        const int tc1 = (c + 1) * pc.a + min((c + 1) * pc.d, pc.b);
        const int t = tc0 + (mr & ((1 << pc.lt) - 1));
        if (c >= pc.nsub || t >= tc1 || t >= S) return;
        const uint32_t v = load16(rsrc(x + (int64_t)t * row_bytes, row_bytes), (q * kPartLanes + lane) << 4).x;
        asm volatile("" ::"v"(v));  // keep the load: it exists to fill the caches
        return;
    }
    const uint32_t mp = (uint32_t)(m - npf);
    const uint32_t item = nparts == 1 ? mp : __umulhi(mp, np_magic);
    const int q = (int)(mp - item * (uint32_t)nparts);
    const int2 e = plan[(int64_t)xcd * pc.nsx * pc.cap + item];
    const int64_t s = e.x;
    if (s < 0 || s >= (int64_t)S * K) return;
    const int t = e.y >> 4, k = e.y & 15;
    if ((unsigned)t >= (unsigned)S || k >= K) return;  // a record of another table: never outside x
    const int v = q * kPartLanes + lane;
    const u32x4 val = load16(rsrc(x + (int64_t)t * row_bytes, row_bytes), v << 4);
    const __amdgpu_buffer_rsrc_t dst = rsrc(window + s * g.slot_bytes, g.tail_end);
    if (v < nvec) store16(val, dst, v << 4);
    if (q == nparts - 1 && lane < ((g.tail_end - g.payload_bytes) >> 4))
        store_tail(dst, g, lane, 0u, src_rank, t, k);
}

}  // namespace

hipError_t launch_pack_from_plan(const void *x, const void *plan, const PackChunks &pc, int32_t S,
                                 int32_t H, int32_t K, int32_t src_rank, void *window,
                                 hipStream_t stream) {
    const SlotGeom g = slot_geom(H, MOE_QUANT_NONE);
    const int nvec = H / 8;
    const int nparts = (nvec + kPartLanes - 1) / kPartLanes;
    const uint32_t magic = nparts > 1 ? (uint32_t)((0x100000000ull + nparts - 1) / nparts) : 0u;
    const int64_t nwg = 8 * (((int64_t)pc.nsx << pc.lt) * nparts + (int64_t)pc.nsx * pc.cap * nparts);
    hipLaunchKernelGGL(pack_planned_kernel, dim3((uint32_t)nwg), dim3(kPartLanes), 0, stream,
                       static_cast<const uint8_t *>(x), static_cast<const int2 *>(plan), S, K, nvec,
                       nparts, magic, pc, g, src_rank, static_cast<uint8_t *>(window));
    return hipGetLastError();
}

hipError_t launch_pack_planned(const void *x, const int32_t *slot_idx, int32_t S, int32_t H,
                               int32_t K, int32_t src_rank, void *window, void *workspace,
                               hipStream_t stream) {
    const PlanShape p = plan_shape(S, K);
    int2 *plan = static_cast<int2 *>(workspace);
    hipLaunchKernelGGL(pack_plan_kernel, dim3(8 * p.nsx), dim3(kPlanThreads), 0, stream, slot_idx, S,
                       K, p.lt, p.nsx, p.shift, plan);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_pack_from_plan(x, plan, token_chunks(S, K), S, H, K, src_rank, window, stream);
}

}  // namespace moe
