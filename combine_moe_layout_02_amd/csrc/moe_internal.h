// Internal declarations shared by the kernel translation units and the C ABI layer.
// Not part of the public interface (that is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"
#include "moe_probe.h"

namespace moe {

// Byte geometry of one window slot; see moe_slot_offsets in moe.h.
struct SlotGeom {
    int64_t slot_bytes;
    int32_t payload_bytes;
    int32_t scale_off;
    int32_t triple_off;
    int32_t tail_end;
};

constexpr int64_t ceil_to(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

inline bool valid_quant(int32_t quant) {
    return quant == MOE_QUANT_NONE || quant == MOE_QUANT_FP8_E4M3_DYN || quant == MOE_QUANT_INT8_DYN;
}

inline SlotGeom slot_geom(int32_t H, int32_t quant) {
    SlotGeom g;
    g.slot_bytes = ceil_to(ceil_to(2 * (int64_t)H, 32) + 44, 512);
    g.payload_bytes = quant == MOE_QUANT_NONE ? 2 * H : H;
    g.scale_off = (int32_t)ceil_to(g.payload_bytes, 32);
    g.triple_off = g.scale_off + 32;
    int64_t tail = ceil_to(g.triple_off + 12, 128);
    g.tail_end = (int32_t)(tail < g.slot_bytes ? tail : g.slot_bytes);
    return g;
}

// Limits of the single-launch layout for small routing tables (its LDS tables are sized by them).
constexpr int kSmallLayoutEntries = 4096;   // S * K
constexpr int kSmallLayoutChannels = 1024;  // C

// The argument checks moe_dispatch, moe_dispatch_ws and moe_dispatch_noalloc share (MOE_OK or a
// negative moe_status; no HIP call).
int check_dispatch(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                   int32_t quant, const void *window, int64_t window_bytes);

// True when the single-launch layout can take (S, K, E, P, C).
bool layout_small_fits(int32_t S, int32_t K, int32_t E, int32_t P, int32_t C);

// Launchers: enqueue on `stream`, return hipSuccess or the launch error.

// The multi-launch layout (count per channel, scan along channels, assign), any accepted size.
hipError_t launch_layout(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                         int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                         int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                         int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                         int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                         hipStream_t stream);

hipError_t launch_layout_small(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                               int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                               int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                               int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                               int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                               hipStream_t stream);

// Layout and pack of a small table (layout_small_fits) in one launch; same outputs as
// launch_layout_small followed by launch_pack.
hipError_t launch_layout_dispatch_small(
    const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
    uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
    int32_t *rank_prefix_matrix, int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
    int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status, const void *x, int32_t H,
    int32_t quant, int32_t src_rank, void *window, hipStream_t stream);

hipError_t launch_rank_rows(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                            int32_t C, const int32_t *rank_prefix_matrix,
                            const int32_t *num_tokens_per_rank, int32_t *rank_row_idx,
                            int32_t *rank_token_base, hipStream_t stream);

hipError_t launch_pack_dedup(const void *x, const int32_t *rank_row_idx, const int32_t *topk_idx,
                             int32_t S, int32_t H, int32_t K, int32_t E, int32_t P, int32_t quant,
                             int32_t src_rank, void *window, hipStream_t stream);

hipError_t launch_expand_dedup(const void *window, const int32_t *rank_row_idx,
                               const int32_t *slot_idx, const int32_t *num_slots, int32_t S,
                               int32_t K, int32_t P, int32_t H, int32_t quant, void *expand_x,
                               float *expand_scales, int32_t *expand_idx, hipStream_t stream);

hipError_t launch_pack(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                       int32_t quant, int32_t src_rank, void *window, hipStream_t stream);

// The planned bf16 pack (pack_planned.hip) runs for tables of at least this many entries; smaller
// tables and the quantised modes take the token-order pack of launch_pack.
constexpr int64_t kPlannedMinEntries = 8192;

// Shape of the planned pack's work: token chunks of Tc = 2^lt tokens (the largest power of two with
// Tc * K <= 1024), chunk c owned by XCD c % 8, each XCD's list holding nsx chunks of Tc * K
// records; slots are bucketed by slot >> shift (at most 1024 buckets).
struct PlanShape {
    int lt;
    int nsub;
    int nsx;
    int shift;
};

inline PlanShape plan_shape(int32_t S, int32_t K) {
    PlanShape p;
    int lk = 0;
    while ((1 << lk) < K) ++lk;
    p.lt = 10 - lk;
    const int Tc = 1 << p.lt;
    p.nsub = (S + Tc - 1) / Tc;
    p.nsx = (p.nsub + 7) / 8;
    int bits = 0;
    while ((int64_t(1) << bits) < (int64_t)S * K) ++bits;
    p.shift = bits > 10 ? bits - 10 : 0;
    return p;
}

// True when moe_dispatch_ws takes the planned pack for (S, K, quant).
inline bool pack_planned_used(int32_t S, int32_t K, int32_t quant) {
    return quant == MOE_QUANT_NONE && (int64_t)S * K >= kPlannedMinEntries;
}

// Workspace bytes of the planned pack's record lists (8 bytes per record) for (S, K).
inline int64_t pack_plan_bytes(int32_t S, int32_t K) {
    const PlanShape p = plan_shape(S, K);
    return (int64_t)8 * p.nsx * ((int64_t)K << p.lt) * 8;
}

// Plan kernel + planned pack kernel; workspace holds pack_plan_bytes(S, K) bytes, 16-byte aligned.
hipError_t launch_pack_planned(const void *x, const int32_t *slot_idx, int32_t S, int32_t H,
                               int32_t K, int32_t src_rank, void *window, void *workspace,
                               hipStream_t stream);

// How the planned pack's record lists map to tokens: group g covers tokens
// [g*a + min(g*d, b), (g+1)*a + min((g+1)*d, b)) and belongs to XCD g % 8, whose list holds nsx
// groups of cap records; every group has at most 2^lt tokens. Token chunks of the plan kernel are
// (a, d, b) = (Tc, 0, 0); groups of cpc channels of the layout are (cpc*(S/C), cpc, S%C).
struct PackChunks {
    int lt, nsub, nsx, cap, a, d, b, cpc;
};

inline PackChunks token_chunks(int32_t S, int32_t K) {
    const PlanShape p = plan_shape(S, K);
    return PackChunks{p.lt, p.nsub, p.nsx, K << p.lt, 1 << p.lt, 0, 0, 0};
}

// Groups of whole channels for a plan written by the layout itself: possible when a channel holds
// at most 1024 entries (ceil(S/C) * K <= 1024); cpc = 1024 / (ceil(S/C) * K) channels per group.
inline bool channel_chunks(int32_t S, int32_t K, int32_t C, PackChunks *pc) {
    const int per = S / C, rem = S % C;
    const int maxchan = per + (rem > 0 ? 1 : 0);
    if ((int64_t)maxchan * K > 1024) return false;
    const int cpc = 1024 / (maxchan * K);
    const int ngroups = (C + cpc - 1) / cpc;
    int lt = 0;
    while ((1 << lt) < cpc * maxchan) ++lt;
    *pc = PackChunks{lt, ngroups, (ngroups + 7) / 8, 1024, cpc * per, cpc, rem, cpc};
    return true;
}

inline int64_t chunk_plan_bytes(const PackChunks &pc) { return (int64_t)8 * pc.nsx * pc.cap * 8; }

// The planned pack kernel alone, from record lists already in `plan` laid out by `pc`.
hipError_t launch_pack_from_plan(const void *x, const void *plan, const PackChunks &pc, int32_t S,
                                 int32_t H, int32_t K, int32_t src_rank, void *window,
                                 hipStream_t stream);

// Scratch of the two-launch layout (moe_layout_dispatch_ws): colexcl int32 [E, C], bucket int32
// [S*K], chan int32 [2C], and, when plan is not null, the pack plan laid out by chunks.
struct LayoutWorkspace {
    int32_t *colexcl;
    int32_t *bucket;
    int32_t *chan;
    int2 *plan;
    PackChunks chunks;
};

// Count kernel (workspace form) + finalize kernel: the outputs of launch_layout, and the pack plan
// when ws.plan is set (ws.chunks from channel_chunks).
hipError_t launch_layout_ws(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                            int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                            int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                            int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                            int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                            const LayoutWorkspace &ws, hipStream_t stream);

hipError_t launch_combine(const void *expert_out, int64_t row_stride_bytes, int64_t expert_rows,
                          const int32_t *slot_idx, const float *topk_weights, int32_t S,
                          int32_t H, int32_t K, void *y, hipStream_t stream);

hipError_t launch_combine_scatter(const void *expert_out, int64_t row_stride_bytes,
                                  int64_t expert_rows, const int32_t *expand_idx,
                                  const int32_t *num_rows, int32_t S, int32_t K, int32_t H,
                                  void *staging, int64_t staging_stride_bytes, hipStream_t stream);

hipError_t launch_combine_staged(const void *staging, int64_t staging_stride_bytes,
                                 const int32_t *slot_idx, const float *topk_weights, int32_t S,
                                 int32_t H, int32_t K, void *y, hipStream_t stream);

hipError_t launch_unpack_padded(const void *window, const int32_t *expert_slot_base, int32_t E,
                                int32_t S, int32_t K, int32_t H, int32_t quant,
                                int32_t expert_alignment, int64_t out_rows, void *expand_x,
                                float *expand_scales, int32_t *expand_idx,
                                int32_t *expert_row_base, int32_t *status, hipStream_t stream);

hipError_t launch_unpack(const void *window, const int32_t *num_slots, int32_t S, int32_t K,
                         int32_t H, int32_t quant, void *expand_x, float *expand_scales,
                         int32_t *expand_idx, hipStream_t stream);

}  // namespace moe
