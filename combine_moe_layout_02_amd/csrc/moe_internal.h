// Internal declarations shared by the kernel translation units and the C ABI layer.
// Not part of the public interface (that is include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

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
