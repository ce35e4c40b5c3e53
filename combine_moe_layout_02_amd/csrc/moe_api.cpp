// C ABI of the library (declared in include/moe.h): host-side validation, then kernel launches.
//
// Every check runs before the first HIP call, so a rejected call enqueues nothing and touches no
// device state. This mirrors the host tiling step of the CAM operators, which validates shapes and
// the window size before launching ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 8.2, whose
// "HCCL_BUFFSIZE too SMALL" error becomes MOE_ERR_WINDOW), and the required-input errors of the
// DeepEP Python entry ("Ascend DeepEP MoE Dispatch Optimization", section "从 Python 接口进入真实调用链").

#include <stdint.h>
#include <string.h>

#include <cstring>
#include <type_traits>

#include "moe_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_hidden(int32_t H) {
    if (H < 16 || H > MOE_MAX_HIDDEN) return MOE_ERR_ARG;
    if (H % 16 != 0) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int check_tokens(int32_t S, int32_t K) {
    if (S < 1 || K < 1 || K > MOE_MAX_K) return MOE_ERR_ARG;
    if (S > MOE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// True when rows [0, rows) at `stride` bytes apart have byte offsets an int64 can hold (rows * stride
// <= INT64_MAX), so the kernels' row addresses cannot wrap.
bool extent_fits(int64_t rows, int64_t stride) {
    return rows <= 1 || stride <= INT64_MAX / rows;
}

// Which layout form a call takes: -1 for a path value outside moe_layout_path, 1 for the
// single-launch form, 0 for the multi-launch form. MOE_LAYOUT_SINGLE on a table the single launch
// cannot take is reported as MOE_ERR_UNSUPPORTED by the caller (returned here as 2).
int pick_layout(int32_t path, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C) {
    const bool fits = moe::layout_small_fits(S, K, E, P, C);
    switch (path) {
        case MOE_LAYOUT_AUTO: return fits ? 1 : 0;
        case MOE_LAYOUT_MULTI: return 0;
        case MOE_LAYOUT_SINGLE: return fits ? 1 : 2;
        default: return -1;
    }
}

int check_experts(int32_t E, int32_t P) {
    if (E < 1 || E > MOE_MAX_EXPERTS || P < 1 || P > MOE_MAX_RANKS) return MOE_ERR_ARG;
    if (E % P != 0) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

namespace moe {

int check_dispatch(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                   int32_t quant, const void *window, int64_t window_bytes) {
    if (!x || !slot_idx || !window) return MOE_ERR_ARG;
    int st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    st = check_hidden(H);
    if (st != MOE_OK) return st;
    if (!valid_quant(quant)) return MOE_ERR_ARG;
    if (!aligned(x, 16) || !aligned(slot_idx, 4) || !aligned(window, 512)) return MOE_ERR_ALIGN;
    if (window_bytes < moe_window_bytes(S, K, H)) return MOE_ERR_WINDOW;
    return MOE_OK;
}

bool layout_small_fits(int32_t S, int32_t K, int32_t E, int32_t P, int32_t C) {
    (void)E;
    (void)P;
    return (int64_t)S * K <= kSmallLayoutEntries && C <= kSmallLayoutChannels;
}

}  // namespace moe

namespace {

// Arguments of one call, as validated by its check_* function; run_* launches them unchecked.
struct LayoutArgs {
    const int32_t *topk_idx;
    int32_t S, K, E, P, C;
    uint8_t *is_token_in_rank;
    int32_t *num_tokens_per_rank, *num_tokens_per_expert, *rank_prefix_matrix,
        *expert_prefix_matrix, *rank_slot_base, *expert_slot_base, *slot_idx, *status;
    int32_t form;  // 1 = single launch, 0 = multi-launch (set by check_layout)
};

struct DispatchArgs {
    const void *x;
    const int32_t *slot_idx;
    int32_t S, H, K, quant, src_rank;
    void *window;
    void *workspace;
    bool planned;  // set by check_dispatch_ws
};

struct LayoutDispatchArgs {
    LayoutArgs layout;
    const void *x;
    int32_t H, quant, src_rank;
    void *window;
};

struct CombineArgs {
    const void *expert_out;
    int64_t row_stride_bytes, expert_rows;
    const int32_t *slot_idx;
    const float *topk_weights;
    int32_t S, H, K;
    void *y;
};

// The layout checks shared by moe_layout_ex and moe_layout_dispatch_ex; sets a.form.
int check_layout(LayoutArgs &a, int32_t path) {
    if (!a.topk_idx || !a.is_token_in_rank || !a.num_tokens_per_rank || !a.num_tokens_per_expert ||
        !a.rank_prefix_matrix || !a.expert_prefix_matrix || !a.rank_slot_base ||
        !a.expert_slot_base || !a.slot_idx || !a.status)
        return MOE_ERR_ARG;
    int st = check_tokens(a.S, a.K);
    if (st != MOE_OK) return st;
    if (a.E < 1 || a.E > MOE_MAX_EXPERTS || a.P < 1 || a.P > MOE_MAX_RANKS) return MOE_ERR_ARG;
    if (a.C < 1 || a.C > a.S || a.C > MOE_MAX_CHANNELS) return MOE_ERR_ARG;
    if (a.E % a.P != 0) return MOE_ERR_UNSUPPORTED;
    const int form = pick_layout(path, a.S, a.K, a.E, a.P, a.C);
    if (form < 0) return MOE_ERR_ARG;
    if (form == 2) return MOE_ERR_UNSUPPORTED;
    const void *i32[] = {a.topk_idx, a.num_tokens_per_rank, a.num_tokens_per_expert,
                         a.rank_prefix_matrix, a.expert_prefix_matrix, a.rank_slot_base,
                         a.expert_slot_base, a.slot_idx, a.status};
    for (const void *p : i32)
        if (!aligned(p, 4)) return MOE_ERR_ALIGN;
    a.form = form;
    return MOE_OK;
}

int run_layout(const LayoutArgs &a, hipStream_t stream) {
    if (a.form == 1)
        return from_hip(moe::launch_layout_small(
            a.topk_idx, a.S, a.K, a.E, a.P, a.C, a.is_token_in_rank, a.num_tokens_per_rank,
            a.num_tokens_per_expert, a.rank_prefix_matrix, a.expert_prefix_matrix,
            a.rank_slot_base, a.expert_slot_base, a.slot_idx, a.status, stream));
    return from_hip(moe::launch_layout(a.topk_idx, a.S, a.K, a.E, a.P, a.C, a.is_token_in_rank,
                                       a.num_tokens_per_rank, a.num_tokens_per_expert,
                                       a.rank_prefix_matrix, a.expert_prefix_matrix,
                                       a.rank_slot_base, a.expert_slot_base, a.slot_idx, a.status,
                                       stream));
}

int check_dispatch_ws(DispatchArgs &a, int64_t window_bytes, int64_t workspace_bytes) {
    const int st = moe::check_dispatch(a.x, a.slot_idx, a.S, a.H, a.K, a.quant, a.window,
                                       window_bytes);
    if (st != MOE_OK) return st;
    const bool planned = moe::pack_planned_used(a.S, a.K, a.quant);
    if (planned && !a.workspace) return MOE_ERR_ARG;
    if (planned && !aligned(a.workspace, 16)) return MOE_ERR_ALIGN;
    if (planned && workspace_bytes < moe::pack_plan_bytes(a.S, a.K)) return MOE_ERR_WINDOW;
    a.planned = planned;
    return MOE_OK;
}

int run_dispatch_ws(const DispatchArgs &a, hipStream_t stream) {
    if (a.planned)
        return from_hip(moe::launch_pack_planned(a.x, a.slot_idx, a.S, a.H, a.K, a.src_rank,
                                                 a.window, a.workspace, stream));
    return from_hip(moe::launch_pack(a.x, a.slot_idx, a.S, a.H, a.K, a.quant, a.src_rank,
                                     a.window, stream));
}

int check_layout_dispatch(LayoutDispatchArgs &a, int32_t path, int64_t window_bytes) {
    if (!a.x || !a.window) return MOE_ERR_ARG;
    int st = check_layout(a.layout, path);
    if (st != MOE_OK) return st;
    st = check_hidden(a.H);
    if (st != MOE_OK) return st;
    if (!moe::valid_quant(a.quant)) return MOE_ERR_ARG;
    if (!aligned(a.x, 16) || !aligned(a.window, 512)) return MOE_ERR_ALIGN;
    if (window_bytes < moe_window_bytes(a.layout.S, a.layout.K, a.H)) return MOE_ERR_WINDOW;
    return MOE_OK;
}

int run_layout_dispatch(const LayoutDispatchArgs &a, hipStream_t stream) {
    const LayoutArgs &l = a.layout;
    if (l.form == 1)
        return from_hip(moe::launch_layout_dispatch_small(
            l.topk_idx, l.S, l.K, l.E, l.P, l.C, l.is_token_in_rank, l.num_tokens_per_rank,
            l.num_tokens_per_expert, l.rank_prefix_matrix, l.expert_prefix_matrix,
            l.rank_slot_base, l.expert_slot_base, l.slot_idx, l.status, a.x, a.H, a.quant,
            a.src_rank, a.window, stream));
    const int st = run_layout(l, stream);
    if (st != MOE_OK) return st;
    return from_hip(moe::launch_pack(a.x, l.slot_idx, l.S, a.H, l.K, a.quant, a.src_rank,
                                     a.window, stream));
}

int check_combine(const CombineArgs &a) {
    if (!a.expert_out || !a.slot_idx || !a.topk_weights || !a.y) return MOE_ERR_ARG;
    int st = check_tokens(a.S, a.K);
    if (st != MOE_OK) return st;
    st = check_hidden(a.H);
    if (st != MOE_OK) return st;
    if (a.expert_rows < 0 || a.row_stride_bytes < 2 * (int64_t)a.H) return MOE_ERR_ARG;
    if (!extent_fits(a.expert_rows, a.row_stride_bytes)) return MOE_ERR_ARG;
    if (a.row_stride_bytes % 16 != 0 || !aligned(a.expert_out, 16) || !aligned(a.y, 16) ||
        !aligned(a.slot_idx, 4) || !aligned(a.topk_weights, 4))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

int run_combine(const CombineArgs &a, hipStream_t stream) {
    return from_hip(moe::launch_combine(a.expert_out, a.row_stride_bytes, a.expert_rows,
                                        a.slot_idx, a.topk_weights, a.S, a.H, a.K, a.y, stream));
}

// The workspace of moe_layout_ws / moe_dispatch_planned / moe_layout_dispatch_ws: the pack plan
// first (its size depends on S, K, C and quant only, so the dispatch can find it without E), then the
// layout's scratch. Byte offsets; every part 256-aligned.
struct LayoutWsShape {
    int64_t plan_bytes, colexcl, bucket, chan, total;
    int planned;   // 0: token-order pack; 1: plan written by the layout; 2: separate plan kernel
    moe::PackChunks chunks;
};

int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

LayoutWsShape plan_part(int32_t S, int32_t K, int32_t C, int32_t quant) {
    LayoutWsShape w{};
    if (moe::pack_planned_used(S, K, quant)) {
        if (moe::channel_chunks(S, K, C, &w.chunks)) {
            w.planned = 1;
            w.plan_bytes = moe::chunk_plan_bytes(w.chunks);
        } else {
            w.planned = 2;
            w.plan_bytes = moe::pack_plan_bytes(S, K);
        }
    }
    w.total = w.plan_bytes;
    return w;
}

LayoutWsShape layout_ws_shape(int32_t S, int32_t K, int32_t E, int32_t C, int32_t quant) {
    LayoutWsShape w = plan_part(S, K, C, quant);
    w.colexcl = align256(w.plan_bytes);
    w.bucket = w.colexcl + align256((int64_t)E * C * 4);
    w.chan = w.bucket + align256((int64_t)S * K * 4);
    w.total = w.chan + (int64_t)2 * C * 4;
    return w;
}

// Checks of moe_layout_ws on top of check_layout (sets a.form): quant and, for the two-launch form,
// the workspace.
int check_layout_ws(LayoutArgs &a, int32_t path, int32_t quant, const void *workspace,
                    int64_t workspace_bytes) {
    int st = check_layout(a, path);
    if (st != MOE_OK) return st;
    if (!moe::valid_quant(quant)) return MOE_ERR_ARG;
    if (a.form == 1) return MOE_OK;
    if (!workspace) return MOE_ERR_ARG;
    if (!aligned(workspace, 16)) return MOE_ERR_ALIGN;
    if (workspace_bytes < layout_ws_shape(a.S, a.K, a.E, a.C, quant).total) return MOE_ERR_WINDOW;
    return MOE_OK;
}

int run_layout_ws(const LayoutArgs &a, int32_t quant, void *workspace, hipStream_t stream) {
    if (a.form == 1) return run_layout(a, stream);
    const LayoutWsShape w = layout_ws_shape(a.S, a.K, a.E, a.C, quant);
    uint8_t *base = static_cast<uint8_t *>(workspace);
    const moe::LayoutWorkspace lw{reinterpret_cast<int32_t *>(base + w.colexcl),
                                  reinterpret_cast<int32_t *>(base + w.bucket),
                                  reinterpret_cast<int32_t *>(base + w.chan),
                                  w.planned == 1 ? reinterpret_cast<int2 *>(base) : nullptr, w.chunks};
    return from_hip(moe::launch_layout_ws(a.topk_idx, a.S, a.K, a.E, a.P, a.C, a.is_token_in_rank,
                                          a.num_tokens_per_rank, a.num_tokens_per_expert,
                                          a.rank_prefix_matrix, a.expert_prefix_matrix,
                                          a.rank_slot_base, a.expert_slot_base, a.slot_idx,
                                          a.status, lw, stream));
}

int check_dispatch_planned(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                           int32_t C, int32_t quant, const void *window, int64_t window_bytes,
                           const void *workspace, int64_t workspace_bytes) {
    const int st = moe::check_dispatch(x, slot_idx, S, H, K, quant, window, window_bytes);
    if (st != MOE_OK) return st;
    if (C < 1 || C > S || C > MOE_MAX_CHANNELS) return MOE_ERR_ARG;
    const LayoutWsShape w = plan_part(S, K, C, quant);
    if (w.planned == 0) return MOE_OK;
    if (!workspace) return MOE_ERR_ARG;
    if (!aligned(workspace, 16)) return MOE_ERR_ALIGN;
    if (workspace_bytes < w.plan_bytes) return MOE_ERR_WINDOW;
    return MOE_OK;
}

int run_dispatch_planned(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                         int32_t C, int32_t quant, int32_t src_rank, void *window, void *workspace,
                         hipStream_t stream) {
    const LayoutWsShape w = plan_part(S, K, C, quant);
    if (w.planned == 1)
        return from_hip(moe::launch_pack_from_plan(x, workspace, w.chunks, S, H, K, src_rank, window,
                                                   stream));
    if (w.planned == 2)
        return from_hip(moe::launch_pack_planned(x, slot_idx, S, H, K, src_rank, window, workspace,
                                                 stream));
    return from_hip(moe::launch_pack(x, slot_idx, S, H, K, quant, src_rank, window, stream));
}

struct LayoutWsArgs {
    LayoutArgs layout;
    int32_t quant;
    void *workspace;
};

struct DispatchPlannedArgs {
    const void *x;
    const int32_t *slot_idx;
    int32_t S, H, K, C, quant, src_rank;
    void *window;
    void *workspace;
};

// What a moe_plan holds: a tag, the call kind and its checked arguments.
struct PlanRecord {
    static constexpr uint64_t kMagic = 0x6d6f65706c616e31ull;  // "moeplan1"
    enum Kind : int32_t {
        kNone = 0, kLayout = 1, kDispatch = 2, kLayoutDispatch = 3, kCombine = 4, kLayoutWs = 5,
        kDispatchPlanned = 6
    };
    uint64_t magic;
    Kind kind;
    union {
        LayoutArgs layout;
        DispatchArgs dispatch;
        LayoutDispatchArgs layout_dispatch;
        CombineArgs combine;
        LayoutWsArgs layout_ws;
        DispatchPlannedArgs dispatch_planned;
    };
};
static_assert(sizeof(PlanRecord) <= sizeof(moe_plan), "moe_plan is too small for a plan record");
static_assert(std::is_trivially_copyable<PlanRecord>::value, "plan records are copied as bytes");

// Stores rec in plan when st is MOE_OK; otherwise clears the plan (moe_plan_run then refuses it).
int store_plan(moe_plan *plan, PlanRecord &rec, int st) {
    std::memset(plan, 0, sizeof(*plan));
    if (st != MOE_OK) return st;
    rec.magic = PlanRecord::kMagic;
    std::memcpy(plan, &rec, sizeof(rec));
    return MOE_OK;
}

}  // namespace

extern "C" {

int64_t moe_slot_bytes(int32_t H) {
    const int st = check_hidden(H);
    if (st != MOE_OK) return st;
    return moe::slot_geom(H, MOE_QUANT_NONE).slot_bytes;
}

int64_t moe_window_bytes(int32_t S, int32_t K, int32_t H) {
    int st = check_hidden(H);
    if (st != MOE_OK) return st;
    st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    return (int64_t)S * K * moe::slot_geom(H, MOE_QUANT_NONE).slot_bytes;
}

int64_t moe_dedup_window_bytes(int32_t S, int32_t K, int32_t P, int32_t H) {
    int st = check_hidden(H);
    if (st != MOE_OK) return st;
    st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    if (P < 1 || P > MOE_MAX_RANKS) return MOE_ERR_ARG;
    return (int64_t)S * (K < P ? K : P) * moe::slot_geom(H, MOE_QUANT_NONE).slot_bytes;
}

int moe_slot_offsets(int32_t H, int32_t quant, int64_t *payload_bytes, int64_t *scale_off,
                     int64_t *triple_off, int64_t *tail_end) {
    const int st = check_hidden(H);
    if (st != MOE_OK) return st;
    if (!moe::valid_quant(quant)) return MOE_ERR_ARG;
    const moe::SlotGeom g = moe::slot_geom(H, quant);
    if (payload_bytes) *payload_bytes = g.payload_bytes;
    if (scale_off) *scale_off = g.scale_off;
    if (triple_off) *triple_off = g.triple_off;
    if (tail_end) *tail_end = g.tail_end;
    return MOE_OK;
}

int moe_layout_ex(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
                  uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                  int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                  int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                  int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status, int32_t path,
                  hipStream_t stream) {
    LayoutArgs a{topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank,
                 num_tokens_per_expert, rank_prefix_matrix, expert_prefix_matrix, rank_slot_base,
                 expert_slot_base, slot_idx, status, 0};
    const int st = check_layout(a, path);
    return st != MOE_OK ? st : run_layout(a, stream);
}

int moe_layout(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
               uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
               int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
               int32_t *expert_prefix_matrix, int32_t *rank_slot_base, int32_t *expert_slot_base,
               int32_t *slot_idx, int32_t *status, hipStream_t stream) {
    return moe_layout_ex(topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank,
                         num_tokens_per_expert, rank_prefix_matrix, expert_prefix_matrix,
                         rank_slot_base, expert_slot_base, slot_idx, status, MOE_LAYOUT_AUTO,
                         stream);
}

int moe_dispatch(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                 int32_t quant, int32_t src_rank, void *window, int64_t window_bytes,
                 hipStream_t stream) {
    const int st = moe::check_dispatch(x, slot_idx, S, H, K, quant, window, window_bytes);
    if (st != MOE_OK) return st;
    return from_hip(moe::launch_pack(x, slot_idx, S, H, K, quant, src_rank, window, stream));
}

int64_t moe_dispatch_workspace_bytes(int32_t S, int32_t K, int32_t quant) {
    const int st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    if (!moe::valid_quant(quant)) return MOE_ERR_ARG;
    return moe::pack_planned_used(S, K, quant) ? moe::pack_plan_bytes(S, K) : 0;
}

int moe_dispatch_ws(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                    int32_t quant, int32_t src_rank, void *window, int64_t window_bytes,
                    void *workspace, int64_t workspace_bytes, hipStream_t stream) {
    DispatchArgs a{x, slot_idx, S, H, K, quant, src_rank, window, workspace, false};
    const int st = check_dispatch_ws(a, window_bytes, workspace_bytes);
    return st != MOE_OK ? st : run_dispatch_ws(a, stream);
}

int moe_layout_dispatch_ex(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                           int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                           int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                           int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                           int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                           const void *x, int32_t H, int32_t quant, int32_t src_rank, void *window,
                           int64_t window_bytes, int32_t path, hipStream_t stream) {
    LayoutDispatchArgs a{{topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank,
                          num_tokens_per_expert, rank_prefix_matrix, expert_prefix_matrix,
                          rank_slot_base, expert_slot_base, slot_idx, status, 0},
                         x, H, quant, src_rank, window};
    const int st = check_layout_dispatch(a, path, window_bytes);
    return st != MOE_OK ? st : run_layout_dispatch(a, stream);
}

int moe_layout_dispatch(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                        int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                        int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                        int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                        int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                        const void *x, int32_t H, int32_t quant, int32_t src_rank, void *window,
                        int64_t window_bytes, hipStream_t stream) {
    return moe_layout_dispatch_ex(topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank,
                                  num_tokens_per_expert, rank_prefix_matrix, expert_prefix_matrix,
                                  rank_slot_base, expert_slot_base, slot_idx, status, x, H, quant,
                                  src_rank, window, window_bytes, MOE_LAYOUT_AUTO, stream);
}

int64_t moe_layout_dispatch_workspace_bytes(int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
                                             int32_t quant, int32_t path) {
    int st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    st = check_experts(E, P);
    if (st != MOE_OK) return st;
    if (C < 1 || C > S || C > MOE_MAX_CHANNELS) return MOE_ERR_ARG;
    if (!moe::valid_quant(quant)) return MOE_ERR_ARG;
    const int form = pick_layout(path, S, K, E, P, C);
    if (form < 0) return MOE_ERR_ARG;
    if (form == 2) return MOE_ERR_UNSUPPORTED;
    return form == 1 ? 0 : layout_ws_shape(S, K, E, C, quant).total;
}

int moe_layout_ws(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
                  uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                  int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                  int32_t *expert_prefix_matrix, int32_t *rank_slot_base, int32_t *expert_slot_base,
                  int32_t *slot_idx, int32_t *status, int32_t quant, int32_t path, void *workspace,
                  int64_t workspace_bytes, hipStream_t stream) {
    LayoutArgs a{topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank,
                 num_tokens_per_expert, rank_prefix_matrix, expert_prefix_matrix, rank_slot_base,
                 expert_slot_base, slot_idx, status, 0};
    const int st = check_layout_ws(a, path, quant, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    return run_layout_ws(a, quant, workspace, stream);
}

int moe_dispatch_planned(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                         int32_t C, int32_t quant, int32_t src_rank, void *window,
                         int64_t window_bytes, void *workspace, int64_t workspace_bytes,
                         hipStream_t stream) {
    const int st = check_dispatch_planned(x, slot_idx, S, H, K, C, quant, window, window_bytes,
                                          workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    return run_dispatch_planned(x, slot_idx, S, H, K, C, quant, src_rank, window, workspace,
                                stream);
}

int moe_layout_dispatch_ws(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                           int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                           int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                           int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                           int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                           const void *x, int32_t H, int32_t quant, int32_t src_rank, void *window,
                           int64_t window_bytes, int32_t path, void *workspace,
                           int64_t workspace_bytes, hipStream_t stream) {
    LayoutDispatchArgs a{{topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank,
                          num_tokens_per_expert, rank_prefix_matrix, expert_prefix_matrix,
                          rank_slot_base, expert_slot_base, slot_idx, status, 0},
                         x, H, quant, src_rank, window};
    int st = check_layout_dispatch(a, path, window_bytes);
    if (st != MOE_OK) return st;
    if (a.layout.form == 1) return run_layout_dispatch(a, stream);  // one kernel, no workspace
    st = check_layout_ws(a.layout, path, quant, workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    st = run_layout_ws(a.layout, quant, workspace, stream);
    if (st != MOE_OK) return st;
    return run_dispatch_planned(x, slot_idx, S, H, K, C, quant, src_rank, window, workspace, stream);
}

int moe_combine(const void *expert_out, int64_t row_stride_bytes, int64_t expert_rows,
                const int32_t *slot_idx, const float *topk_weights, int32_t S, int32_t H,
                int32_t K, void *y, hipStream_t stream) {
    CombineArgs a{expert_out, row_stride_bytes, expert_rows, slot_idx, topk_weights, S, H, K, y};
    const int st = check_combine(a);
    return st != MOE_OK ? st : run_combine(a, stream);
}

// ---- pre-validated calls (moe_plan_*): the checks above run once, moe_plan_run only launches

int moe_plan_layout(moe_plan *plan, const int32_t *topk_idx, int32_t S, int32_t K, int32_t E,
                    int32_t P, int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                    int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                    int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                    int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status, int32_t path) {
    if (!plan) return MOE_ERR_ARG;
    PlanRecord rec{};
    rec.kind = PlanRecord::kLayout;
    rec.layout = LayoutArgs{topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank,
                            num_tokens_per_expert, rank_prefix_matrix, expert_prefix_matrix,
                            rank_slot_base, expert_slot_base, slot_idx, status, 0};
    return store_plan(plan, rec, check_layout(rec.layout, path));
}

int moe_plan_dispatch_ws(moe_plan *plan, const void *x, const int32_t *slot_idx, int32_t S,
                         int32_t H, int32_t K, int32_t quant, int32_t src_rank, void *window,
                         int64_t window_bytes, void *workspace, int64_t workspace_bytes) {
    if (!plan) return MOE_ERR_ARG;
    PlanRecord rec{};
    rec.kind = PlanRecord::kDispatch;
    rec.dispatch = DispatchArgs{x, slot_idx, S, H, K, quant, src_rank, window, workspace, false};
    return store_plan(plan, rec, check_dispatch_ws(rec.dispatch, window_bytes, workspace_bytes));
}

int moe_plan_layout_dispatch(moe_plan *plan, const int32_t *topk_idx, int32_t S, int32_t K,
                             int32_t E, int32_t P, int32_t C, uint8_t *is_token_in_rank,
                             int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                             int32_t *rank_prefix_matrix, int32_t *expert_prefix_matrix,
                             int32_t *rank_slot_base, int32_t *expert_slot_base, int32_t *slot_idx,
                             int32_t *status, const void *x, int32_t H, int32_t quant,
                             int32_t src_rank, void *window, int64_t window_bytes, int32_t path) {
    if (!plan) return MOE_ERR_ARG;
    PlanRecord rec{};
    rec.kind = PlanRecord::kLayoutDispatch;
    rec.layout_dispatch = LayoutDispatchArgs{
        {topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank, num_tokens_per_expert,
         rank_prefix_matrix, expert_prefix_matrix, rank_slot_base, expert_slot_base, slot_idx,
         status, 0},
        x, H, quant, src_rank, window};
    return store_plan(plan, rec, check_layout_dispatch(rec.layout_dispatch, path, window_bytes));
}

int moe_plan_combine(moe_plan *plan, const void *expert_out, int64_t row_stride_bytes,
                     int64_t expert_rows, const int32_t *slot_idx, const float *topk_weights,
                     int32_t S, int32_t H, int32_t K, void *y) {
    if (!plan) return MOE_ERR_ARG;
    PlanRecord rec{};
    rec.kind = PlanRecord::kCombine;
    rec.combine = CombineArgs{expert_out, row_stride_bytes, expert_rows, slot_idx, topk_weights,
                              S, H, K, y};
    return store_plan(plan, rec, check_combine(rec.combine));
}

int moe_plan_layout_ws(moe_plan *plan, const int32_t *topk_idx, int32_t S, int32_t K, int32_t E,
                       int32_t P, int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                       int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                       int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                       int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status, int32_t quant,
                       int32_t path, void *workspace, int64_t workspace_bytes) {
    if (!plan) return MOE_ERR_ARG;
    PlanRecord rec{};
    rec.kind = PlanRecord::kLayoutWs;
    rec.layout_ws = LayoutWsArgs{{topk_idx, S, K, E, P, C, is_token_in_rank, num_tokens_per_rank,
                                  num_tokens_per_expert, rank_prefix_matrix, expert_prefix_matrix,
                                  rank_slot_base, expert_slot_base, slot_idx, status, 0},
                                 quant, workspace};
    return store_plan(plan, rec,
                      check_layout_ws(rec.layout_ws.layout, path, quant, workspace, workspace_bytes));
}

int moe_plan_dispatch_planned(moe_plan *plan, const void *x, const int32_t *slot_idx, int32_t S,
                              int32_t H, int32_t K, int32_t C, int32_t quant, int32_t src_rank,
                              void *window, int64_t window_bytes, void *workspace,
                              int64_t workspace_bytes) {
    if (!plan) return MOE_ERR_ARG;
    PlanRecord rec{};
    rec.kind = PlanRecord::kDispatchPlanned;
    rec.dispatch_planned =
        DispatchPlannedArgs{x, slot_idx, S, H, K, C, quant, src_rank, window, workspace};
    return store_plan(plan, rec,
                      check_dispatch_planned(x, slot_idx, S, H, K, C, quant, window, window_bytes,
                                             workspace, workspace_bytes));
}

int moe_plan_run(const moe_plan *plan, hipStream_t stream) {
    if (!plan) return MOE_ERR_ARG;
    PlanRecord rec;
    std::memcpy(&rec, plan, sizeof(rec));
    if (rec.magic != PlanRecord::kMagic) return MOE_ERR_ARG;
    switch (rec.kind) {
        case PlanRecord::kLayout: return run_layout(rec.layout, stream);
        case PlanRecord::kDispatch: return run_dispatch_ws(rec.dispatch, stream);
        case PlanRecord::kLayoutDispatch: return run_layout_dispatch(rec.layout_dispatch, stream);
        case PlanRecord::kCombine: return run_combine(rec.combine, stream);
        case PlanRecord::kLayoutWs:
            return run_layout_ws(rec.layout_ws.layout, rec.layout_ws.quant, rec.layout_ws.workspace,
                                 stream);
        case PlanRecord::kDispatchPlanned: {
            const DispatchPlannedArgs &d = rec.dispatch_planned;
            return run_dispatch_planned(d.x, d.slot_idx, d.S, d.H, d.K, d.C, d.quant, d.src_rank,
                                        d.window, d.workspace, stream);
        }
        default: return MOE_ERR_ARG;
    }
}

int moe_combine_scatter(const void *expert_out, int64_t row_stride_bytes, int64_t expert_rows,
                        const int32_t *expand_idx, const int32_t *num_rows, int32_t S, int32_t K,
                        int32_t H, void *staging, int64_t staging_stride_bytes,
                        int64_t staging_bytes, hipStream_t stream) {
    if (!expert_out || !expand_idx || !num_rows || !staging) return MOE_ERR_ARG;
    int st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    st = check_hidden(H);
    if (st != MOE_OK) return st;
    if (expert_rows < 0 || expert_rows > MOE_MAX_OUT_ROWS) return MOE_ERR_ARG;
    if (row_stride_bytes < 2 * (int64_t)H || staging_stride_bytes < 2 * (int64_t)H) return MOE_ERR_ARG;
    if (!extent_fits(expert_rows, row_stride_bytes)) return MOE_ERR_ARG;
    if (row_stride_bytes % 16 != 0 || staging_stride_bytes % 16 != 0 || !aligned(expert_out, 16) ||
        !aligned(staging, 16) || !aligned(expand_idx, 4) || !aligned(num_rows, 4))
        return MOE_ERR_ALIGN;
    // staging_bytes >= (S*K - 1) * staging_stride_bytes + 2H, in a form that cannot overflow
    if (staging_bytes < 2 * (int64_t)H ||
        (staging_bytes - 2 * (int64_t)H) / staging_stride_bytes < (int64_t)S * K - 1)
        return MOE_ERR_WINDOW;
    return from_hip(moe::launch_combine_scatter(expert_out, row_stride_bytes, expert_rows,
                                                expand_idx, num_rows, S, K, H, staging,
                                                staging_stride_bytes, stream));
}

int moe_combine_staged(const void *staging, int64_t staging_stride_bytes, int64_t staging_bytes,
                       const int32_t *slot_idx, const float *topk_weights, int32_t S, int32_t H,
                       int32_t K, void *y, hipStream_t stream) {
    if (!staging || !slot_idx || !topk_weights || !y) return MOE_ERR_ARG;
    int st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    st = check_hidden(H);
    if (st != MOE_OK) return st;
    if (staging_stride_bytes < 2 * (int64_t)H) return MOE_ERR_ARG;
    if (staging_stride_bytes % 16 != 0 || !aligned(staging, 16) || !aligned(y, 16) ||
        !aligned(slot_idx, 4) || !aligned(topk_weights, 4))
        return MOE_ERR_ALIGN;
    // staging_bytes >= (S*K - 1) * staging_stride_bytes + 2H, in a form that cannot overflow
    if (staging_bytes < 2 * (int64_t)H ||
        (staging_bytes - 2 * (int64_t)H) / staging_stride_bytes < (int64_t)S * K - 1)
        return MOE_ERR_WINDOW;
    return from_hip(moe::launch_combine_staged(staging, staging_stride_bytes, slot_idx,
                                               topk_weights, S, H, K, y, stream));
}

int moe_rank_rows(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
                  const int32_t *rank_prefix_matrix, const int32_t *num_tokens_per_rank,
                  int32_t *rank_row_idx, int32_t *rank_token_base, hipStream_t stream) {
    if (!topk_idx || !rank_prefix_matrix || !num_tokens_per_rank || !rank_row_idx ||
        !rank_token_base)
        return MOE_ERR_ARG;
    int st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    st = check_experts(E, P);
    if (st != MOE_OK) return st;
    if (C < 1 || C > S || C > MOE_MAX_CHANNELS) return MOE_ERR_ARG;
    if (!aligned(topk_idx, 4) || !aligned(rank_prefix_matrix, 4) ||
        !aligned(num_tokens_per_rank, 4) || !aligned(rank_row_idx, 4) || !aligned(rank_token_base, 4))
        return MOE_ERR_ALIGN;
    return from_hip(moe::launch_rank_rows(topk_idx, S, K, E, P, C, rank_prefix_matrix,
                                          num_tokens_per_rank, rank_row_idx, rank_token_base,
                                          stream));
}

int moe_dispatch_dedup(const void *x, const int32_t *rank_row_idx, const int32_t *topk_idx,
                       int32_t S, int32_t H, int32_t K, int32_t E, int32_t P, int32_t quant,
                       int32_t src_rank, void *window, int64_t window_bytes, hipStream_t stream) {
    if (!x || !rank_row_idx || !topk_idx || !window) return MOE_ERR_ARG;
    int st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    st = check_hidden(H);
    if (st != MOE_OK) return st;
    st = check_experts(E, P);
    if (st != MOE_OK) return st;
    if (!moe::valid_quant(quant)) return MOE_ERR_ARG;
    if (!aligned(x, 16) || !aligned(window, 512) || !aligned(rank_row_idx, 4) || !aligned(topk_idx, 4))
        return MOE_ERR_ALIGN;
    if (window_bytes < moe_dedup_window_bytes(S, K, P, H)) return MOE_ERR_WINDOW;
    return from_hip(moe::launch_pack_dedup(x, rank_row_idx, topk_idx, S, H, K, E, P, quant,
                                           src_rank, window, stream));
}

int moe_expand_dedup(const void *window, int64_t window_bytes, const int32_t *rank_row_idx,
                     const int32_t *slot_idx, const int32_t *num_slots, int32_t S, int32_t K,
                     int32_t P, int32_t H, int32_t quant, void *expand_x, float *expand_scales,
                     int32_t *expand_idx, hipStream_t stream) {
    if (!window || !rank_row_idx || !slot_idx || !num_slots || !expand_x || !expand_idx)
        return MOE_ERR_ARG;
    int st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    st = check_hidden(H);
    if (st != MOE_OK) return st;
    if (P < 1 || P > MOE_MAX_RANKS) return MOE_ERR_ARG;
    if (!moe::valid_quant(quant)) return MOE_ERR_ARG;
    if (quant != MOE_QUANT_NONE && !expand_scales) return MOE_ERR_ARG;
    if (!aligned(window, 512) || !aligned(expand_x, 16) || !aligned(rank_row_idx, 4) ||
        !aligned(slot_idx, 4) || !aligned(num_slots, 4) || !aligned(expand_idx, 4) ||
        (expand_scales && !aligned(expand_scales, 4)))
        return MOE_ERR_ALIGN;
    if (window_bytes < moe_dedup_window_bytes(S, K, P, H)) return MOE_ERR_WINDOW;
    return from_hip(moe::launch_expand_dedup(window, rank_row_idx, slot_idx, num_slots, S, K, P, H,
                                             quant, expand_x, expand_scales, expand_idx, stream));
}

int moe_unpack(const void *window, int64_t window_bytes, const int32_t *num_slots, int32_t S,
               int32_t K, int32_t H, int32_t quant, void *expand_x, float *expand_scales,
               int32_t *expand_idx, hipStream_t stream) {
    if (!window || !num_slots || !expand_x || !expand_idx) return MOE_ERR_ARG;
    int st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    st = check_hidden(H);
    if (st != MOE_OK) return st;
    if (!moe::valid_quant(quant)) return MOE_ERR_ARG;
    if (quant != MOE_QUANT_NONE && !expand_scales) return MOE_ERR_ARG;
    if (!aligned(window, 512) || !aligned(expand_x, 16) || !aligned(num_slots, 4) ||
        !aligned(expand_idx, 4) || (expand_scales && !aligned(expand_scales, 4)))
        return MOE_ERR_ALIGN;
    if (window_bytes < moe_window_bytes(S, K, H)) return MOE_ERR_WINDOW;
    return from_hip(moe::launch_unpack(window, num_slots, S, K, H, quant, expand_x, expand_scales,
                                       expand_idx, stream));
}

int moe_unpack_padded(const void *window, int64_t window_bytes, const int32_t *expert_slot_base,
                      int32_t E, int32_t S, int32_t K, int32_t H, int32_t quant,
                      int32_t expert_alignment, int64_t out_rows, void *expand_x,
                      float *expand_scales, int32_t *expand_idx, int32_t *expert_row_base,
                      int32_t *status, hipStream_t stream) {
    if (!window || !expert_slot_base || !expand_x || !expand_idx || !expert_row_base || !status)
        return MOE_ERR_ARG;
    int st = check_tokens(S, K);
    if (st != MOE_OK) return st;
    st = check_hidden(H);
    if (st != MOE_OK) return st;
    if (!moe::valid_quant(quant)) return MOE_ERR_ARG;
    if (quant != MOE_QUANT_NONE && !expand_scales) return MOE_ERR_ARG;
    if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_ARG;
    if (expert_alignment < 1 || expert_alignment > MOE_MAX_ALIGNMENT) return MOE_ERR_ARG;
    if (out_rows < 1 || out_rows > MOE_MAX_OUT_ROWS) return MOE_ERR_ARG;
    if (!aligned(window, 512) || !aligned(expand_x, 16) || !aligned(expert_slot_base, 4) ||
        !aligned(expand_idx, 4) || !aligned(expert_row_base, 4) || !aligned(status, 4) ||
        (expand_scales && !aligned(expand_scales, 4)))
        return MOE_ERR_ALIGN;
    if (window_bytes < moe_window_bytes(S, K, H)) return MOE_ERR_WINDOW;
    return from_hip(moe::launch_unpack_padded(window, expert_slot_base, E, S, K, H, quant,
                                              expert_alignment, out_rows, expand_x, expand_scales,
                                              expand_idx, expert_row_base, status, stream));
}

const char *moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_ARG: return "invalid argument (null pointer or size out of range)";
        case MOE_ERR_ALIGN: return "misaligned pointer or stride";
        case MOE_ERR_WINDOW: return "buffer too small: the window (S*K*moe_slot_bytes(H) bytes), staging rows or workspace";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape (E % P != 0, H % 16 != 0 or S too large)";
        case MOE_ERR_HIP: return "HIP launch error";
        case MOE_ERR_SCRATCH:
            return "table too large for the fixed scratch of moe_dispatch_noalloc (see MOE_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

}  // extern "C"
