/*
 * moe.h - C ABI of the MI355X (gfx950) MoE normal-mode layout / dispatch / combine library.
 *
 * One GPU's share of expert-parallel dispatch and combine: the P expert-parallel ranks are P
 * contiguous partitions of one caller-owned HBM window, so nothing here talks to another GPU.
 *
 * Notation follows "Ascend DeepEP MoE Dispatch Optimization", section "一条 token 如何走完 MoE":
 * x[S,H] token rows, topk_idx[S,K] and topk_weights[S,K] from the router, E global experts spread
 * over P ranks with experts_per_rank = E / P, dst_rank = expert_id / experts_per_rank and
 * dst_local_expert = expert_id % experts_per_rank.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers; sizes are element counts unless named *_bytes.
 *   - All arrays are dense and row-major.
 *   - The caller allocates and owns every buffer; the library allocates nothing and keeps no
 *     state between calls beyond a per-device cache of the compute-unit count (which sizes the
 *     grid of moe_layout_dispatch), and is reentrant. Calls that take a stream only enqueue work
 *     on it and return without synchronising the host.
 *   - Arguments are validated on the host before any HIP call. On a validation failure nothing is
 *     enqueued and a negative moe_status is returned. MOE_ERR_HIP reports a failed launch.
 */
#ifndef MOE_LAYOUT_MI355X_H
#define MOE_LAYOUT_MI355X_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_ARG = -1,         /* null pointer or a size outside its documented range          */
    MOE_ERR_ALIGN = -2,       /* a pointer or stride is not aligned as documented             */
    MOE_ERR_WINDOW = -3,      /* window_bytes < moe_window_bytes(S, K, H), or a staging buffer
                                 shorter than its S*K rows                                    */
    MOE_ERR_UNSUPPORTED = -4, /* E % P != 0, H % 16 != 0, or S above MOE_MAX_TOKENS           */
    MOE_ERR_HIP = -5,         /* the HIP runtime reported an error for a launch               */
    MOE_ERR_SCRATCH = -6      /* moe_dispatch_noalloc: the table needs more than its fixed scratch */
} moe_status;

typedef enum {
    MOE_QUANT_NONE = 0,         /* bf16 payload                                              */
    MOE_QUANT_FP8_E4M3_DYN = 1, /* per-token E4M3FN payload + fp32 scale in the slot tail    */
    MOE_QUANT_INT8_DYN = 2      /* per-token symmetric INT8 payload + fp32 scale             */
} moe_quant;

/* Limits. The expert, rank and top-k bounds are those the CAM kernels check ("HCCL Window 模式
 * (Non-SHMEM) 代码深度剖析", section 9.6 限制常量: MOE_EXPERT_MAX_NUM 512, K_MAX 16, 384 ranks). The
 * CAM batch bound of 8000 tokens is not kept, so that S = 8192 fits; H may go below the CAM H_MIN. */
#define MOE_MAX_K 16
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_RANKS 384
#define MOE_MAX_CHANNELS 4096
#define MOE_MAX_TOKENS 65536
#define MOE_MAX_HIDDEN 16384
#define MOE_MAX_ALIGNMENT 65536   /* expert_alignment of moe_unpack_padded */
#define MOE_MAX_OUT_ROWS 1048576  /* out_rows of moe_unpack_padded */

/* Bytes of one window slot: Ceil(Ceil(2H, 32) * 32 + 44, 512) * 512, the dispatch token size of
 * "HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 8.2 (Window 大小校验): the bf16 row padded to
 * 32 bytes, a 32-byte scale block and a 12-byte triple, rounded up to 512 bytes (14848 at H=7168).
 * The fp8 slot has the same size. Returns a negative moe_status if H is not in [16, MOE_MAX_HIDDEN]
 * or not a multiple of 16. */
int64_t moe_slot_bytes(int32_t H);

/* Window bytes moe_dispatch needs: S * K * moe_slot_bytes(H), room for every (token, k) copy, so
 * the caller never reads a count back (the worst-case sizing of "Ascend DeepEP MoE Dispatch
 * Optimization", section "输出长度有动态和固定两种模式"). Negative moe_status on bad arguments. */
int64_t moe_window_bytes(int32_t S, int32_t K, int32_t H);

/* Byte offsets inside one slot ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 2.3 数据区 Token
 * 格式): payload [0, payload_bytes) = 2H (bf16) or H (fp8); scale block [scale_off, scale_off+32)
 * with scale_off = Ceil(payload_bytes, 32) * 32 and the fp32 scale in its first 4 bytes (zero in
 * bf16 mode); triple int32 (src_rank, token, k) at triple_off = scale_off + 32; zero padding up
 * to tail_end = Ceil(triple_off + 12, 128). moe_dispatch writes exactly [0, tail_end) of each
 * used slot. Both quantised modes have payload_bytes = H. Any output pointer may be NULL. Returns
 * MOE_OK or a negative moe_status. */
int moe_slot_offsets(int32_t H, int32_t quant, int64_t *payload_bytes, int64_t *scale_off,
                     int64_t *triple_off, int64_t *tail_end);

/* Routing layout: topk_idx -> membership, counts, prefix matrices and the slot of every (t, k).
 *
 * Follows the dispatch handle and notify stage of "Ascend DeepEP MoE Dispatch Optimization"
 * (sections "Dispatch handle 六项分别保存什么", "Notify 先交换数量和前缀", "Device 侧如何把 channel
 * 变成远端 Put") and the per-expert offset + running count of the CAM pack ("HCCL Window 模式
 * (Non-SHMEM) 代码深度剖析", section 3.6 InputToShare).
 *
 * In:  topk_idx  int32 [S, K]. Ids in [0, E) are valid; -1 is a pad; any other value is treated
 *                as a pad and sets bit 0 of *status.
 *      S in [1, MOE_MAX_TOKENS], K in [1, MOE_MAX_K], E in [1, MOE_MAX_EXPERTS],
 *      P in [1, MOE_MAX_RANKS] with E % P == 0, C (channels) in [1, min(S, MOE_MAX_CHANNELS)].
 *      Channel c owns tokens [c*(S/C) + min(c, S%C), ...) with S/C + (c < S%C) tokens
 *      ("HCCL Window 模式", section 8.3 分片策略).
 * Out (all fully overwritten):
 *      is_token_in_rank      uint8 [S, P]  1 iff token t has a valid expert on rank r
 *      num_tokens_per_rank   int32 [P]     tokens routed to each rank (a token counts once)
 *      num_tokens_per_expert int32 [E]     valid (t, k) entries per expert
 *      rank_prefix_matrix    int32 [P, C]  tokens of channels 0..c routed to rank r (inclusive)
 *      expert_prefix_matrix  int32 [E, C]  entries of channels 0..c routed to expert e (inclusive)
 *      rank_slot_base        int32 [P+1]   first slot of rank r; [P] = N, the valid-entry count
 *      expert_slot_base      int32 [E+1]   first slot of expert e; [E] = N
 *      slot_idx              int32 [S, K]  slot of (t, k), or -1 for pads. Slots are ordered by
 *                                          expert id, then source token, then k, so each rank's
 *                                          slots are the contiguous range
 *                                          [rank_slot_base[r], rank_slot_base[r+1]).
 *      status                int32 [1]     0, or bit 0 set if an id outside [-1, E) was seen
 * Enqueues one kernel on `stream` when S*K <= 4096 and C <= 1024 (decode-sized tables: every
 * workgroup rereads the table and writes its own share of the outputs), otherwise three kernels
 * (count per channel, scan along channels, assign). Both forms give identical outputs; the choice
 * depends on the sizes only. No output may alias an input or another output. */
int moe_layout(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
               uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
               int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
               int32_t *expert_prefix_matrix, int32_t *rank_slot_base, int32_t *expert_slot_base,
               int32_t *slot_idx, int32_t *status, hipStream_t stream);

/* Which form of the layout a call of moe_layout_ex / moe_layout_dispatch_ex takes. The forms give
 * identical outputs; the choice exists so that tests and benchmarks can run each form on the same
 * table. */
typedef enum {
    MOE_LAYOUT_AUTO = 0,   /* what moe_layout does: one launch when S*K <= 4096 and C <= 1024     */
    MOE_LAYOUT_MULTI = 1,  /* always the multi-launch form (count, scan, assign)                  */
    MOE_LAYOUT_SINGLE = 2  /* always the single-launch form; MOE_ERR_UNSUPPORTED where S*K > 4096
                              or C > 1024                                                        */
} moe_layout_path;

/* moe_layout with an explicit form: same arguments, outputs and errors, plus `path` (a
 * moe_layout_path; any other value is MOE_ERR_ARG). */
int moe_layout_ex(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
                  uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                  int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                  int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                  int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status, int32_t path,
                  hipStream_t stream);

/* Dispatch pack: for every (t, k) with slot s = slot_idx[t, k] >= 0, write slot s of the window
 * (byte offset s * moe_slot_bytes(H)) as the slot layout above: the bf16 row x[t], or its
 * per-token dynamic quantisation with amax = max |x[t]| in fp32:
 *   MOE_QUANT_FP8_E4M3_DYN: scale = amax / 448, codes = E4M3FN(x / scale), round to nearest even,
 *                           saturating to +-448;
 *   MOE_QUANT_INT8_DYN:     scale = amax / 127, codes = clamp(rint(x / scale), -127, 127), rint
 *                           rounding half to even, two's complement bytes;
 * every division an IEEE fp32 division (codes are those of the correctly rounded quotient; x must
 * be finite in these modes: a NaN or infinity gives unspecified codes); an all-zero row gives
 * scale 0 and zero codes. Then the
 * scale block and the triple (src_rank, t, k). This is the CAM InputToShare copy with its
 * DynamicQuant branch ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.6, whose quantised output
 * type is INT8, and the slot format of section 2.3), with each row read once per token instead of
 * once per copy.
 *
 * In:  x        bf16 [S, H] as raw 16-bit words, 16-byte aligned.
 *      slot_idx int32 [S, K] from moe_layout (or any table of distinct slots); entries < 0 and
 *               entries >= S * K are skipped.
 *      H in [16, MOE_MAX_HIDDEN], H % 16 == 0; quant is a moe_quant; src_rank is stored verbatim.
 *      window   512-byte aligned device buffer of window_bytes >= moe_window_bytes(S, K, H).
 * Writes bytes [0, tail_end) of each used slot and nothing else. Slots nobody maps to, and
 * the bytes after tail_end in every slot, keep their contents. */
int moe_dispatch(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                 int32_t quant, int32_t src_rank, void *window, int64_t window_bytes,
                 hipStream_t stream);

/* Dispatch pack with a caller workspace: the same window bytes as moe_dispatch (same arguments,
 * same meaning, same bytes written and left untouched), written in an order that HBM absorbs
 * faster. The CAM pack ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.6 InputToShare) writes
 * each token's copies as soon as its row is read, which spreads the writes in flight over every
 * expert's slot range; here a plan kernel first lists each chunk of tokens' (slot, token, k)
 * records by slot, and the pack kernel then writes every chunk in slot order from rows its XCD
 * has just read.
 *
 * moe_dispatch_workspace_bytes(S, K, quant): bytes the workspace needs (0 when the call takes the
 *      token-order pack: quantised modes, and bf16 tables of fewer than 8192 entries); a negative
 *      moe_status on bad S, K or quant.
 * moe_dispatch_ws: as moe_dispatch, plus
 *      workspace       device buffer, 16-byte aligned, of workspace_bytes >=
 *                      moe_dispatch_workspace_bytes(S, K, quant) (MOE_ERR_WINDOW otherwise; it may
 *                      be NULL when that size is 0, MOE_ERR_ARG if it is NULL otherwise). Its
 *                      contents are overwritten; the caller owns it and must not use it for
 *                      anything else until the call's kernels have finished. Calls that may run at
 *                      the same time need workspaces of their own.
 * Enqueues the plan kernel and the pack kernel (or only the token-order pack when the workspace
 * size is 0) on `stream`. */
int64_t moe_dispatch_workspace_bytes(int32_t S, int32_t K, int32_t quant);

int moe_dispatch_ws(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                    int32_t quant, int32_t src_rank, void *window, int64_t window_bytes,
                    void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* moe_dispatch_ws for callers that cannot allocate (code under HIP graph capture, serving loops
 * that may not call hipMalloc, harnesses that forbid allocation): the same window bytes and the
 * same kernels, with the planned pack's record lists in a fixed scratch array that the library
 * holds in device memory (MOE_NOALLOC_SCRATCH_BYTES per GPU, kept until the process ends) instead
 * of a caller workspace. It allocates nothing.
 *
 * Arguments, checks and errors as moe_dispatch, plus MOE_ERR_SCRATCH (nothing enqueued) when
 * moe_dispatch_workspace_bytes(S, K, quant) exceeds MOE_NOALLOC_SCRATCH_BYTES (bf16 tables up to
 * 16384 tokens at K = 8 fit). The first call on a device looks up that device's copy of the array;
 * a failure there is MOE_ERR_HIP. Every call on a GPU uses that GPU's one array: calls that may run
 * at the same time on one GPU (two streams, two host threads) race on it and must not overlap.
 * The plan kernel rewrites every record the pack kernel reads, so no call depends on what an
 * earlier call left in the array. */
#define MOE_NOALLOC_SCRATCH_BYTES (1 << 20)

int moe_dispatch_noalloc(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                         int32_t quant, int32_t src_rank, void *window, int64_t window_bytes,
                         hipStream_t stream);

/* Layout and dispatch pack in one call: the outputs of moe_layout (same arguments, same meaning)
 * and the window of moe_dispatch (same x, H, quant, src_rank, window, window_bytes), bit for bit.
 * It is the fused single-kernel layout + pack for decode-sized batches, where both steps are
 * latency: the routing plan of "Ascend DeepEP MoE Dispatch Optimization" (section "Dispatch handle
 * 六项分别保存什么") and the InputToShare copy of "HCCL Window 模式 (Non-SHMEM) 代码深度剖析"
 * (section 3.6) without a launch between them.
 *
 * When S*K <= 4096 and C <= 1024 it enqueues ONE kernel: its layout workgroups write the layout
 * outputs while its pack workgroups derive the slots of their own tokens from topk_idx (the number
 * of valid entries before (t, k) in expert-major, token, k order) and store the rows; nothing in it
 * reads slot_idx. Otherwise it enqueues the moe_layout kernels followed by the moe_dispatch
 * kernel. Argument checks, alignment rules and error codes are the union of the two calls'; the
 * window must not overlap any other argument. */
int moe_layout_dispatch(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                        int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                        int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                        int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                        int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                        const void *x, int32_t H, int32_t quant, int32_t src_rank, void *window,
                        int64_t window_bytes, hipStream_t stream);

/* moe_layout_dispatch with an explicit form (a moe_layout_path): MOE_LAYOUT_SINGLE is the one
 * kernel above, MOE_LAYOUT_MULTI the moe_layout kernels followed by the pack. */
int moe_layout_dispatch_ex(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                           int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                           int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                           int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                           int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                           const void *x, int32_t H, int32_t quant, int32_t src_rank, void *window,
                           int64_t window_bytes, int32_t path, hipStream_t stream);

/* The layout and the pack with a caller workspace: the outputs of moe_layout_ex and the window bytes
 * of moe_dispatch, in fewer launches. For tables that do not take the single kernel, the layout runs
 * as two kernels instead of three: a count kernel per channel that also groups each channel's
 * entries by expert into the workspace, then workgroups per expert that scan its prefix row and hand
 * its entries their slots straight from those groups (the per-expert offset + running count of
 * "HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.6, with the counts of "Ascend DeepEP MoE
 * Dispatch Optimization", section "Notify 先交换数量和前缀"). In bf16 mode with at least 8192 entries
 * and at most 1024 entries a channel (ceil(S / C) * K <= 1024), that second kernel also writes the
 * plan of the planned pack (see moe_dispatch_ws), so no separate plan kernel runs.
 *
 * The workspace (device memory, 16-byte aligned, contents overwritten) holds the pack plan first,
 * then the layout's scratch; calls that may run at the same time need workspaces of their own.
 *
 * moe_layout_dispatch_workspace_bytes(S, K, E, P, C, quant, path): the bytes these calls need for
 *      these arguments: 0 when the layout takes the single kernel (its table is small, see
 *      moe_layout_ex); negative moe_status on bad arguments (those of moe_layout_ex, quant).
 * moe_layout_ws: moe_layout_ex's arguments plus quant (the payload type the following
 *      moe_dispatch_planned will use: the plan is written only for MOE_QUANT_NONE) and the workspace
 *      (NULL allowed when the size above is 0; MOE_ERR_ARG if NULL otherwise, MOE_ERR_ALIGN if not
 *      16-byte aligned, MOE_ERR_WINDOW if workspace_bytes is below that size). Enqueues 1 kernel
 *      (single form) or 2.
 * moe_dispatch_planned: the window bytes of moe_dispatch for slot_idx (the one moe_layout_ws wrote),
 *      using the plan moe_layout_ws left in the same workspace; S, K, C and quant must be those of
 *      that moe_layout_ws call, and the workspace must not have been written in between (a plan from
 *      another table writes that table's bytes; records are bounds-checked, so never outside the
 *      window or x). Where the layout writes no plan, the call runs moe_dispatch_ws's plan kernel on
 *      slot_idx (bf16, S*K >= 8192; it writes the workspace's plan part) or the token-order pack (no
 *      workspace needed). Checks: those of
 *      moe_dispatch, C in [1, min(S, MOE_MAX_CHANNELS)], then the workspace as above, against the plan's
 *      part only. Enqueues 1 kernel (2 when it runs the plan kernel).
 * moe_layout_dispatch_ws: moe_layout_dispatch_ex's arguments plus the workspace: moe_layout_ws then
 *      moe_dispatch_planned (the single layout + pack kernel of moe_layout_dispatch for small tables).
 */
int64_t moe_layout_dispatch_workspace_bytes(int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
                                             int32_t quant, int32_t path);

int moe_layout_ws(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
                  uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                  int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                  int32_t *expert_prefix_matrix, int32_t *rank_slot_base, int32_t *expert_slot_base,
                  int32_t *slot_idx, int32_t *status, int32_t quant, int32_t path, void *workspace,
                  int64_t workspace_bytes, hipStream_t stream);

int moe_dispatch_planned(const void *x, const int32_t *slot_idx, int32_t S, int32_t H, int32_t K,
                         int32_t C, int32_t quant, int32_t src_rank, void *window,
                         int64_t window_bytes, void *workspace, int64_t workspace_bytes,
                         hipStream_t stream);

int moe_layout_dispatch_ws(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P,
                           int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                           int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                           int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                           int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status,
                           const void *x, int32_t H, int32_t quant, int32_t src_rank, void *window,
                           int64_t window_bytes, int32_t path, void *workspace,
                           int64_t workspace_bytes, hipStream_t stream);

/* Combine: y[t] = bf16( sum over k = 0..K-1 ascending with slot_idx[t, k] valid of
 *                       fp32(topk_weights[t, k] * fp32(expert_out row slot_idx[t, k])) ),
 * accumulated in fp32 from +0.0, each product and each sum rounded to fp32 (no fused
 * multiply-add), one round-to-nearest-even to bf16 at the end; a token with no valid entry gives
 * +0.0. Infinities and NaNs in the rows or weights propagate as IEEE fp32 arithmetic makes them;
 * the payload of a NaN result is not specified. This is ReadBufferAndWeightedSum of "HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 7.8,
 * with the K rows gathered by slot index instead of first scattered to position t*K + k.
 *
 * In:  expert_out    bf16 rows, row r at byte offset r * row_stride_bytes; 16-byte aligned;
 *                    row_stride_bytes >= 2H and a multiple of 16. Passing the window with
 *                    row_stride_bytes = moe_slot_bytes(H) combines the dispatched bf16 payload.
 *      expert_rows   number of readable rows; entries of slot_idx outside [0, expert_rows) are
 *                    skipped like pads. expert_rows * row_stride_bytes must not exceed INT64_MAX
 *                    (MOE_ERR_ARG otherwise).
 *      slot_idx      int32 [S, K]; topk_weights fp32 [S, K].
 * Out: y             bf16 [S, H], 16-byte aligned, fully overwritten; must not overlap the inputs. */
int moe_combine(const void *expert_out, int64_t row_stride_bytes, int64_t expert_rows,
                const int32_t *slot_idx, const float *topk_weights, int32_t S, int32_t H,
                int32_t K, void *y, hipStream_t stream);

/* Two-pass combine, the CAM form of the combine ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", sections
 * 7.5 CopyBufferToShareAndSetStatus and 7.8 ReadBufferAndWeightedSum): first every expert output
 * row is copied to position t*K + k of a staging buffer, (t, k) taken from the triple its slot
 * carried; then each token reduces its K contiguous staging rows with the arithmetic of
 * moe_combine. moe_combine_staged(moe_combine_scatter(...)) gives bit for bit what moe_combine
 * gives on the same rows; the two-pass form moves each row twice more and exists to compare the
 * page's design with the single gather.
 *
 * moe_combine_scatter
 * In:  expert_out     bf16 rows as for moe_combine (row s = the output for slot s); expert_rows
 *                     rows are readable, expert_rows in [0, MOE_MAX_OUT_ROWS], and
 *                     expert_rows * row_stride_bytes must not exceed INT64_MAX.
 *      expand_idx     int32 [expert_rows, 3]: the (src_rank, t, k) triple of each row, e.g. from
 *                     moe_unpack.
 *      num_rows       DEVICE pointer to N (e.g. &expert_slot_base[E]); rows s >= min(N,
 *                     expert_rows) and rows whose (t, k) lies outside [0, S) x [0, K) are not moved.
 * Out: staging        bf16, row t*K + k at byte offset (t*K + k) * staging_stride_bytes (stride
 *                     >= 2H, multiple of 16; the page uses rows rounded up to 512 bytes);
 *                     staging_bytes must cover S*K rows. Rows that receive nothing keep their
 *                     contents.
 * moe_combine_staged
 * In:  staging as written by moe_combine_scatter, staging_bytes long (MOE_ERR_WINDOW unless it
 *      covers S*K rows of staging_stride_bytes: (S*K - 1) * stride + 2H bytes); slot_idx int32
 *      [S, K] (only its sign is used: entries < 0 are skipped, all others read staging row
 *      t*K + k); topk_weights fp32 [S, K].
 * Out: y bf16 [S, H], fully overwritten. */
int moe_combine_scatter(const void *expert_out, int64_t row_stride_bytes, int64_t expert_rows,
                        const int32_t *expand_idx, const int32_t *num_rows, int32_t S, int32_t K,
                        int32_t H, void *staging, int64_t staging_stride_bytes,
                        int64_t staging_bytes, hipStream_t stream);

int moe_combine_staged(const void *staging, int64_t staging_stride_bytes, int64_t staging_bytes,
                       const int32_t *slot_idx, const float *topk_weights, int32_t S, int32_t H,
                       int32_t K, void *y, hipStream_t stream);

/* Unpack: window slots -> compact expert input rows ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析",
 * section 3.9 ShareToOutput, which copies each received slot's token data to the next row of
 * expandXOut and its triple to expandIdxOut). On one GPU the window is already expert-major with
 * ascending source tokens, so row s of the output is slot s without its padding and tail: the
 * contiguous per-expert input of a grouped GEMM, with experts starting at expert_slot_base.
 *
 * In:  window      the dispatched window (512-byte aligned, window_bytes >= moe_window_bytes).
 *      num_slots   DEVICE pointer to N, the number of used slots (e.g. &expert_slot_base[E] from
 *                  moe_layout); read on the device, so nothing is copied back to the host. Values
 *                  above S*K are clamped to S*K.
 *      S, K, H, quant as given to moe_dispatch.
 * Out: expand_x     [S*K, payload_bytes] bytes, 16-byte aligned: bf16 [., H] or codes [., H].
 *      expand_scales fp32 [S*K], the per-row scale (quantised modes; may be NULL for bf16).
 *      expand_idx   int32 [S*K, 3], the (src_rank, token, k) triple of each row.
 * Rows 0..N-1 are written; rows N..S*K-1 keep their contents. */
int moe_unpack(const void *window, int64_t window_bytes, const int32_t *num_slots, int32_t S,
               int32_t K, int32_t H, int32_t quant, void *expand_x, float *expand_scales,
               int32_t *expand_idx, hipStream_t stream);

/* Per-rank deduplicated dispatch, DeepEP's form of the dispatch ("Ascend DeepEP MoE Dispatch
 * Optimization", section "一条 token 如何走完 MoE": a token's row is copied once to each rank that holds
 * one of its experts, and the receiving rank rearranges it into per-local-expert input; sections
 * "P 维路由为什么值得单独优化" and "所谓 compact plan 到底压缩了什么": only a token's real destinations
 * are planned, aggregated into one contiguous segment per rank). Payloads as for moe_dispatch: bf16,
 * or per-token dynamic fp8 E4M3 / INT8 codes with the scale in the row's scale block.
 *
 * Rank r's segment starts at rank_token_base[r] (exclusive prefix of num_tokens_per_rank, [P] = M,
 * the number of rows) and lists the tokens with a valid expert on r in ascending token order.
 * rank_row_idx[t, k] (int32 [S, K]) is the row of token t in the segment of the rank of its k-th
 * expert, the same for every k of the token on that rank, and -1 for masked entries: the compact
 * [S, K] form of DeepEP's send_head. Rows use the slot format of moe_dispatch with the triple
 * (src_rank, t, destination rank). At S=4096, K=8, P=8 with uniform routing M is about 5.3 S
 * instead of the 8 S rows of the K-fold window.
 *
 * moe_dedup_window_bytes: S * min(K, P) * moe_slot_bytes(H), the worst case; negative moe_status on
 *                         bad sizes.
 * moe_rank_rows:      in:  topk_idx, S, K, E, P, C as for moe_layout, and its outputs
 *                          rank_prefix_matrix [P, C] and num_tokens_per_rank [P];
 *                     out: rank_row_idx int32 [S, K], rank_token_base int32 [P + 1]. One kernel.
 * moe_dispatch_dedup: in:  x bf16 [S, H] (16-byte aligned), rank_row_idx, topk_idx, E, P, quant,
 *                          src_rank; window 512-byte aligned, window_bytes >= moe_dedup_window_bytes;
 *                     writes bytes [0, tail_end) of rows 0..M-1 (see moe_slot_offsets), the codes
 *                     and scale computed exactly as moe_dispatch computes them.
 * moe_expand_dedup:   in:  the deduplicated window; rank_row_idx [S, K] from moe_rank_rows;
 *                          slot_idx [S, K] from moe_layout; num_slots = DEVICE pointer to N, the
 *                          valid-entry count (&expert_slot_base[E]); P; quant as dispatched;
 *                     out: expand_x [S*K, payload_bytes] bytes (16-byte aligned), expand_scales
 *                          fp32 [S*K] (quantised modes; may be NULL for bf16) and expand_idx int32
 *                          [S*K, 3]:
 *                          for every valid (t, k), row slot_idx[t, k] gets row rank_row_idx[t, k]
 *                          (token t on the rank of expert k) and the triple (src_rank read from that
 *                          row, t, k), which is exactly what moe_unpack of the K-fold window writes;
 *                          other rows keep their contents. Two kernels; output rows are written
 *                          in order. */
int64_t moe_dedup_window_bytes(int32_t S, int32_t K, int32_t P, int32_t H);

int moe_rank_rows(const int32_t *topk_idx, int32_t S, int32_t K, int32_t E, int32_t P, int32_t C,
                  const int32_t *rank_prefix_matrix, const int32_t *num_tokens_per_rank,
                  int32_t *rank_row_idx, int32_t *rank_token_base, hipStream_t stream);

int moe_dispatch_dedup(const void *x, const int32_t *rank_row_idx, const int32_t *topk_idx,
                       int32_t S, int32_t H, int32_t K, int32_t E, int32_t P, int32_t quant,
                       int32_t src_rank, void *window, int64_t window_bytes, hipStream_t stream);

int moe_expand_dedup(const void *window, int64_t window_bytes, const int32_t *rank_row_idx,
                     const int32_t *slot_idx, const int32_t *num_slots, int32_t S, int32_t K,
                     int32_t P, int32_t H, int32_t quant, void *expand_x, float *expand_scales,
                     int32_t *expand_idx, hipStream_t stream);

/* Padded unpack: the rows of moe_unpack placed for a grouped GEMM whose per-expert blocks start on
 * a multiple of expert_alignment, in an output of exactly out_rows rows. Two options of DeepEP's
 * normal dispatch: expert_alignment rounds every per-expert row count up to a multiple of the
 * alignment ("internode.cu", section 1 notify_dispatch), and num_worst_tokens fixes the output
 * length so that no count has to be read back on the host, with zero data and -1 indices in the
 * rows past the real ones ("Ascend DeepEP MoE Dispatch Optimization", section
 * "输出长度有动态和固定两种模式").
 *
 *   count[e]    = expert_slot_base[e+1] - expert_slot_base[e]
 *   row_base[e] = sum over e' < e of ceil(count[e'] / A) * A,   row_base[E] = the aligned total
 *   row row_base[e] + j (j < count[e]) <- slot expert_slot_base[e] + j, as moe_unpack writes it;
 *   every other row r < out_rows is padding: zero bytes, scale 0, triple (-1, -1, -1).
 *
 * In:  window, window_bytes, S, K, H, quant as for moe_unpack.
 *      expert_slot_base  DEVICE int32 [E+1] from moe_layout; read on the device.
 *      E                 in [1, MOE_MAX_EXPERTS].
 *      expert_alignment  A in [1, MOE_MAX_ALIGNMENT].
 *      out_rows          R in [1, MOE_MAX_OUT_ROWS].
 * Out (all R rows fully written):
 *      expand_x          [R, payload_bytes] bytes, 16-byte aligned.
 *      expand_scales     fp32 [R] (quantised modes; may be NULL for bf16).
 *      expand_idx        int32 [R, 3].
 *      expert_row_base   int32 [E+1], row_base above (the grouped GEMM's group offsets; the
 *                        aligned count of expert e is row_base[e+1] - row_base[e]).
 *      status            int32 [1]: 1 if row_base[E] > R (rows at or past R were dropped; the page
 *                        notes the same truncation happens silently in DeepEP), else 0.
 * Enqueues two kernels on `stream`; nothing is read back to the host. */
int moe_unpack_padded(const void *window, int64_t window_bytes, const int32_t *expert_slot_base,
                      int32_t E, int32_t S, int32_t K, int32_t H, int32_t quant,
                      int32_t expert_alignment, int64_t out_rows, void *expand_x,
                      float *expand_scales, int32_t *expand_idx, int32_t *expert_row_base,
                      int32_t *status, hipStream_t stream);

/* Pre-validated calls, for callers that launch the same calls on the same buffers again and again
 * (a decode loop; "Ascend DeepEP MoE Dispatch Optimization", section "从 Python 接口进入真实调用链"
 * shows how much of a small dispatch's time goes to the host side of the call). moe_plan_* takes
 * the arguments of the call it names (without the stream), runs exactly that call's checks and, if
 * they pass, records the arguments in *plan and returns MOE_OK; otherwise it returns the call's
 * error and leaves *plan cleared. moe_plan_run(plan, stream) then enqueues the call's kernels on
 * stream without checking anything again, exactly as the direct call would: the buffers the plan
 * names must stay allocated and keep their sizes while the plan is in use. A plan is plain
 * caller-owned memory (no handle, nothing to free) and may be copied; moe_plan_run refuses
 * (MOE_ERR_ARG) a plan that no moe_plan_* call filled.
 *   moe_plan_layout           -> moe_layout_ex (path as there)
 *   moe_plan_dispatch_ws      -> moe_dispatch_ws
 *   moe_plan_layout_dispatch  -> moe_layout_dispatch_ex (path as there)
 *   moe_plan_combine          -> moe_combine
 *   moe_plan_layout_ws        -> moe_layout_ws (path as there)
 *   moe_plan_dispatch_planned -> moe_dispatch_planned */
typedef struct {
    uint64_t opaque[40];
} moe_plan;

int moe_plan_layout(moe_plan *plan, const int32_t *topk_idx, int32_t S, int32_t K, int32_t E,
                    int32_t P, int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                    int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                    int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                    int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status, int32_t path);

int moe_plan_dispatch_ws(moe_plan *plan, const void *x, const int32_t *slot_idx, int32_t S,
                         int32_t H, int32_t K, int32_t quant, int32_t src_rank, void *window,
                         int64_t window_bytes, void *workspace, int64_t workspace_bytes);

int moe_plan_layout_dispatch(moe_plan *plan, const int32_t *topk_idx, int32_t S, int32_t K,
                             int32_t E, int32_t P, int32_t C, uint8_t *is_token_in_rank,
                             int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                             int32_t *rank_prefix_matrix, int32_t *expert_prefix_matrix,
                             int32_t *rank_slot_base, int32_t *expert_slot_base, int32_t *slot_idx,
                             int32_t *status, const void *x, int32_t H, int32_t quant,
                             int32_t src_rank, void *window, int64_t window_bytes, int32_t path);

int moe_plan_combine(moe_plan *plan, const void *expert_out, int64_t row_stride_bytes,
                     int64_t expert_rows, const int32_t *slot_idx, const float *topk_weights,
                     int32_t S, int32_t H, int32_t K, void *y);

int moe_plan_layout_ws(moe_plan *plan, const int32_t *topk_idx, int32_t S, int32_t K, int32_t E,
                       int32_t P, int32_t C, uint8_t *is_token_in_rank, int32_t *num_tokens_per_rank,
                       int32_t *num_tokens_per_expert, int32_t *rank_prefix_matrix,
                       int32_t *expert_prefix_matrix, int32_t *rank_slot_base,
                       int32_t *expert_slot_base, int32_t *slot_idx, int32_t *status, int32_t quant,
                       int32_t path, void *workspace, int64_t workspace_bytes);
int moe_plan_dispatch_planned(moe_plan *plan, const void *x, const int32_t *slot_idx, int32_t S,
                              int32_t H, int32_t K, int32_t C, int32_t quant, int32_t src_rank,
                              void *window, int64_t window_bytes, void *workspace,
                              int64_t workspace_bytes);
int moe_plan_run(const moe_plan *plan, hipStream_t stream);

/* Static description of a moe_status value (never NULL). */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYOUT_MI355X_H */
