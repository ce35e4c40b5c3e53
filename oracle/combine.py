"""Combine: weighted K-way reduction of expert output rows back to token order.

Test infrastructure only (see the package docstring).

Arithmetic ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 7.8
ReadBufferAndWeightedSum): the accumulator starts at 0 in fp32; for each k in
ascending order the bf16 row is cast to fp32, multiplied by the token's k-th
weight, and added to the accumulator; the sum is cast back to bf16 with
round-half-even (CAST_RINT). The page stresses that accumulation is fp32.

Readings taken: each product and each sum is rounded to fp32 on its own (the
page issues Muls and Add as separate vector instructions, so no fused
multiply-add); weights are used as given; entries with slot -1 (masked) are
skipped; a token with no valid entry gives +0.0. On one GPU the K rows of token
t are gathered from the expert output buffer by slot index (row slot_idx[t, k])
instead of being first scattered to position t*K + k, which leaves the
arithmetic unchanged.
"""

import numpy as np

from .formats import bf16_bits_to_f32, f32_to_bf16_bits


def combine(expert_out_bits, slot_idx, topk_weights):
    """y bits uint16 [S, H] from expert rows uint16 [R, H] (row s = slot s)."""
    rows = np.asarray(expert_out_bits, dtype=np.uint16)
    slot_idx = np.asarray(slot_idx)
    w = np.asarray(topk_weights, dtype=np.float32)
    S, K = slot_idx.shape
    H = rows.shape[1]
    acc = np.zeros((S, H), dtype=np.float32)
    for k in range(K):
        s = slot_idx[:, k]
        live = s >= 0
        xk = bf16_bits_to_f32(rows[np.where(live, s, 0)])
        prod = np.multiply(w[:, k : k + 1], xk, dtype=np.float32)
        acc = np.where(live[:, None], np.add(acc, prod, dtype=np.float32), acc)
    return f32_to_bf16_bits(acc)


def combine_bruteforce(expert_out_bits, slot_idx, topk_weights):
    """Same reduction one element at a time with fp32 scalars (tiny inputs)."""
    rows = np.asarray(expert_out_bits, dtype=np.uint16)
    S, K = np.asarray(slot_idx).shape
    H = rows.shape[1]
    y = np.zeros((S, H), dtype=np.float32)
    for t in range(S):
        for h in range(H):
            acc = np.float32(0.0)
            for k in range(K):
                s = int(slot_idx[t][k])
                if s < 0:
                    continue
                v = bf16_bits_to_f32(rows[s, h : h + 1])[0]
                acc = np.float32(acc + np.float32(np.float32(topk_weights[t][k]) * v))
            y[t, h] = acc
    return f32_to_bf16_bits(y)


def combine_scatter(expert_out_bits, expand_idx, n_rows, S, K, staging=None):
    """First pass of the CAM combine ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 7.5
    CopyBufferToShareAndSetStatus): each expert output row is copied to the token owner's combine
    buffer at row t*K + k, with (t, k) taken from the triple the row's slot carried. (The page's
    rows are 512-byte aligned; row spacing does not change the values.)

    expert_out_bits uint16 [>= n_rows, H] (row s = slot s); expand_idx int32 [>= n_rows, 3] holds
    (src_rank, t, k). Rows whose t or k is out of range are not moved. Returns staging uint16
    [S*K, H]: the given array updated in place, or a new one with unwritten rows zero.
    """
    rows = np.asarray(expert_out_bits, dtype=np.uint16)
    H = rows.shape[1]
    out = np.zeros((S * K, H), dtype=np.uint16) if staging is None else staging
    for s in range(int(n_rows)):
        t, k = int(expand_idx[s][1]), int(expand_idx[s][2])
        if 0 <= t < S and 0 <= k < K:
            out[t * K + k] = rows[s]
    return out


def combine_staged(staging_bits, slot_idx, topk_weights):
    """Second pass of the CAM combine: token t's K rows are the contiguous rows t*K .. t*K+K-1 of
    the staging buffer, reduced with the same fp32 arithmetic as `combine`; entries masked in
    slot_idx (-1) are skipped, as the scatter never filled their rows."""
    slot_idx = np.asarray(slot_idx)
    S, K = slot_idx.shape
    pos = np.arange(S * K, dtype=np.int64).reshape(S, K)
    return combine(staging_bits, np.where(slot_idx >= 0, pos, -1), topk_weights)
