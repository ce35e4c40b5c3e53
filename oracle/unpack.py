"""Unpack: window slots -> compact expert input rows, their triples and scales.

Test infrastructure only (see the package docstring).

The CAM receive side ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.9 ShareToOutput)
walks the received slots in (local expert, source rank) order and copies each slot's token data to
the next row of expandXOut and its triple (source rank, token index, k) to the same row of
expandIdxOut. On one GPU the window's slots are already in expert-major, source-token order, so
row s of the compact output is slot s: the unpack strips each slot's padding and tail. For the
quantised modes the per-row scale read from the slot's scale block goes to its own vector, since
the codes alone do not carry it.
"""

import numpy as np

from .dispatch import QUANT_NONE, slot_geometry


def unpack(regions, H, quant=QUANT_NONE):
    """regions: uint8 [N, >= tail_end] (slot s = row s, as dispatch_slots returns).

    Returns (expand_x uint8 [N, payload_bytes], expand_idx int32 [N, 3],
    expand_scales float32 [N] or None for bf16).
    """
    g = slot_geometry(H, quant)
    regions = np.ascontiguousarray(regions, dtype=np.uint8)
    n = regions.shape[0]
    expand_x = regions[:, : g.payload_bytes].copy()
    expand_idx = regions[:, g.triple_off : g.triple_off + 12].copy().view("<i4").reshape(n, 3)
    scales = None
    if quant != QUANT_NONE:
        scales = regions[:, g.scale_off : g.scale_off + 4].copy().view("<f4").reshape(n)
    return expand_x, expand_idx.astype(np.int32), scales


def aligned_row_base(expert_slot_base, expert_alignment):
    """First output row of each expert when every expert's row count is rounded up to a multiple
    of expert_alignment: DeepEP's notify stage rounds each per-expert receive count up the same
    way before publishing it ("internode.cu", section 1 notify_dispatch). int64 [E + 1], [E] is the
    total number of rows the aligned layout needs."""
    esb = np.asarray(expert_slot_base, dtype=np.int64)
    counts = esb[1:] - esb[:-1]
    a = int(expert_alignment)
    aligned = -(-counts // a) * a  # ceil(count / a) * a
    return np.concatenate([[0], np.cumsum(aligned)]).astype(np.int64)


def unpack_padded(regions, expert_slot_base, H, quant, expert_alignment, out_rows):
    """Unpack into a fixed number of rows with per-expert alignment padding.

    Expert e's j-th slot (slot expert_slot_base[e] + j) goes to row aligned_row_base[e] + j;
    every other row is padding: zero payload bytes, scale 0, triple (-1, -1, -1). The output has
    exactly out_rows rows, like DeepEP's num_worst_tokens outputs ("Ascend DeepEP MoE Dispatch
    Optimization", sections "输出长度有动态和固定两种模式" and "双层解释：num_worst_tokens > 0 到底是什么":
    a fixed upper bound spares the host from reading the count back; the rows past the real
    ones carry zero data and -1 indices). Rows at or past out_rows are dropped, which the page
    describes as silent truncation; here `truncated` reports that the aligned rows did not fit.

    regions: uint8 [N, >= tail_end], slot s = row s (as dispatch_slots returns).
    Returns (expand_x uint8 [out_rows, payload_bytes], expand_idx int32 [out_rows, 3],
    expand_scales float32 [out_rows] or None for bf16, row_base int32 [E + 1], truncated bool).
    """
    g = slot_geometry(H, quant)
    ex_all, idx_all, sc_all = unpack(regions, H, quant)
    esb = np.asarray(expert_slot_base, dtype=np.int64)
    base = aligned_row_base(esb, expert_alignment)
    R = int(out_rows)
    expand_x = np.zeros((R, g.payload_bytes), dtype=np.uint8)
    expand_idx = np.full((R, 3), -1, dtype=np.int32)
    scales = None if quant == QUANT_NONE else np.zeros(R, dtype=np.float32)
    for e in range(len(esb) - 1):
        for j in range(int(esb[e + 1] - esb[e])):
            row, s = int(base[e]) + j, int(esb[e]) + j
            if row >= R:
                break
            expand_x[row] = ex_all[s]
            expand_idx[row] = idx_all[s]
            if scales is not None:
                scales[row] = sc_all[s]
    return expand_x, expand_idx, scales, base.astype(np.int32), bool(base[-1] > R)
