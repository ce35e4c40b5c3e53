"""Per-rank deduplicated dispatch: one copy of a token per destination rank, expanded to the
rank's local experts on the receive side.

Test infrastructure only (see the package docstring).

What the pages fix ("Ascend DeepEP MoE Dispatch Optimization"):

* Section "一条 token 如何走完 MoE": when a token's experts sit on several ranks, the same hidden
  row is copied once to each of those ranks, and the destination rank rearranges what it
  received into contiguous per-local-expert input.
* Sections "P 维路由为什么值得单独优化" and "所谓 compact plan 到底压缩了什么": the compact plan keeps
  only each token's real destinations; aggregated by destination it gives one contiguous segment
  per rank listing its tokens (token ids ascending in the page's example), each entry carrying
  the token id and its local expert / top-k slot.
* Section "Dispatch handle 六项分别保存什么": send_head records, per token and rank, where the token
  went (or -1), and recv_src_idx gives each received row's source token.

Readings taken (one source rank on one GPU):

* Rank r's segment starts at rank_token_base[r], the exclusive prefix sum of num_tokens_per_rank,
  and lists the tokens that have at least one valid expert on r in ascending token order.
* rank_row_idx[t, k] is the row of token t in the segment of rank e/epr for a valid id e (equal
  for every k of the token on that rank), -1 for a masked entry. It is the compact [S, K] form of
  send_head: only real destinations are stored.
* A row holds the token's payload (bf16, or the per-token fp8 / INT8 codes with the fp32 scale in
  the scale block, quantised exactly as the K-fold dispatch does), and the triple (src_rank, t, r):
  the slot format of the K-fold dispatch with the destination rank in the third field (a row no
  longer belongs to one k).
* The receive-side expansion writes, for every valid (t, k), the row of (t, rank of e_k) to
  expert-major row slot_idx[t, k] with the triple (src_rank, t, k): exactly what unpacking the
  K-fold window gives.
"""

import numpy as np

from .dispatch import (QUANT_FP8_E4M3_DYN, QUANT_NONE, quantize_e4m3_dynamic, quantize_int8_dynamic,
                       slot_geometry)


def rank_rows(topk_idx, E, P):
    """(rank_row_idx int32 [S, K], rank_token_base int64 [P + 1]) by the definition above."""
    idx = np.asarray(topk_idx)
    S, K = idx.shape
    epr = E // P
    valid = (idx >= 0) & (idx < E)
    rank = np.where(valid, idx // epr, -1)
    members = [[t for t in range(S) if np.any(rank[t] == r)] for r in range(P)]
    base = np.concatenate([[0], np.cumsum([len(m) for m in members])]).astype(np.int64)
    pos = [dict((t, j) for j, t in enumerate(m)) for m in members]
    out = np.full((S, K), -1, dtype=np.int32)
    for t in range(S):
        for k in range(K):
            r = int(rank[t, k])
            if r >= 0:
                out[t, k] = base[r] + pos[r][t]
    return out, base


def dispatch_dedup(x_bits, rank_row_idx, topk_idx, E, P, src_rank=0, quant=QUANT_NONE):
    """Written region of every deduplicated row: uint8 [M, tail_end], row j as rank_row_idx names
    it. M = rank_token_base[P]."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    S, H = x_bits.shape
    rr = np.asarray(rank_row_idx)
    idx = np.asarray(topk_idx)
    epr = E // P
    g = slot_geometry(H, quant)
    if quant == QUANT_NONE:
        payload = x_bits.view(np.uint8).reshape(S, 2 * H)
        scales = None
    else:
        quantize = quantize_e4m3_dynamic if quant == QUANT_FP8_E4M3_DYN else quantize_int8_dynamic
        codes, scales = quantize(x_bits)
        payload = codes.view(np.uint8).reshape(S, H)
    m = int(rr.max()) + 1 if (rr >= 0).any() else 0
    out = np.zeros((m, g.tail_end), dtype=np.uint8)
    written = np.zeros(m, dtype=bool)
    for t in range(S):
        for k in range(idx.shape[1]):
            j = int(rr[t, k])
            if j < 0:
                continue
            out[j, : g.payload_bytes] = payload[t]
            if scales is not None:
                out[j, g.scale_off : g.scale_off + 4] = np.asarray(scales[t], "<f4").reshape(1).view(np.uint8)
            triple = np.array([src_rank, t, int(idx[t, k]) // epr], dtype="<i4")
            out[j, g.triple_off : g.triple_off + 12] = triple.view(np.uint8)
            written[j] = True
    if not written.all():
        raise ValueError("rank_row_idx must cover rows 0..M-1")
    return out


def expand_dedup(regions, topk_idx, slot_idx, E, P, H, quant=QUANT_NONE):
    """Receive-side expansion of the deduplicated rows: (expand_x uint8 [N, payload_bytes],
    expand_idx int32 [N, 3], expand_scales float32 [N] or None for bf16) with row s = slot s of
    the K-fold layout."""
    g = slot_geometry(H, quant)
    regions = np.ascontiguousarray(regions, dtype=np.uint8)
    idx = np.asarray(topk_idx)
    slot = np.asarray(slot_idx)
    epr = E // P
    n = int((slot >= 0).sum())
    expand_x = np.zeros((n, g.payload_bytes), dtype=np.uint8)
    expand_idx = np.zeros((n, 3), dtype=np.int32)
    scales = None if quant == QUANT_NONE else np.zeros(n, dtype=np.float32)
    for j in range(regions.shape[0]):
        src, t, r = regions[j, g.triple_off : g.triple_off + 12].copy().view("<i4").tolist()
        for k in range(idx.shape[1]):
            e = int(idx[t, k])
            if 0 <= e < E and e // epr == r:
                s = int(slot[t, k])
                expand_x[s] = regions[j, : g.payload_bytes]
                expand_idx[s] = (src, t, k)
                if scales is not None:
                    scales[s] = regions[j, g.scale_off : g.scale_off + 4].copy().view("<f4")[0]
    return expand_x, expand_idx, scales
