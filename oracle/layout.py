"""Routing layout: topk_idx[S,K] -> membership, counts, prefix matrices, slots.

Test infrastructure only (see the package docstring).

What is computed, and where the pages fix it:

* Route decode. A global expert id e maps to dst_rank = e / experts_per_rank and
  dst_local_expert = e % experts_per_rank ("Ascend DeepEP MoE Dispatch
  Optimization", section "一条 token 如何走完 MoE"). topk_idx is padded with -1 for
  "no expert" (same page, "输出长度有动态和固定两种模式", where the padded tail of
  topk_idx is filled with -1). Reading taken: -1 is a masked entry; any other
  id outside [0, E) is also masked and raises bit 0 of the status word.
* is_token_in_rank[t, r] = 1 iff token t has a valid expert on rank r; it is the
  [S, P] boolean routing matrix of the dispatch handle (same page, "Dispatch
  handle 六项分别保存什么"). A rank is counted once per token even when several of
  the token's experts live on it.
* Channels. Token range of channel c follows the floor-plus-remainder split the
  CAM kernels use for cores ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 8.3
  分片策略): the first S % C channels get one extra token.
* Prefix matrices. The handle's channel_prefix_matrix is indexed
  [dst][channel] and read as an inclusive running boundary: a channel starts
  where the previous channel's entry ends ("Device 侧如何把 channel 变成远端 Put",
  cursor = ... + channel_prefix[dst * C + c - 1]). Reading taken on one GPU:
  rank_prefix_matrix[r, c] = number of tokens in channels 0..c that go to
  rank r, and expert_prefix_matrix[e, c] = number of valid (t, k) entries in
  channels 0..c routed to expert e; both inclusive along c, row-major.
* Counts and slot bases. Per-rank / per-expert counts, then a prefix sum gives
  each receiver's starting offset ("Notify 先交换数量和前缀"; "internode.cu", section
  1 notify_dispatch, which sums per-rank and per-expert token counts).
  expert_slot_base is the exclusive prefix sum of num_tokens_per_expert;
  rank_slot_base[r] = expert_slot_base[r * experts_per_rank].
* Slots. The CAM pack writes a (token, k) copy at expert offset + running count
  of that expert ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 3.6
  InputToShare: dstExpertOffset + curExpertCnt). Reading taken: slots are
  ordered expert-major by global expert id, then by ascending source token,
  then ascending k; masked entries get slot -1. Because experts of one rank are
  consecutive ids, each rank's slots form one contiguous range (the compact
  destination plan of "所谓 compact plan 到底压缩了什么").
"""

import numpy as np


def channel_bounds(S, C):
    """Token range [begin_c, end_c) of each channel c in 0..C-1 (C <= S).

    per = S // C, rem = S % C; channel c starts at c*per + min(c, rem) and holds
    per + (c < rem) tokens ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 8.3).
    """
    if not (1 <= C <= S):
        raise ValueError("need 1 <= C <= S")
    c = np.arange(C, dtype=np.int64)
    per, rem = divmod(S, C)
    begin = c * per + np.minimum(c, rem)
    length = per + (c < rem)
    return begin, begin + length


def _check(topk_idx, E, P, C):
    idx = np.asarray(topk_idx)
    if idx.ndim != 2:
        raise ValueError("topk_idx must be [S, K]")
    S, K = idx.shape
    if E % P != 0:
        raise ValueError("E must be a multiple of P")
    if not (1 <= C <= S):
        raise ValueError("need 1 <= C <= S")
    return idx.astype(np.int64), S, K, E // P


def layout(topk_idx, E, P, C):
    """Vectorised definition of the routing layout. Returns a dict of numpy arrays.

    Keys: is_token_in_rank u8 [S,P], num_tokens_per_rank i32 [P],
    num_tokens_per_expert i32 [E], rank_prefix_matrix i32 [P,C],
    expert_prefix_matrix i32 [E,C], rank_slot_base i32 [P+1],
    expert_slot_base i32 [E+1], slot_idx i32 [S,K], status int (bit 0: an id
    outside [-1, E) was seen).
    """
    idx, S, K, epr = _check(topk_idx, E, P, C)

    # route decode
    valid = (idx >= 0) & (idx < E)
    status = int(np.any((idx < -1) | (idx >= E)))
    rank = np.where(valid, idx // epr, 0)
    tok = np.broadcast_to(np.arange(S)[:, None], (S, K))

    # token -> rank membership (a rank hit by several of a token's experts counts once)
    is_in = np.zeros((S, P), dtype=np.uint8)
    is_in[tok[valid], rank[valid]] = 1
    num_tokens_per_rank = is_in.sum(axis=0, dtype=np.int64)

    # per-token expert hit counts (duplicates within a row count separately)
    hits = np.zeros((S, E), dtype=np.int64)
    np.add.at(hits, (tok[valid], idx[valid]), 1)
    num_tokens_per_expert = hits.sum(axis=0)

    # inclusive prefix matrices: value at channel c counts tokens t < end_c
    _, end = channel_bounds(S, C)
    rank_prefix = np.cumsum(is_in, axis=0, dtype=np.int64)[end - 1, :].T
    expert_prefix = np.cumsum(hits, axis=0)[end - 1, :].T

    # slot bases
    expert_slot_base = np.concatenate([[0], np.cumsum(num_tokens_per_expert)])
    rank_slot_base = expert_slot_base[np.arange(P + 1) * epr]

    # slots: stable sort of flattened (t, k) by expert id; masked entries last
    flat = idx.reshape(-1)
    vflat = valid.reshape(-1)
    order = np.argsort(np.where(vflat, flat, E), kind="stable")
    n_valid = int(vflat.sum())
    slot = np.full(S * K, -1, dtype=np.int64)
    slot[order[:n_valid]] = np.arange(n_valid)

    i32 = lambda a: np.ascontiguousarray(a, dtype=np.int32)
    return {
        "is_token_in_rank": is_in,
        "num_tokens_per_rank": i32(num_tokens_per_rank),
        "num_tokens_per_expert": i32(num_tokens_per_expert),
        "rank_prefix_matrix": i32(rank_prefix),
        "expert_prefix_matrix": i32(expert_prefix),
        "rank_slot_base": i32(rank_slot_base),
        "expert_slot_base": i32(expert_slot_base),
        "slot_idx": i32(slot.reshape(S, K)),
        "status": status,
    }


def layout_bruteforce(topk_idx, E, P, C):
    """The same definition as explicit loops, for tiny inputs only.

    Counting is done entry by entry, and slots are handed out by walking the
    experts in id order and, for each, all (t, k) in lexicographic order with a
    single running counter, which is the slot order stated in the module
    docstring taken literally.
    """
    idx, S, K, epr = _check(topk_idx, E, P, C)
    idx = idx.tolist()
    status = 0
    is_in = [[0] * P for _ in range(S)]
    for t in range(S):
        for k in range(K):
            e = idx[t][k]
            if e < -1 or e >= E:
                status = 1
            if 0 <= e < E:
                is_in[t][e // epr] = 1

    # channel of each token, by walking the split rule
    per, rem = divmod(S, C)
    chan_end = []
    start = 0
    for c in range(C):
        start += per + (1 if c < rem else 0)
        chan_end.append(start)

    ntr = [sum(is_in[t][r] for t in range(S)) for r in range(P)]
    nte = [0] * E
    for t in range(S):
        for k in range(K):
            if 0 <= idx[t][k] < E:
                nte[idx[t][k]] += 1

    rpm = [[0] * C for _ in range(P)]
    epm = [[0] * C for _ in range(E)]
    for c in range(C):
        for t in range(chan_end[c]):
            for r in range(P):
                rpm[r][c] += is_in[t][r]
            for k in range(K):
                if 0 <= idx[t][k] < E:
                    epm[idx[t][k]][c] += 1

    esb = [0] * (E + 1)
    for e in range(E):
        esb[e + 1] = esb[e] + nte[e]
    rsb = [esb[r * epr] for r in range(P + 1)]

    slot = [[-1] * K for _ in range(S)]
    counter = 0
    for e in range(E):
        for t in range(S):
            for k in range(K):
                if idx[t][k] == e:
                    slot[t][k] = counter
                    counter += 1

    a = lambda x, dt=np.int32: np.array(x, dtype=dt)
    return {
        "is_token_in_rank": a(is_in, np.uint8).reshape(S, P),
        "num_tokens_per_rank": a(ntr),
        "num_tokens_per_expert": a(nte),
        "rank_prefix_matrix": a(rpm).reshape(P, C),
        "expert_prefix_matrix": a(epm).reshape(E, C),
        "rank_slot_base": a(rsb),
        "expert_slot_base": a(esb),
        "slot_idx": a(slot).reshape(S, K),
        "status": status,
    }
