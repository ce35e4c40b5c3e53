"""Pins for the oracle's routing layout (CPU only).

* two layouts worked by hand (tests/golden/layout_worked.txt);
* the vectorised oracle equals the definitional loops on exhaustive tiny spaces
  and on seeded random tiny tables with duplicates, -1 pads and bad ids;
* invariants the pages fix, on the five full-size routing tables:
  dst_rank = e / experts_per_rank, count conservation, prefix monotonicity,
  slot bijection and stable ascending source-token order per expert range.
"""

import itertools

import numpy as np
import pytest

from conftest import read_golden_sections
from oracle import channel_bounds, layout, layout_bruteforce
from workloads import WORKLOADS, draw_routing, random_tiny_routing

KEYS = [
    "is_token_in_rank", "num_tokens_per_rank", "num_tokens_per_expert", "rank_prefix_matrix",
    "expert_prefix_matrix", "rank_slot_base", "expert_slot_base", "slot_idx",
]


def _same(a, b):
    for k in KEYS:
        assert a[k].dtype == b[k].dtype, k
        assert np.array_equal(a[k], b[k]), k
    assert a["status"] == b["status"]


def _mat(text, dt=np.int32):
    return np.array([[int(v) for v in r.split()] for r in text.split("|")], dtype=dt)


@pytest.mark.parametrize("name", ["A", "B"])
def test_worked_examples(name):
    g = read_golden_sections("layout_worked.txt")[name]
    S, K, E, P, C = (int(v) for v in g["S K E P C"].split())
    idx = _mat(g["topk_idx"])
    assert idx.shape == (S, K)
    for fn in (layout, layout_bruteforce):
        out = fn(idx, E, P, C)
        assert np.array_equal(out["is_token_in_rank"], _mat(g["is_token_in_rank"], np.uint8))
        for k in ["num_tokens_per_rank", "num_tokens_per_expert", "expert_slot_base", "rank_slot_base"]:
            assert np.array_equal(out[k], _mat(g[k])[0]), (fn.__name__, k)
        for k in ["rank_prefix_matrix", "expert_prefix_matrix", "slot_idx"]:
            assert np.array_equal(out[k], _mat(g[k])), (fn.__name__, k)
        assert out["status"] == int(g["status"])


def test_channel_split_rule():
    b, e = channel_bounds(10, 4)  # 10 = 4*2 + 2: the first two channels get 3 tokens
    assert b.tolist() == [0, 3, 6, 8] and e.tolist() == [3, 6, 8, 10]
    b, e = channel_bounds(5, 5)
    assert b.tolist() == [0, 1, 2, 3, 4]
    b, e = channel_bounds(7, 1)
    assert b.tolist() == [0] and e.tolist() == [7]


@pytest.mark.parametrize("S,K,E,P", [(2, 2, 4, 2), (3, 2, 3, 3), (4, 1, 4, 2)])
def test_exhaustive_tiny_spaces(S, K, E, P):
    """Every topk_idx in {-1..E-1}^(S*K), for C in {1, 2, S}."""
    for flat in itertools.product(range(-1, E), repeat=S * K):
        idx = np.array(flat, dtype=np.int32).reshape(S, K)
        for C in sorted({1, min(2, S), S}):
            _same(layout(idx, E, P, C), layout_bruteforce(idx, E, P, C))


def test_random_tiny_tables():
    rng = np.random.default_rng(7)
    for _ in range(10000):
        S = int(rng.integers(1, 10))
        K = int(rng.integers(1, 6))
        P = int(rng.integers(1, 5))
        E = P * int(rng.integers(1, 4))
        C = int(rng.integers(1, S + 1))
        idx = random_tiny_routing(rng, S, K, E, p_mask=0.2, p_bad=0.05)
        _same(layout(idx, E, P, C), layout_bruteforce(idx, E, P, C))


def check_invariants(idx, E, P, C, out):
    """Properties the pages fix, checked without re-deriving the layout."""
    S, K = idx.shape
    epr = E // P
    valid = (idx >= 0) & (idx < E)
    N = int(valid.sum())
    ntr, nte = out["num_tokens_per_rank"], out["num_tokens_per_expert"]
    rpm, epm = out["rank_prefix_matrix"], out["expert_prefix_matrix"]
    esb, rsb, slot = out["expert_slot_base"], out["rank_slot_base"], out["slot_idx"]
    itr = out["is_token_in_rank"]
    # conservation
    assert ntr.sum() == itr.sum()
    assert nte.sum() == N == esb[-1] == rsb[-1]
    assert np.array_equal(rpm[:, -1], ntr) and np.array_equal(epm[:, -1], nte)
    assert np.all(np.diff(rpm, axis=1) >= 0) and np.all(np.diff(epm, axis=1) >= 0)
    assert np.all(rpm[:, 0] >= 0) and np.all(epm[:, 0] >= 0)
    # rank partitions
    rank_slots = np.diff(rsb)
    assert np.all(ntr <= rank_slots) and np.all(rank_slots <= S * epr)
    # slots: bijection onto [0, N), masked -> -1
    assert np.all(slot[~valid] == -1)
    s = slot[valid]
    assert np.array_equal(np.sort(s), np.arange(N))
    # inverse map slot -> (t, k), then per-slot checks
    t_of = np.empty(N, np.int64)
    k_of = np.empty(N, np.int64)
    tt, kk = np.nonzero(valid)
    t_of[slot[tt, kk]] = tt
    k_of[slot[tt, kk]] = kk
    e_of = idx[t_of, k_of]
    # dst_rank = e / experts_per_rank: each slot in rank r's range holds an expert of rank r
    r_of = np.searchsorted(rsb, np.arange(N), side="right") - 1
    assert np.array_equal(e_of // epr, r_of)
    # each slot lies inside its expert's range, and is_token_in_rank agrees
    assert np.all((esb[e_of] <= np.arange(N)) & (np.arange(N) < esb[e_of + 1]))
    assert np.all(itr[t_of, e_of // epr] == 1)
    # stable order: inside one expert range, (t, k) strictly increase
    same_e = e_of[1:] == e_of[:-1]
    lex = t_of * K + k_of
    assert np.all(lex[1:][same_e] > lex[:-1][same_e])


@pytest.mark.parametrize("cfg", sorted(WORKLOADS))
def test_invariants_on_workload_routing(cfg):
    w = WORKLOADS[cfg]
    rng = np.random.default_rng(w.seed)
    idx, _ = draw_routing(rng, w.S, w.E, w.K, w.zipf_s)
    for C in sorted({1, 3, w.C, w.S}):
        out = layout(idx, w.E, w.P, C)
        assert out["status"] == 0
        check_invariants(idx, w.E, w.P, C, out)


def test_invariants_with_masks_and_duplicates():
    rng = np.random.default_rng(11)
    idx = random_tiny_routing(rng, 300, 6, 24, p_mask=0.3)
    for C in (1, 7, 300):
        check_invariants(idx, 24, 6, C, layout(idx, 24, 6, C))


def test_zipf_skew_concentrates_on_rank0():
    """Zipf(1.2) routing over 256 experts puts most tokens on expert 0 (rank 0 at P=128)."""
    w = WORKLOADS[5]
    rng = np.random.default_rng(w.seed)
    idx, _ = draw_routing(rng, w.S, w.E, w.K, w.zipf_s)
    out = layout(idx, w.E, w.P, w.C)
    share0 = out["num_tokens_per_expert"][0] / w.S
    assert 0.85 < share0 <= 1.0
    assert np.diff(out["rank_slot_base"])[0] > 10 * (w.S * w.K / w.P)
