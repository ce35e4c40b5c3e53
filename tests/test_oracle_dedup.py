"""Pins for the oracle's per-rank deduplicated dispatch (CPU only).

* the two routing layouts of layout_worked.txt, deduplicated by hand (dedup_worked.txt);
* the rows agree with the layout's own view of the ranks: rank r's segment has
  num_tokens_per_rank[r] rows and lists exactly the tokens with is_token_in_rank[t, r];
* expanding the deduplicated rows on the receive side gives byte for byte what unpacking the
  K-fold window gives (the two paths share no code: one copies per (t, k), the other per (t, r)
  and then per local expert);
* the write volume falls by the unique-rank factor: rows = sum over r of num_tokens_per_rank.
"""

import numpy as np
import pytest

from oracle import dispatch_dedup, dispatch_slots, expand_dedup, layout, rank_rows, slot_geometry, unpack
from workloads import WORKLOADS, f32_to_bf16_input, make_inputs, random_tiny_routing


def _rows(text):
    return np.array([[int(v) for v in r.split()] for r in text.split("|")], dtype=np.int32)


@pytest.mark.parametrize("name", ["A", "B"])
def test_worked_examples(golden, name):
    sec = golden("dedup_worked.txt")[name]
    S, K, E, P = (int(v) for v in sec["S K E P"].split())
    topk = _rows(sec["topk_idx"])
    rr, base = rank_rows(topk, E, P)
    assert base.tolist() == [int(v) for v in sec["rank_token_base"].split()]
    assert np.array_equal(rr, _rows(sec["rank_row_idx"]))
    H = 16
    x = (np.arange(S * H, dtype=np.uint16).reshape(S, H) * 7 + 3).astype(np.uint16)
    reg = dispatch_dedup(x, rr, topk, E, P, src_rank=2)
    g = slot_geometry(H, 0)
    tri = reg[:, g.triple_off : g.triple_off + 12].copy().view("<i4").reshape(-1, 3)
    assert tri[:, 0].tolist() == [2] * len(tri)
    assert tri[:, 1].tolist() == [int(v) for v in sec["row_token"].split()]
    assert tri[:, 2].tolist() == [int(v) for v in sec["row_rank"].split()]
    for j, t in enumerate(tri[:, 1]):
        assert np.array_equal(reg[j, : 2 * H].view(np.uint16), x[t])
        assert not reg[j, 2 * H : g.triple_off].any()


def test_segments_match_the_layout():
    rng = np.random.default_rng(5)
    for trial in range(200):
        S, K = int(rng.integers(1, 30)), int(rng.integers(1, 6))
        P = int(rng.choice([1, 2, 3, 4]))
        E = P * int(rng.integers(1, 4))
        tab = random_tiny_routing(rng, S, K, E, p_mask=0.2, p_bad=0.05)
        lay = layout(tab, E, P, 1)
        rr, base = rank_rows(tab, E, P)
        assert np.array_equal(np.diff(base), lay["num_tokens_per_rank"])
        epr = E // P
        for r in range(P):
            seg = sorted({int(rr[t, k]) for t in range(S) for k in range(K)
                          if 0 <= tab[t, k] < E and tab[t, k] // epr == r})
            assert seg == list(range(int(base[r]), int(base[r + 1])))
            toks = [t for t in range(S) if lay["is_token_in_rank"][t, r]]
            for j, t in enumerate(toks):  # ascending token order within the segment
                ks = [k for k in range(K) if 0 <= tab[t, k] < E and tab[t, k] // epr == r]
                assert all(rr[t, k] == base[r] + j for k in ks)
        assert np.all(rr[(tab < 0) | (tab >= E)] == -1)


@pytest.mark.parametrize("cfg", [1, 3])
def test_expansion_equals_kfold_unpack(cfg):
    w = WORKLOADS[cfg]
    inp = make_inputs(w, with_expert_out=False)
    lay = layout(inp["topk_idx"], w.E, w.P, w.C)
    rr, base = rank_rows(inp["topk_idx"], w.E, w.P)
    reg = dispatch_dedup(inp["x"], rr, inp["topk_idx"], w.E, w.P, src_rank=1)
    assert reg.shape[0] == int(base[-1]) == int(lay["num_tokens_per_rank"].sum())
    ex, idx, sc = expand_dedup(reg, inp["topk_idx"], lay["slot_idx"], w.E, w.P, w.H)
    rex, ridx, _ = unpack(dispatch_slots(inp["x"], lay["slot_idx"], 0, 1), w.H, 0)
    assert sc is None and np.array_equal(ex, rex) and np.array_equal(idx, ridx)
    if cfg == 3:  # about 5.3 unique ranks per token instead of 8 copies
        assert 5.0 < reg.shape[0] / w.S < 5.6


def test_expansion_with_masks_and_duplicates():
    rng = np.random.default_rng(9)
    S, K, E, P, H = 45, 6, 12, 4, 32
    tab = random_tiny_routing(rng, S, K, E, p_mask=0.3)  # duplicates allowed
    x = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    lay = layout(tab, E, P, 5)
    rr, _ = rank_rows(tab, E, P)
    for quant in (0, 1, 2):
        ex, idx, sc = expand_dedup(dispatch_dedup(x, rr, tab, E, P, quant=quant), tab, lay["slot_idx"], E, P,
                                   H, quant)
        rex, ridx, rsc = unpack(dispatch_slots(x, lay["slot_idx"], quant, 0), H, quant)
        assert np.array_equal(ex, rex) and np.array_equal(idx, ridx), quant
        if quant:
            assert np.array_equal(sc.view(np.uint32), rsc.view(np.uint32))
