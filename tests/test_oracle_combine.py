"""Pins for the oracle's combine (CPU only).

* three tokens worked by hand, including a bf16 tie and signed zeros;
* K=1 with weight 1 reduces to a row gather (torch.index_select);
* constant rows with power-of-two weights give an exact closed form;
* identity experts (the dispatched payload fed back) with softmax weights
  return x to within a few bf16 ulp, because the weights sum to 1;
* the vectorised reduction equals the element-at-a-time fp32 loop.
"""

import numpy as np
import torch

from conftest import read_golden_sections
from oracle import bf16_bits_to_f32, combine, combine_bruteforce, dispatch_slots, layout
from workloads import WORKLOADS, f32_to_bf16_input, make_inputs, random_tiny_routing


def _rows(text, conv):
    return [[conv(v) for v in r.split()] for r in text.split("|")]


def test_worked_tokens():
    g = read_golden_sections("combine_worked.txt")[""]
    rows = f32_to_bf16_input(np.array(_rows(g["rows"], float), dtype=np.float32))
    slot = np.array(_rows(g["slot_idx"], int), dtype=np.int32)
    w = np.array(_rows(g["weights"], float), dtype=np.float32)
    y = np.array(_rows(g["y_bits"], lambda s: int(s, 16)), dtype=np.uint16)
    assert np.array_equal(combine(rows, slot, w), y)
    assert np.array_equal(combine_bruteforce(rows, slot, w), y)


def test_k1_unit_weight_is_a_gather():
    rng = np.random.default_rng(2)
    S, H, R = 50, 64, 80
    rows = f32_to_bf16_input(rng.standard_normal((R, H)).astype(np.float32))
    slot = rng.permutation(R)[:S].astype(np.int32)[:, None]
    y = combine(rows, slot, np.ones((S, 1), np.float32))
    ref = torch.index_select(torch.from_numpy(rows.view(np.int16)), 0,
                             torch.from_numpy(slot[:, 0].astype(np.int64)))
    assert np.array_equal(y, ref.numpy().view(np.uint16))


def test_constant_rows_power_of_two_weights_closed_form():
    rng = np.random.default_rng(3)
    S, K, H = 40, 4, 32
    R = S * K
    # row r holds the constant c_r = integer / 8 (exact in bf16); weights are 2^-j
    c = rng.integers(-64, 64, size=R).astype(np.float32) / 8
    rows = f32_to_bf16_input(np.repeat(c[:, None], H, axis=1))
    slot = rng.permutation(R).astype(np.int32).reshape(S, K)
    slot[rng.random((S, K)) < 0.2] = -1
    w = np.exp2(-rng.integers(0, 4, size=(S, K))).astype(np.float32)
    y = combine(rows, slot, w)
    expect = np.where(slot >= 0, w * c[np.maximum(slot, 0)], 0).sum(axis=1)
    # every partial sum is a multiple of 2^-6 below 2^5, so the fp32 accumulation is exact;
    # the one rounding left is fp32 -> bf16, done here by torch's cast
    exact = torch.from_numpy(np.repeat(expect[:, None], H, axis=1).astype(np.float32))
    ref = exact.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)


def test_identity_experts_round_trip():
    w = WORKLOADS[1]
    inp = make_inputs(w, with_expert_out=False)
    lay = layout(inp["topk_idx"], w.E, w.P, w.C)
    slots = dispatch_slots(inp["x"], lay["slot_idx"], 0, 0)
    rows = slots[:, : 2 * w.H].copy().view(np.uint16)
    y = bf16_bits_to_f32(combine(rows, lay["slot_idx"], inp["topk_weights"])).astype(np.float64)
    x = bf16_bits_to_f32(inp["x"]).astype(np.float64)
    # sum_k w_k * x = x * (1 +- a few 2^-24) before one bf16 rounding: <= 1 bf16 ulp apart
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0**-7 + 1e-30)


def test_vectorised_equals_bruteforce():
    rng = np.random.default_rng(5)
    for _ in range(5):
        S, K, H, E, P = 7, 3, 16, 6, 2
        idx = random_tiny_routing(rng, S, K, E, p_mask=0.25)
        slot = layout(idx, E, P, 2)["slot_idx"]
        R = int((slot >= 0).sum())
        rows = f32_to_bf16_input(rng.standard_normal((max(R, 1), H)).astype(np.float32))
        wts = rng.random((S, K)).astype(np.float32)
        assert np.array_equal(combine(rows, slot, wts), combine_bruteforce(rows, slot, wts))


def test_two_pass_combine_equals_the_gather():
    """Scattering expert rows to t*K + k by their triples and reducing K contiguous rows gives the
    same bits as gathering by slot index, on a workload and on tables with masked entries; the
    staging rows are the expert rows of slot_idx's inverse."""
    from oracle import combine_scatter, combine_staged, unpack

    cases = [WORKLOADS[1]]
    for w in cases:
        inp = make_inputs(w)
        lay = layout(inp["topk_idx"], w.E, w.P, w.C)
        slot = lay["slot_idx"]
        n = int(lay["expert_slot_base"][-1])
        _, idx, _ = unpack(dispatch_slots(inp["x"], slot, 0, 0), w.H, 0)
        staging = combine_scatter(inp["expert_out"], idx, n, w.S, w.K)
        for t in range(w.S):
            for k in range(w.K):
                assert np.array_equal(staging[t * w.K + k], inp["expert_out"][slot[t, k]])
        y2 = combine_staged(staging, slot, inp["topk_weights"])
        assert np.array_equal(y2, combine(inp["expert_out"], slot, inp["topk_weights"]))
    rng = np.random.default_rng(12)
    S, K, E, P, H = 33, 5, 9, 3, 40
    tab = random_tiny_routing(rng, S, K, E, p_mask=0.3)
    slot = layout(tab, E, P, 2)["slot_idx"]
    n = int((slot >= 0).sum())
    rows = f32_to_bf16_input(rng.standard_normal((S * K, H)).astype(np.float32))
    w = rng.random((S, K)).astype(np.float32)
    idx = np.full((S * K, 3), -1, np.int32)
    for t, k in zip(*np.nonzero(slot >= 0)):
        idx[slot[t, k]] = (0, t, k)
    poison = np.full((S * K, H), 0xFFFF, np.uint16)
    staging = combine_scatter(rows, idx, n, S, K, staging=poison)
    assert np.all(staging[(slot < 0).reshape(-1)] == 0xFFFF)  # masked positions never written
    assert np.array_equal(combine_staged(staging, slot, w), combine(rows, slot, w))
    assert np.array_equal(combine_staged(staging, slot, w), combine_bruteforce(rows, slot, w))
