"""Pins for the oracle's unpack (CPU only).

Unpack is the receive-side inverse of the pack: for every valid (t, k) the compact row
slot_idx[t, k] must hold x[t]'s bytes (or the token's codes and scale) and the triple
(src_rank, t, k), and the rows of one expert must be that expert's tokens in ascending order.
These are checked against x and the routing table directly, not by re-running the pack's
arithmetic.
"""

import numpy as np
import pytest

from oracle import bf16_bits_to_f32, dispatch_slots, layout, quantize_int8_dynamic, unpack
from workloads import WORKLOADS, f32_to_bf16_input, make_inputs, random_tiny_routing


def test_unpack_inverts_bf16_pack_on_workload1():
    w = WORKLOADS[1]
    inp = make_inputs(w, with_expert_out=False)
    lay = layout(inp["topk_idx"], w.E, w.P, w.C)
    ex, idx, sc = unpack(dispatch_slots(inp["x"], lay["slot_idx"], 0, 3), w.H, 0)
    assert sc is None and ex.shape == (w.S * w.K, 2 * w.H)
    rows = ex.view(np.uint16)
    for t in range(w.S):
        for k in range(w.K):
            s = lay["slot_idx"][t, k]
            assert np.array_equal(rows[s], inp["x"][t])
            assert idx[s].tolist() == [3, t, k]
    # rows of expert e are its tokens in ascending order
    esb = lay["expert_slot_base"]
    for e in range(w.E):
        tok = idx[esb[e]:esb[e + 1], 1]
        assert np.all(np.diff(tok) >= 0)
        assert np.all(inp["topk_idx"][tok].__eq__(e).any(axis=1))


@pytest.mark.parametrize("quant", [1, 2])
def test_unpack_quantised_rows_and_scales(quant):
    rng = np.random.default_rng(quant)
    S, K, E, P, H = 20, 3, 6, 3, 64
    idx_tab = random_tiny_routing(rng, S, K, E, p_mask=0.2)
    xb = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32))
    slot = layout(idx_tab, E, P, 2)["slot_idx"]
    ex, idx, sc = unpack(dispatch_slots(xb, slot, quant, 0), H, quant)
    amax = np.abs(bf16_bits_to_f32(xb)).max(axis=1)
    top = 448.0 if quant == 1 else 127.0
    for t, k in zip(*np.nonzero(slot >= 0)):
        s = slot[t, k]
        assert idx[s].tolist() == [0, t, k]
        # the scale travelling with the row is amax / top, rounded once to fp32
        assert abs(float(sc[s]) * top - amax[t]) <= amax[t] * 2.0**-23
    if quant == 2:
        codes, _ = quantize_int8_dynamic(xb)
        for t, k in zip(*np.nonzero(slot >= 0)):
            assert np.array_equal(ex[slot[t, k]].view(np.int8), codes[t])
