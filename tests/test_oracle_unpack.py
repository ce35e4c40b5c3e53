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


# ---------------------------------------------------------------- padded unpack

from oracle import aligned_row_base, slot_geometry, unpack_padded  # noqa: E402


def _labelled_regions(n, H, quant):
    """n slots whose payload bytes, scale and triple all identify the slot (no pack involved)."""
    g = slot_geometry(H, quant)
    reg = np.zeros((n, g.tail_end), dtype=np.uint8)
    for s in range(n):
        reg[s, : g.payload_bytes] = (s * 37 + np.arange(g.payload_bytes)) % 251 + 1
        reg[s, g.triple_off : g.triple_off + 12] = np.array([5, s, 100 + s], "<i4").view(np.uint8)
        if quant:
            reg[s, g.scale_off : g.scale_off + 4] = np.array([0.5 + s], "<f4").view(np.uint8)
    return reg


@pytest.mark.parametrize("quant", [0, 1])
def test_unpack_padded_worked_examples(golden, quant):
    esb = [0, 2, 2, 3, 4, 4, 4, 5, 7]
    H = 32
    reg = _labelled_regions(7, H, quant)
    g = slot_geometry(H, quant)
    for name, sec in golden("unpack_padded_worked.txt").items():
        if not name:
            continue
        A, R = (int(v) for v in sec["A R"].split())
        ex, idx, sc, base, trunc = unpack_padded(reg, esb, H, quant, A, R)
        assert base.tolist() == [int(v) for v in sec["row_base"].split()], name
        assert aligned_row_base(esb, A).tolist() == base.tolist()
        assert trunc == bool(int(sec["truncated"])), name
        src = [int(v) for v in sec["row_source"].split()]
        assert ex.shape == (R, g.payload_bytes) and idx.shape == (R, 3) and len(src) == R
        for row, s in enumerate(src):
            if s < 0:
                assert not ex[row].any() and idx[row].tolist() == [-1, -1, -1], (name, row)
                if quant:
                    assert sc[row] == 0.0
            else:
                assert np.array_equal(ex[row], reg[s, : g.payload_bytes]), (name, row)
                assert idx[row].tolist() == [5, s, 100 + s], (name, row)
                if quant:
                    assert sc[row] == np.float32(0.5 + s)
        if not quant:
            assert sc is None


def test_unpack_padded_invariants_on_random_layouts():
    """Every slot lands exactly once, in order, at an aligned block start + its index; each
    expert's block is a multiple of the alignment; padding rows are zero / -1."""
    rng = np.random.default_rng(7)
    for trial in range(30):
        S, K, E, P = int(rng.integers(1, 40)), int(rng.integers(1, 5)), 8, 4
        tab = random_tiny_routing(rng, S, K, E, p_mask=0.2)
        esb = layout(tab, E, P, 1)["expert_slot_base"]
        n = int(esb[-1])
        A = int(rng.integers(1, 9))
        base = aligned_row_base(esb, A)
        assert np.all(np.diff(base) % A == 0) and np.all(np.diff(base) >= np.diff(esb))
        assert np.all(np.diff(base) - np.diff(esb) < A)  # less than one block of padding each
        R = int(base[-1]) + int(rng.integers(-3, 4))
        if R < 1:
            continue
        reg = _labelled_regions(max(n, 1), 16, 0)[:n]
        ex, idx, _, b2, trunc = unpack_padded(reg, esb, 16, 0, A, R)
        assert trunc == (base[-1] > R)
        seen = idx[idx[:, 0] >= 0, 1]
        assert np.array_equal(seen, np.arange(len(seen)))  # slots in order, none twice
        assert len(seen) == min(n, sum(max(0, min(int(esb[e + 1] - esb[e]), R - int(base[e])))
                                       for e in range(E)))
        pad = idx[:, 0] < 0
        assert not ex[pad].any() and np.all(idx[pad] == -1)
