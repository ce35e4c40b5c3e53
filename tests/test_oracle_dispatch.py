"""Pins for the oracle's dispatch pack (CPU only).

* slot geometry: the page's printed 14848 B at h=7168 and the size formula
  worked by hand (tests/golden/slot_geometry.txt);
* bf16 slots: the payload is byte-identical to the token row, the triple read
  back from slot s inverts slot_idx, and every pad byte is zero;
* fp8 slots: a row quantised by hand, the E4M3 rounding error bound, the amax
  element landing on +-448, a zero row, and the scale as amax/448 to 1 ulp;
* int8 slots: a row quantised by hand with rounding ties, the half-step error
  bound, the amax element landing on +-127, a zero row;
* the vectorised pack equals the one-entry-at-a-time byte-string build.
"""

import struct

import numpy as np
import pytest

from conftest import read_golden_sections
from oracle import (
    bf16_bits_to_f32,
    dispatch_slots,
    dispatch_slots_bruteforce,
    e4m3fn_decode,
    layout,
    quantize_e4m3_dynamic,
    quantize_int8_dynamic,
    slot_geometry,
)
from workloads import WORKLOADS, f32_to_bf16_input, make_inputs, random_tiny_routing


def _geometry_rows():
    rows = []
    with open("tests/golden/slot_geometry.txt") as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(v) for v in line.split()])
    return rows


def test_slot_geometry_golden():
    rows = _geometry_rows()
    assert any(r[0] == 7168 and r[2] == 14848 for r in rows)
    for H, q, *expect in rows:
        assert list(slot_geometry(H, q)) == expect, (H, q)


def test_slot_geometry_rejects_bad_h():
    for H in (0, 8, 1000):
        with pytest.raises(ValueError):
            slot_geometry(H)


def _tiny_case(seed, S=9, K=3, E=6, P=3, H=64, C=2):
    rng = np.random.default_rng(seed)
    idx = random_tiny_routing(rng, S, K, E, p_mask=0.2)
    x = f32_to_bf16_input(rng.standard_normal((S, H)).astype(np.float32) * 3)
    return x, layout(idx, E, P, C)["slot_idx"]


def _check_bf16_slots(x, slot, src_rank):
    S, H = x.shape
    g = slot_geometry(H, 0)
    out = dispatch_slots(x, slot, 0, src_rank)
    for t, k in zip(*np.nonzero(slot >= 0)):
        s = slot[t, k]
        reg = out[s]
        assert reg.tobytes()[: 2 * H] == x[t].astype("<u2").tobytes()
        assert struct.unpack_from("<iii", reg.tobytes(), g.triple_off) == (src_rank, t, k)
        assert not reg[2 * H : g.triple_off].any() and not reg[g.triple_off + 12 :].any()
    return out


def test_bf16_payload_and_triple_tiny():
    x, slot = _tiny_case(3)
    _check_bf16_slots(x, slot, src_rank=5)


def test_bf16_payload_and_triple_workload1():
    w = WORKLOADS[1]
    inp = make_inputs(w, with_expert_out=False)
    slot = layout(inp["topk_idx"], w.E, w.P, w.C)["slot_idx"]
    out = _check_bf16_slots(inp["x"], slot, src_rank=0)
    assert out.shape == (w.S * w.K, slot_geometry(w.H).tail_end)


@pytest.mark.parametrize("quant", [0, 1, 2])
def test_vectorised_equals_bruteforce(quant):
    for seed in range(4):
        x, slot = _tiny_case(seed, H=32 if seed % 2 else 48)
        a = dispatch_slots(x, slot, quant, src_rank=seed)
        b = dispatch_slots_bruteforce(x, slot, quant, src_rank=seed)
        assert np.array_equal(a, b)


def test_fp8_worked_row():
    g = read_golden_sections("fp8_quant_worked.txt")[""]
    x = np.array([float(s) for s in g["x"].split()], dtype=np.float32)
    xb = f32_to_bf16_input(x)[None, :]
    assert np.array_equal(bf16_bits_to_f32(xb)[0], x)  # the row is exact in bf16
    codes, scale = quantize_e4m3_dynamic(xb)
    assert scale.view(np.uint32)[0] == int(g["scale_bits"], 16)
    assert codes[0].tolist() == [int(s, 16) for s in g["codes"].split()]
    # and the same bytes land in the slot, scale in the first 4 bytes of its block
    slot = np.array([[0]], dtype=np.int32)
    geo = slot_geometry(16, 1)
    reg = dispatch_slots(xb, slot, 1, src_rank=2)[0]
    assert reg[:16].tolist() == codes[0].tolist()
    assert reg[16 : geo.scale_off].sum() == 0
    assert struct.unpack_from("<f", reg.tobytes(), geo.scale_off)[0] == 2.0**-7
    assert struct.unpack_from("<iii", reg.tobytes(), geo.triple_off) == (2, 0, 0)


def _ulp32(v):
    v = np.abs(np.asarray(v, dtype=np.float32))
    return np.nextafter(v, np.float32(np.inf)) - v


def test_fp8_quant_error_bound_on_outlier_rows():
    """|decode(q)*scale - x| <= (ulp_e4m3(v)/2 + 2^-24 |v|) * scale, v = x/scale (float64)."""
    w = WORKLOADS[4]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    xf = (rng.standard_normal((64, w.H)) * w.x_std).astype(np.float32)
    xf = np.where(rng.random(xf.shape) < w.outlier_prob, xf * w.outlier_mul, xf).astype(np.float32)
    xf[3] = 0.0  # an all-zero row
    xb = f32_to_bf16_input(xf)
    codes, scale = quantize_e4m3_dynamic(xb)
    x = bf16_bits_to_f32(xb).astype(np.float64)
    amax = np.abs(x).max(axis=1)
    assert scale[3] == 0 and not codes[3].any()
    live = amax > 0
    # scale is amax / 448 rounded once to fp32
    assert np.all(np.abs(scale[live].astype(np.float64) * 448 - amax[live])
                  <= 448 * _ulp32(scale[live]) / 2 * (1 + 1e-12))
    sc = scale[live].astype(np.float64)[:, None]
    v = x[live] / sc
    dec = e4m3fn_decode(codes[live])
    a = np.minimum(np.abs(v), 448.0)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    half_ulp = np.exp2(e - 3) / 2
    err = np.abs(dec * sc - x[live])
    bound = (half_ulp + 2.0**-24 * np.abs(v)) * sc + np.maximum(np.abs(v) - 448, 0) * sc
    assert np.all(err <= bound * (1 + 1e-9))
    # the largest element of each row encodes to +-448
    arg = np.abs(x[live]).argmax(axis=1)
    top = codes[live][np.arange(live.sum()), arg]
    assert np.all((top == 0x7E) | (top == 0xFE))
    # signs follow x (nonzero codes)
    nz = (codes[live] & 0x7F) != 0
    assert np.all(((codes[live] >> 7) == 1)[nz] == (x[live] < 0)[nz])


def test_int8_worked_row():
    g = read_golden_sections("int8_quant_worked.txt")[""]
    x = np.array([float(s) for s in g["x"].split()], dtype=np.float32)
    xb = f32_to_bf16_input(x)[None, :]
    assert np.array_equal(bf16_bits_to_f32(xb)[0], x)
    codes, scale = quantize_int8_dynamic(xb)
    assert scale.view(np.uint32)[0] == int(g["scale_bits"], 16)
    assert codes[0].view(np.uint8).tolist() == [int(s, 16) for s in g["codes"].split()]
    geo = slot_geometry(16, 2)
    reg = dispatch_slots(xb, np.array([[0]], dtype=np.int32), 2, src_rank=1)[0]
    assert reg[:16].tolist() == codes[0].view(np.uint8).tolist()
    assert struct.unpack_from("<f", reg.tobytes(), geo.scale_off)[0] == 2.0**-6
    assert struct.unpack_from("<iii", reg.tobytes(), geo.triple_off) == (1, 0, 0)


def test_int8_quant_error_bound():
    """|q*scale - x| <= scale/2 (plus fp32 division rounding); amax maps to +-127; zero rows."""
    w = WORKLOADS[4]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    xf = (rng.standard_normal((64, 1024)) * w.x_std).astype(np.float32)
    xf = np.where(rng.random(xf.shape) < w.outlier_prob, xf * w.outlier_mul, xf).astype(np.float32)
    xf[5] = 0.0
    xb = f32_to_bf16_input(xf)
    codes, scale = quantize_int8_dynamic(xb)
    x = bf16_bits_to_f32(xb).astype(np.float64)
    assert scale[5] == 0 and not codes[5].any()
    live = np.abs(x).max(axis=1) > 0
    sc = scale[live].astype(np.float64)[:, None]
    q = codes[live].astype(np.float64)
    assert np.all(np.abs(q) <= 127)
    err = np.abs(q * sc - x[live])
    assert np.all(err <= sc * (0.5 + 127 * 2.0**-23))
    arg = np.abs(x[live]).argmax(axis=1)
    top = q[np.arange(live.sum()), arg]
    assert np.all(np.abs(top) == 127)
    assert np.all(np.sign(q[q != 0]) == np.sign(x[live][q != 0]))
