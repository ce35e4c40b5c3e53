"""Pins for the oracle's number-format converters (CPU only).

bf16 narrowing is checked against torch's fp32 -> bf16 cast (a library routine
with the same round-to-nearest-even definition); E4M3FN narrowing against a
brute-force nearest-code search over the decoded code table and against
torch.float8_e4m3fn, plus a row worked by hand.
"""

import numpy as np
import pytest
import torch

from conftest import read_golden_sections
from oracle import bf16_bits_to_f32, e4m3fn_decode, e4m3fn_encode, f32_to_bf16_bits


def _fp32_sweep():
    """All exponents x (strided mantissas + edge mantissas + bf16 halfway ties), both signs."""
    exps = np.arange(0, 255, dtype=np.uint32)  # finite values only
    mants = np.concatenate([
        np.arange(0, 1 << 23, 4099, dtype=np.uint32),
        np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x10000, 0x18000, 0x7F8000,
                  0x7FFFFF, 0x7F7FFF, 0x3F8000, 0x7FC000], dtype=np.uint32),
    ])
    bits = (exps[:, None] << 23) | mants[None, :]
    bits = bits.reshape(-1)
    bits = np.concatenate([bits, bits | 0x80000000])
    return bits.view(np.float32)


def test_bf16_matches_torch_cast_on_dense_sweep():
    v = _fp32_sweep()
    ours = f32_to_bf16_bits(v)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mism = np.nonzero(ours != ref)[0]
    assert mism.size == 0, f"{mism.size} mismatches, first input bits {v[mism[:4]].view(np.uint32)}"


def test_bf16_ties_and_widen():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert f32_to_bf16_bits(np.float32(1 + 2**-8))[()] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert f32_to_bf16_bits(np.float32(1 + 3 * 2**-8))[()] == 0x3F82
    assert f32_to_bf16_bits(np.float32(-0.0))[()] == 0x8000
    b = np.arange(0, 1 << 16, dtype=np.uint16)
    f = bf16_bits_to_f32(b)
    finite = ~np.isnan(f)
    assert np.array_equal(f32_to_bf16_bits(f[finite]), b[finite])  # widen is exact


def test_e4m3fn_decode_spot_values():
    t = e4m3fn_decode(np.arange(256))
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0**-6 and t[0x01] == 2.0**-9 and t[0x07] == 7 * 2.0**-9
    assert t[0x38] == 1.0 and t[0x39] == 1.125
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x80] == 0 and np.signbit(t[0x80])
    fin = t[~np.isnan(t)]
    assert fin.size == 254 and np.unique(fin).size == 253  # +0 and -0 compare equal


def _nearest_code_bruteforce(v):
    """Nearest finite code by exhaustive search; ties -> even code; |v| > 448 -> 448."""
    table = e4m3fn_decode(np.arange(0x7F))  # non-negative finite codes 0x00..0x7E
    a = np.minimum(np.abs(v), 448.0)
    d = np.abs(a[:, None] - table[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes prefer the even one (lsb 0)
    even = cand & ((np.arange(0x7F) & 1) == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (pick | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def test_e4m3fn_encode_matches_bruteforce_nearest_code():
    table = e4m3fn_decode(np.arange(0x7F))
    mids = (table[:-1] + table[1:]) / 2
    rng = np.random.default_rng(0)
    v = np.concatenate([
        table, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        rng.uniform(0, 480, 20000), np.exp2(rng.uniform(-14, 9, 20000)),
        [0.0, 448.0, 464.0, 470.0, 479.9],
    ])
    v = np.concatenate([v, -v]).astype(np.float32).astype(np.float64)
    assert np.array_equal(e4m3fn_encode(v), _nearest_code_bruteforce(v))


def test_e4m3fn_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 50000), np.exp2(rng.uniform(-12, 8.8, 50000))])
    v = v.astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3fn_encode(v), ref)


def test_e4m3fn_saturates_and_keeps_zero_sign():
    big = np.array([448.0, 448.00003, 463.9, 464.0, 1e6, np.inf], dtype=np.float32)
    assert np.all(e4m3fn_encode(big) == 0x7E)
    assert np.all(e4m3fn_encode(-big) == 0xFE)
    assert e4m3fn_encode(np.float32(-0.0))[()] == 0x80
    assert e4m3fn_encode(np.float32(0.0))[()] == 0x00


def test_e4m3fn_worked_row():
    g = read_golden_sections("fp8_quant_worked.txt")[""]
    x = np.array([float(s) for s in g["x"].split()], dtype=np.float32)
    codes = np.array([int(s, 16) for s in g["codes"].split()], dtype=np.uint8)
    scale = np.uint32(int(g["scale_bits"], 16)).view(np.float32)
    assert np.array_equal(e4m3fn_encode(x / scale), codes)
