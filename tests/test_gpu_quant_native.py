"""The pack's quantisation arithmetic on the GPU against the oracle, through the native checker
tests/c_abi/quant_gpu.cpp (built with the library's flags from combine_moe_layout_02_amd/csrc/pack_rows.h,
the helpers the pack kernels use):

* the E4M3FN encode (gfx950's packed fp8 convert after a clamp to +-448) over every non-negative
  finite fp32 input: the GPU reports, for each code, the smallest input that produces it and
  checks that the codes never decrease and that -q gives the code of q with the sign bit; the
  test compares those 127 code boundaries with the oracle's encoder;
* the reciprocal division with two FMA corrections (div_by_scale): for row maxima drawn as bf16
  values, the codes of every bf16 x the row can hold, against the oracle's quantisers on that
  row; and, over 20,000 further scales, the GPU's own count of quotients and codes that differ
  from the IEEE division's.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle
from conftest import ROOT

pytestmark = pytest.mark.gpu

EXE = os.path.join(ROOT, "tests", "c_abi", "quant_gpu")
FAST_MIN_SCALE = np.float32(2.0**-90)  # the smallest scale the reciprocal division takes


def run(*args):
    assert os.path.exists(EXE), f"{EXE} is missing: run python combine_moe_layout_02_amd/build.py"
    print("quant_gpu", *args[:1], flush=True)
    res = subprocess.run([EXE, *args], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    print(res.stdout, flush=True)


def oracle_code(bits):
    return int(oracle.e4m3fn_encode(np.array([bits], np.uint32).view(np.float32))[0])


def oracle_code_boundaries():
    """Smallest non-negative finite input (as fp32 bits) of each code 0..126 under the oracle's
    encoder, by bisection (the encoder is monotone in the magnitude)."""
    first = []
    for c in range(0x7F):
        lo, hi = 0, 0x7F800000
        while lo < hi:
            mid = (lo + hi) // 2
            if oracle_code(mid) >= c:
                hi = mid
            else:
                lo = mid + 1
        assert oracle_code(lo) == c and (lo == 0 or oracle_code(lo - 1) == c - 1), c
        first.append(lo)
    return np.array(first, np.uint32)


def test_e4m3_encode_every_fp32(tmp_path):
    out = tmp_path / "cvt.bin"
    run("cvt", str(out))
    raw = out.read_bytes()
    first = np.frombuffer(raw, np.uint32, 256)
    non_monotone, sign_mismatch = (int(v) for v in np.frombuffer(raw, np.uint64, 2, 1024))
    assert non_monotone == 0
    assert sign_mismatch == 0
    ref = oracle_code_boundaries()
    bad = np.nonzero(first[:0x7F] != ref)[0]
    assert bad.size == 0, [(int(c), hex(int(first[c])), hex(int(ref[c]))) for c in bad[:5]]
    assert np.all(first[0x7F:] == 0xFFFFFFFF)  # no NaN code, no sign bit for q >= 0


def finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    return bits[(bits & 0x7F80) != 0x7F80].astype(np.uint16)


def test_fast_division_codes_match_oracle(tmp_path):
    rng = np.random.default_rng(91)
    xs_all = finite_bf16()
    mag = np.abs((xs_all.astype(np.uint32) << 16).view(np.float32))
    # row maxima: powers of two and their bf16 neighbours, the largest bf16, and random values
    amax = [0x3F80 + d for d in (-1, 0, 1)] + [0x43E0, 0x42FE, 0x7F7F, 0x0B80, 0x0C00]
    amax += list(rng.integers(0x0C00, 0x7F7F, 100))
    rows, scales = [], []
    for quant, top in ((1, 448.0), (2, 127.0)):
        for ab in amax:
            a = float((np.uint32(ab) << 16).view(np.float32))
            scale = np.divide(np.float32(a), np.float32(top), dtype=np.float32)
            if scale < FAST_MIN_SCALE:
                continue
            rows.append((quant, ab, xs_all[mag <= a]))
            scales.append(scale)
    n = len(scales)
    src, out = tmp_path / "scales.bin", tmp_path / "div.bin"
    np.array(scales, np.float32).tofile(src)
    run("div", str(src), str(out))
    raw = np.fromfile(out, np.uint8)
    e4m3 = raw[: n * 65536].reshape(n, 65536)
    int8 = raw[n * 65536 : 2 * n * 65536].reshape(n, 65536)
    q_bad, code_bad = (int(v) for v in raw[2 * n * 65536 :].view(np.uint64))
    assert q_bad == 0 and code_bad == 0
    for i, (quant, ab, xs) in enumerate(rows):
        row = np.concatenate([np.array([ab], np.uint16), xs])[None, :]
        quantize = oracle.quantize_e4m3_dynamic if quant == 1 else oracle.quantize_int8_dynamic
        codes, scale = quantize(row)
        assert np.float32(scale[0]) == np.float32(scales[i])
        got = (e4m3 if quant == 1 else int8)[i][row[0].astype(np.int64)]
        want = codes[0].view(np.uint8)
        if not np.array_equal(got, want):
            j = int(np.nonzero(got != want)[0][0])
            raise AssertionError(f"amax bits {ab:#x} quant {quant}: x bits {int(row[0, j]):#x} "
                                 f"gpu {int(got[j]):#x} oracle {int(want[j]):#x}")


def test_fast_division_matches_ieee_over_many_scales(tmp_path):
    """20,000 log-uniform scales over the reciprocal division's whole range: the GPU compares every
    quotient that can change a code with its IEEE quotient, and both codes."""
    rng = np.random.default_rng(92)
    scales = np.float32(2.0) ** rng.uniform(-90, 121, 20000).astype(np.float32)
    scales = scales[(scales >= FAST_MIN_SCALE) & np.isfinite(scales)].astype(np.float32)
    src, out = tmp_path / "scales.bin", tmp_path / "count.bin"
    scales.tofile(src)
    run("divcount", str(src), str(out))
    q_bad, code_bad = (int(v) for v in np.fromfile(out, np.uint64))
    assert q_bad == 0 and code_bad == 0
