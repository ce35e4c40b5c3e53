"""Number-format conversions the path needs, written from the format definitions.

Test infrastructure only (see the package docstring): nothing outside tests,
the smoke check and the bench's CPU baseline may import this module.

* bfloat16: the top 16 bits of an IEEE-754 binary32. Narrowing rounds to
  nearest, ties to even, on the discarded low 16 bits. The CAM combine casts its
  fp32 accumulator back to bf16 with CAST_RINT ("HCCL Window 模式 (Non-SHMEM)
  代码深度剖析", section 7.8 ReadBufferAndWeightedSum); rint is round-half-even.
* E4M3FN: the OCP 8-bit floating point format (OFP8, E4M3 variant): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits, subnormals when the exponent
  field is 0, no infinities, and only S.1111.111 is NaN. Largest finite
  magnitude 448 (S.1111.110), smallest normal 2^-6, smallest subnormal 2^-9.
  Narrowing rounds to nearest, ties to even, and saturates to +-448
  ("satfinite"), keeping the sign of zero.

All arithmetic below is done in float64 or on integer bit patterns, where every
step is exact, so the only rounding is the one the definition asks for.
"""

import numpy as np

E4M3FN_MAX = 448.0


def f32_to_bf16_bits(a):
    """Round fp32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    For a finite input with bit pattern u, the result is the high half of
    u + 0x7FFF + bit16(u): adding just under half an ulp of bf16, plus one when
    the kept lsb is odd, carries into the kept bits exactly when the discarded
    half is above the midpoint, or at the midpoint with an odd kept lsb.
    NaNs become quiet NaNs with the same sign.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    is_nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    quiet = ((u >> 16) | 0x0040) & 0xFFFF
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def bf16_bits_to_f32(b):
    """Widen bfloat16 bit patterns to fp32 (exact: append 16 zero bits)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _e4m3fn_table():
    """Value of each of the 256 E4M3FN codes (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            vals[code] = np.nan
        elif exp_field == 0:
            vals[code] = sign * mant * 2.0 ** -9  # subnormal: 0.mmm x 2^(1-7)
        else:
            vals[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return vals


_E4M3FN_VALUES = _e4m3fn_table()


def e4m3fn_decode(codes):
    """Decode uint8 E4M3FN codes to float64 values."""
    return _E4M3FN_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3fn_encode(v):
    """Encode values to E4M3FN codes: round to nearest even, saturate to +-448.

    Steps, on |v| (the sign bit is re-attached at the end, so -0.0 -> 0x80):
      1. |v| >= 448 -> 448 (satfinite; 448 is the largest finite code).
      2. Otherwise take the binade e = floor(log2|v|), but never below -6 (the
         subnormal range shares the spacing of the lowest normal binade).
         The code spacing there is ulp = 2^(e-3) (3 mantissa bits).
      3. m = |v| / ulp rounded half-to-even (exact in float64: division by a
         power of two). m == 16 means rounding carried into the next binade.
      4. Pack: in the subnormal range (e == -6, m < 8) the code is m; otherwise
         exponent field e + 7 and mantissa m - 8.
    NaN inputs map to 0x7F (with sign).
    """
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    sat = a >= E4M3FN_MAX
    a_fin = np.where(sat, 1.0, a)
    # frexp: a = f * 2^ex with f in [0.5, 1)  =>  floor(log2 a) = ex - 1
    _, ex = np.frexp(np.where(a_fin > 0, a_fin, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    ulp = np.ldexp(1.0, e - 3)
    m = np.rint(a_fin / ulp).astype(np.int64)  # rint: ties to even
    carry = m == 16
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 8, m)
    sub = (e == -6) & (m < 8)
    code = np.where(sub, m, ((e + 7) << 3) | (m - 8))
    code = np.where(a == 0, 0, code)
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)
