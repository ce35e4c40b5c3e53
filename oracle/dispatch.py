"""Dispatch pack: K-fold expanded copy of token rows into fixed-size window slots.

Test infrastructure only (see the package docstring).

Slot format ("HCCL Window 模式 (Non-SHMEM) 代码深度剖析", section 2.3 数据区 Token 格式, and
the size check of section 8.2 Window 大小校验): each (token, k) copy occupies one
slot of slot_bytes = Ceil(Ceil(2h, 32) * 32 + 44, 512) * 512 bytes; the 44 bytes
are a 32-byte scale block plus a 12-byte triple. Inside a slot:

  [0, payload)             the token row: 2h bytes of bf16, or h bytes of fp8
  [payload, scale_off)     zero padding to a 32-byte boundary
  [scale_off, +32)         the dynamic scale as fp32 in its first 4 bytes, rest
                           zero; all 32 bytes zero when not quantising (the page
                           marks the scale as present only in DynamicQuant mode)
  [triple_off, +12)        int32 little-endian (source rank, token index, k),
                           the triple FillTriple appends (section 3.6)
  [triple_off+12, tail_end) zero padding to the end of the 128-byte line that
                           holds the triple
  [tail_end, slot_bytes)   not written: keeps whatever the window held

Readings taken (the page's box lists a 4-byte scale right after the 32-byte pad,
while the size formula counts 44 = 32 + 12): the scale gets a whole 32-byte
block, so triple_off = scale_off + 32. The page's "14848 -> 15360" for h=7168 is
not reproduced by either formula on the page; 14848 is used. The fp8 slot keeps
the bf16 slot size, since the size check is written with h * 2 regardless of
output type. Bytes past the triple are zero up to the 128-byte line end and
untouched after it; the page leaves their content open.

Dynamic quantisation: the page's DynamicQuant path goes bf16 -> fp32 -> abs ->
row max -> scale -> narrow, once per token row (section 3.6). Two narrow types:

* E4M3FN with scale = amax / 448, the largest E4M3FN magnitude, so the row's
  largest element maps to +-448. Each element is divided by the scale in fp32
  (IEEE round-to-nearest division) and then narrowed with round-to-nearest-even
  and saturation.
* INT8, the page's own output type (its tiling key selects an INT8 expandX
  when DynamicQuant is on). Reading taken for the unstated "Scale" step: the
  symmetric per-token form scale = amax / 127; each element is divided by the
  scale in fp32, rounded half to even (the CAST_RINT mode the same page uses)
  and clamped to [-127, 127]; stored as two's-complement bytes.

In both, a row of zeros gets scale 0 and all-zero codes.
"""

import struct
from collections import namedtuple

import numpy as np

from .formats import bf16_bits_to_f32, e4m3fn_encode

QUANT_NONE = 0
QUANT_FP8_E4M3_DYN = 1
QUANT_INT8_DYN = 2

SlotGeometry = namedtuple(
    "SlotGeometry", "slot_bytes payload_bytes scale_off triple_off tail_end"
)


def _ceil(a, b):
    return (a + b - 1) // b * b


def slot_geometry(H, quant=QUANT_NONE):
    """Byte geometry of one slot for hidden size H (section 8.2 and 2.3)."""
    if H <= 0 or H % 16:
        raise ValueError("H must be a positive multiple of 16")
    slot_bytes = _ceil(_ceil(2 * H, 32) + 44, 512)
    payload = 2 * H if quant == QUANT_NONE else H
    scale_off = _ceil(payload, 32)
    triple_off = scale_off + 32
    tail_end = min(_ceil(triple_off + 12, 128), slot_bytes)
    return SlotGeometry(slot_bytes, payload, scale_off, triple_off, tail_end)


def quantize_int8_dynamic(x_bits):
    """Per-token dynamic symmetric INT8 quantisation of bf16 rows.

    Returns (codes int8 [S, H], scale float32 [S]). scale = fp32(amax / 127);
    codes = clamp(rint(fp32(x / scale)), -127, 127) with rint = half to even.
    """
    xf = bf16_bits_to_f32(x_bits)
    amax = np.max(np.abs(xf), axis=1)
    scale = np.divide(amax, np.float32(127.0), dtype=np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    q = np.rint(np.divide(xf, safe[:, None], dtype=np.float32))
    codes = np.clip(q, -127, 127).astype(np.int8)
    codes[zero, :] = 0
    return codes, scale.astype(np.float32)


def quantize_e4m3_dynamic(x_bits):
    """Per-token dynamic E4M3FN quantisation of bf16 rows.

    x_bits: uint16 [S, H] bf16 bit patterns. Returns (codes uint8 [S, H],
    scale float32 [S]). amax is the fp32 maximum of |x| over the row (exact);
    scale = fp32(amax / 448); codes = E4M3FN(fp32(x / scale)).
    """
    xf = bf16_bits_to_f32(x_bits)
    amax = np.max(np.abs(xf), axis=1)
    scale = np.divide(amax, np.float32(448.0), dtype=np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    q = np.divide(xf, safe[:, None], dtype=np.float32)
    codes = e4m3fn_encode(q)
    codes[zero, :] = 0
    return codes, scale.astype(np.float32)


def dispatch_slots(x_bits, slot_idx, quant=QUANT_NONE, src_rank=0):
    """Written region of every slot: uint8 [N, tail_end], row s = slot s.

    x_bits: uint16 [S, H] bf16 bit patterns; slot_idx: int32 [S, K] from the
    layout (-1 = masked). N is the number of valid entries; slots 0..N-1 are all
    written exactly once.
    """
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    slot_idx = np.asarray(slot_idx)
    S, H = x_bits.shape
    K = slot_idx.shape[1]
    g = slot_geometry(H, quant)
    valid = slot_idx >= 0
    s = slot_idx[valid].astype(np.int64)
    t = np.broadcast_to(np.arange(S)[:, None], (S, K))[valid]
    k = np.broadcast_to(np.arange(K)[None, :], (S, K))[valid]
    n = s.size
    if n and not np.array_equal(np.sort(s), np.arange(n)):
        raise ValueError("slot_idx must be a bijection onto [0, N)")
    out = np.zeros((n, g.tail_end), dtype=np.uint8)
    if quant == QUANT_NONE:
        out[s, : 2 * H] = x_bits.view(np.uint8).reshape(S, 2 * H)[t]
    else:
        quantize = quantize_e4m3_dynamic if quant == QUANT_FP8_E4M3_DYN else quantize_int8_dynamic
        codes, scale = quantize(x_bits)
        out[s, :H] = codes.view(np.uint8)[t]
        out[s, g.scale_off : g.scale_off + 4] = scale.view(np.uint8).reshape(S, 4)[t]
    triple = np.stack([np.full(n, src_rank), t, k], axis=1).astype("<i4")
    out[s, g.triple_off : g.triple_off + 12] = triple.view(np.uint8).reshape(n, 12)
    return out


def dispatch_slots_bruteforce(x_bits, slot_idx, quant=QUANT_NONE, src_rank=0):
    """The same slots built one (t, k) at a time with byte strings (tiny inputs)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    S, H = x_bits.shape
    K = len(slot_idx[0]) if S else 0
    g = slot_geometry(H, quant)
    n = sum(1 for t in range(S) for k in range(K) if slot_idx[t][k] >= 0)
    out = np.zeros((n, g.tail_end), dtype=np.uint8)
    for t in range(S):
        row = [np.float32(v) for v in bf16_bits_to_f32(x_bits[t])]
        if quant == QUANT_NONE:
            body = x_bits[t].astype("<u2").tobytes()
            scale_bytes = b""
        else:
            amax = np.float32(0.0)
            for v in row:
                amax = max(amax, np.float32(abs(v)))
            top = np.float32(448.0 if quant == QUANT_FP8_E4M3_DYN else 127.0)
            scale = np.float32(np.float32(amax) / top)
            if amax == 0:
                codes = bytes(H)
            elif quant == QUANT_FP8_E4M3_DYN:
                codes = bytes(int(e4m3fn_encode(np.float32(v / scale))) for v in row)
            else:
                codes = bytes(int(min(127.0, max(-127.0, float(np.rint(np.float32(v / scale)))))) & 0xFF
                              for v in row)
            body = codes
            scale_bytes = struct.pack("<f", float(scale))
        for k in range(K):
            s = int(slot_idx[t][k])
            if s < 0:
                continue
            buf = bytearray(g.tail_end)
            buf[: len(body)] = body
            buf[g.scale_off : g.scale_off + len(scale_bytes)] = scale_bytes
            buf[g.triple_off : g.triple_off + 12] = struct.pack("<iii", src_rank, t, k)
            out[s] = np.frombuffer(bytes(buf), dtype=np.uint8)
    return out
