"""C ABI checks that need no GPU: the library loads, exports every function that
include/moe.h declares, reports the slot geometry the pages fix, and rejects bad
arguments on the host before any HIP call (fake, never-dereferenced pointers)."""

import ctypes
import os
import re

import pytest

import combine_moe_layout_02_amd as moe
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe.h")
PROBE_HEADER = os.path.join(ROOT, "include", "moe_probe.h")
A = 0x10000  # a fake, 512-byte aligned device address; never dereferenced on these paths
NULL = None


def declared_functions(header=HEADER):
    text = open(header, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(moe.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(moe._LIB_PATH)
    for name in declared_functions() + declared_functions(PROBE_HEADER):
        assert hasattr(lib, name), name


def test_probe_header_declares_the_probes():
    assert declared_functions(PROBE_HEADER) == sorted(moe.PROBES)


@pytest.mark.parametrize("fn,args", [
    ("moe_probe_fill", (NULL, 1 << 20, None)),
    ("moe_probe_fill", (A, 1000, None)),          # not a multiple of 16
    ("moe_probe_fill", (A + 8, 1 << 20, None)),   # misaligned
    ("moe_probe_read", (A, 0, A, None)),
    ("moe_probe_read", (A, 1 << 20, NULL, None)),
    ("moe_probe_copy", (A, NULL, 1 << 20, None)),
    ("moe_probe_copy", (A, A, -16, None)),
])
def test_probe_validation(fn, args):
    assert getattr(moe._lib, fn)(*args) == moe.MOE_ERR_ARG


def test_slot_geometry_matches_golden():
    with open(os.path.join(ROOT, "tests", "golden", "slot_geometry.txt")) as f:
        rows = [[int(v) for v in l.split()] for l in f if l.strip() and not l.startswith("#")]
    for H, q, slot, payload, scale_off, triple_off, tail_end in rows:
        assert moe.moe_slot_bytes(H) == slot
        assert moe.moe_slot_offsets(H, q) == dict(
            payload_bytes=payload, scale_off=scale_off, triple_off=triple_off, tail_end=tail_end)
    assert moe.moe_window_bytes(4096, 8, 7168) == 4096 * 8 * 14848


def test_slot_geometry_every_hidden_size():
    """The library's slot arithmetic against the oracle's for every accepted H and every mode."""
    import oracle

    for H in range(16, 16384 + 1, 16):
        assert moe.moe_slot_bytes(H) == oracle.slot_geometry(H, 0).slot_bytes
        for q in (0, 1, 2):
            geo = oracle.slot_geometry(H, q)
            assert moe.moe_slot_offsets(H, q) == dict(
                payload_bytes=geo.payload_bytes, scale_off=geo.scale_off, triple_off=geo.triple_off,
                tail_end=geo.tail_end), (H, q)


@pytest.mark.parametrize("H,err", [(0, -1), (8, -1), (1000, -4), (16400, -1), (32768, -1)])
def test_bad_hidden(H, err):
    assert moe._lib.moe_slot_bytes(H) == err
    assert moe._lib.moe_window_bytes(4, 2, H) == err


def layout_call(topk=A, S=64, K=8, E=256, P=8, C=16, outs=None):
    outs = outs if outs is not None else [A] * 9
    return moe._lib.moe_layout(topk, S, K, E, P, C, *outs, None)


@pytest.mark.parametrize("kw,err", [
    (dict(topk=NULL), moe.MOE_ERR_ARG),
    (dict(outs=[A] * 8 + [NULL]), moe.MOE_ERR_ARG),
    (dict(S=0), moe.MOE_ERR_ARG),
    (dict(S=70000, C=16), moe.MOE_ERR_UNSUPPORTED),
    (dict(K=0), moe.MOE_ERR_ARG),
    (dict(K=17), moe.MOE_ERR_ARG),
    (dict(E=0), moe.MOE_ERR_ARG),
    (dict(E=1024, P=8), moe.MOE_ERR_ARG),
    (dict(P=0), moe.MOE_ERR_ARG),
    (dict(E=512, P=512), moe.MOE_ERR_ARG),
    (dict(E=250, P=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(C=0), moe.MOE_ERR_ARG),
    (dict(C=65), moe.MOE_ERR_ARG),
    (dict(S=8192, C=4097), moe.MOE_ERR_ARG),
    (dict(topk=A + 2), moe.MOE_ERR_ALIGN),
    (dict(outs=[A] * 7 + [A + 1, A]), moe.MOE_ERR_ALIGN),
])
def test_layout_validation(kw, err):
    assert layout_call(**kw) == err


def dispatch_call(x=A, slot=A, S=64, H=7168, K=8, quant=0, window=A, nbytes=None):
    if nbytes is None:
        nbytes = S * K * 14848
    return moe._lib.moe_dispatch(x, slot, S, H, K, quant, 0, window, nbytes, None)


@pytest.mark.parametrize("kw,err", [
    (dict(x=NULL), moe.MOE_ERR_ARG),
    (dict(slot=NULL), moe.MOE_ERR_ARG),
    (dict(window=NULL), moe.MOE_ERR_ARG),
    (dict(K=17), moe.MOE_ERR_ARG),
    (dict(S=0), moe.MOE_ERR_ARG),
    (dict(H=7160), moe.MOE_ERR_UNSUPPORTED),
    (dict(H=8), moe.MOE_ERR_ARG),
    (dict(quant=3), moe.MOE_ERR_ARG),
    (dict(quant=-1), moe.MOE_ERR_ARG),
    (dict(x=A + 8), moe.MOE_ERR_ALIGN),
    (dict(window=A + 256), moe.MOE_ERR_ALIGN),
    (dict(slot=A + 2), moe.MOE_ERR_ALIGN),
    (dict(nbytes=64 * 8 * 14848 - 1), moe.MOE_ERR_WINDOW),
    (dict(nbytes=0), moe.MOE_ERR_WINDOW),
])
def test_dispatch_validation(kw, err):
    assert dispatch_call(**kw) == err


def dispatch_ws_call(x=A, slot=A, S=4096, H=7168, K=8, quant=0, window=A, nbytes=None, ws=A, wsbytes=None):
    if nbytes is None:
        nbytes = S * K * 14848
    if wsbytes is None:
        wsbytes = max(0, moe._lib.moe_dispatch_workspace_bytes(S, K, quant))
    return moe._lib.moe_dispatch_ws(x, slot, S, H, K, quant, 0, window, nbytes, ws, wsbytes, None)


def test_dispatch_workspace_bytes():
    # chunks of Tc = 2^floor(log2(1024 / K')) tokens (K' = K rounded up to a power of two), ceil(S / Tc)
    # chunks over 8 XCD lists of ceil(chunks / 8) chunks, Tc * K records of 8 bytes each
    assert moe.moe_dispatch_workspace_bytes(4096, 8) == 8 * 4 * 128 * 8 * 8
    assert moe.moe_dispatch_workspace_bytes(8192, 8) == 8 * 8 * 128 * 8 * 8
    assert moe.moe_dispatch_workspace_bytes(1024, 8) == 8 * 1 * 1024 * 8
    assert moe.moe_dispatch_workspace_bytes(4096, 3) == 8 * 2 * 256 * 3 * 8
    assert moe.moe_dispatch_workspace_bytes(65536, 16) == 8 * 128 * 64 * 16 * 8
    assert moe.moe_dispatch_workspace_bytes(1023, 8) == 0  # S*K below 8192: token-order pack
    assert moe.moe_dispatch_workspace_bytes(4096, 8, moe.MOE_QUANT_FP8_E4M3_DYN) == 0
    assert moe.moe_dispatch_workspace_bytes(4096, 8, moe.MOE_QUANT_INT8_DYN) == 0
    assert moe._lib.moe_dispatch_workspace_bytes(0, 8, 0) == moe.MOE_ERR_ARG
    assert moe._lib.moe_dispatch_workspace_bytes(16, 8, 3) == moe.MOE_ERR_ARG


@pytest.mark.parametrize("kw,err", [
    (dict(x=NULL), moe.MOE_ERR_ARG),
    (dict(ws=NULL), moe.MOE_ERR_ARG),
    (dict(ws=A + 8), moe.MOE_ERR_ALIGN),
    (dict(wsbytes=8 * 4 * 128 * 8 * 8 - 1), moe.MOE_ERR_WINDOW),
    (dict(nbytes=4096 * 8 * 14848 - 1), moe.MOE_ERR_WINDOW),
    (dict(window=A + 256), moe.MOE_ERR_ALIGN),
    (dict(quant=3), moe.MOE_ERR_ARG),
    (dict(H=7160), moe.MOE_ERR_UNSUPPORTED),
    (dict(K=17), moe.MOE_ERR_ARG),
])
def test_dispatch_ws_validation(kw, err):
    assert dispatch_ws_call(**kw) == err


def test_noalloc_rejects_tables_beyond_its_scratch():
    """Checked before any HIP call: the bf16 table whose plan needs more than the fixed scratch, and
    the ordinary argument errors."""
    lib = moe._lib
    assert moe.moe_dispatch_workspace_bytes(16384, 8) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    assert moe.moe_dispatch_workspace_bytes(16385, 8) > moe.MOE_NOALLOC_SCRATCH_BYTES
    nb = 16385 * 8 * 14848
    assert lib.moe_dispatch_noalloc(A, A, 16385, 7168, 8, 0, 0, A, nb, None) == moe.MOE_ERR_SCRATCH
    assert lib.moe_dispatch_noalloc(A, A, 65536, 16, 16, 0, 0, A, 65536 * 16 * 512, None) == moe.MOE_ERR_SCRATCH
    assert lib.moe_dispatch_noalloc(NULL, A, 64, 7168, 8, 0, 0, A, nb, None) == moe.MOE_ERR_ARG
    assert lib.moe_dispatch_noalloc(A, A, 64, 7168, 8, 3, 0, A, nb, None) == moe.MOE_ERR_ARG
    assert lib.moe_dispatch_noalloc(A, A, 64, 7168, 8, 0, 0, A + 256, nb, None) == moe.MOE_ERR_ALIGN
    assert lib.moe_dispatch_noalloc(A, A, 4096, 7168, 8, 0, 0, A, 4096 * 8 * 14848 - 1, None) == moe.MOE_ERR_WINDOW
    assert "scratch" in moe.moe_status_string(moe.MOE_ERR_SCRATCH)


def test_plan_size_matches_the_header():
    text = open(HEADER, encoding="utf-8").read()
    words = int(re.search(r"uint64_t opaque\[(\d+)\];", text).group(1))
    assert moe.MOE_PLAN_BYTES == 8 * words


def test_plans_check_like_the_calls_and_refuse_unfilled_plans():
    """Each moe_plan_* returns the error of the call it stands for and leaves the plan cleared, so
    moe_plan_run refuses it (no HIP call is made on these paths)."""
    lib = moe._lib
    buf = ctypes.create_string_buffer(moe.MOE_PLAN_BYTES)
    addr = ctypes.addressof(buf)
    assert lib.moe_plan_run(addr, None) == moe.MOE_ERR_ARG  # never filled
    assert lib.moe_plan_run(None, None) == moe.MOE_ERR_ARG
    outs = [A] * 9
    assert lib.moe_plan_layout(addr, A, 64, 8, 250, 8, 16, *outs, 0) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_plan_layout(addr, A, 64, 8, 256, 8, 65, *outs, 0) == moe.MOE_ERR_ARG
    assert lib.moe_plan_layout(addr, A, 513, 8, 256, 8, 16, *outs, moe.MOE_LAYOUT_SINGLE) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_plan_run(addr, None) == moe.MOE_ERR_ARG
    assert lib.moe_plan_dispatch_ws(addr, A, A, 4096, 7168, 8, 0, 0, A, 4096 * 8 * 14848, NULL, 0) == moe.MOE_ERR_ARG
    assert lib.moe_plan_dispatch_ws(addr, A, A, 64, 7168, 8, 0, 0, A, 10, NULL, 0) == moe.MOE_ERR_WINDOW
    assert lib.moe_plan_layout_dispatch(addr, A, 64, 8, 256, 8, 16, *outs, A, 7168, 0, 0, A, 0, 0) == \
        moe.MOE_ERR_WINDOW
    assert lib.moe_plan_layout_dispatch(addr, A, 64, 8, 256, 8, 16, *outs, A + 8, 7168, 0, 0, A,
                                        64 * 8 * 14848, 0) == moe.MOE_ERR_ALIGN
    assert lib.moe_plan_combine(addr, A, 14000, 512, A, A, 64, 7168, 8, A) == moe.MOE_ERR_ARG
    assert lib.moe_plan_combine(addr, A, 14336, 512, A, A, 64, 7168, 8, A + 8) == moe.MOE_ERR_ALIGN
    assert lib.moe_plan_combine(None, A, 14336, 512, A, A, 64, 7168, 8, A) == moe.MOE_ERR_ARG
    wsb = moe.moe_layout_dispatch_workspace_bytes(4096, 8, 256, 8, 128)
    assert lib.moe_plan_layout_ws(addr, A, 4096, 8, 256, 8, 128, *outs, 0, 0, NULL, wsb) == moe.MOE_ERR_ARG
    assert lib.moe_plan_layout_ws(addr, A, 4096, 8, 256, 8, 128, *outs, 0, 0, A, wsb - 1) == moe.MOE_ERR_WINDOW
    assert lib.moe_plan_layout_ws(addr, A, 4096, 8, 256, 8, 128, *outs, 4, 0, A, wsb) == moe.MOE_ERR_ARG
    assert lib.moe_plan_dispatch_planned(addr, A, A, 4096, 7168, 8, 128, 0, 0, A, 4096 * 8 * 14848, A + 4,
                                         wsb) == moe.MOE_ERR_ALIGN
    assert lib.moe_plan_dispatch_planned(addr, A, A, 4096, 7168, 8, 0, 0, 0, A, 4096 * 8 * 14848, A,
                                         wsb) == moe.MOE_ERR_ARG
    assert lib.moe_plan_run(addr, None) == moe.MOE_ERR_ARG
    assert buf.raw == bytes(moe.MOE_PLAN_BYTES)  # cleared after every failed check


def layout_dispatch_call(topk=A, S=64, K=8, E=256, P=8, C=16, outs=None, x=A, H=7168, quant=0,
                         window=A, nbytes=None):
    outs = outs if outs is not None else [A] * 9
    if nbytes is None:
        nbytes = S * K * 14848
    return moe._lib.moe_layout_dispatch(topk, S, K, E, P, C, *outs, x, H, quant, 0, window, nbytes,
                                        None)


@pytest.mark.parametrize("kw,err", [
    (dict(topk=NULL), moe.MOE_ERR_ARG),
    (dict(outs=[A] * 8 + [NULL]), moe.MOE_ERR_ARG),
    (dict(x=NULL), moe.MOE_ERR_ARG),
    (dict(window=NULL), moe.MOE_ERR_ARG),
    (dict(S=0), moe.MOE_ERR_ARG),
    (dict(K=17), moe.MOE_ERR_ARG),
    (dict(E=250, P=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(C=65), moe.MOE_ERR_ARG),
    (dict(H=7160), moe.MOE_ERR_UNSUPPORTED),
    (dict(H=8), moe.MOE_ERR_ARG),
    (dict(quant=3), moe.MOE_ERR_ARG),
    (dict(topk=A + 2), moe.MOE_ERR_ALIGN),
    (dict(outs=[A] * 7 + [A + 1, A]), moe.MOE_ERR_ALIGN),
    (dict(x=A + 8), moe.MOE_ERR_ALIGN),
    (dict(window=A + 256), moe.MOE_ERR_ALIGN),
    (dict(nbytes=64 * 8 * 14848 - 1), moe.MOE_ERR_WINDOW),
    (dict(S=8192, K=8, C=128, nbytes=8192 * 8 * 14848 - 512), moe.MOE_ERR_WINDOW),
])
def test_layout_dispatch_validation(kw, err):
    """The union of moe_layout's and moe_dispatch's checks, all before any HIP call."""
    assert layout_dispatch_call(**kw) == err


def combine_call(eo=A, stride=14336, rows=512, slot=A, w=A, S=64, H=7168, K=8, y=A):
    return moe._lib.moe_combine(eo, stride, rows, slot, w, S, H, K, y, None)


@pytest.mark.parametrize("kw,err", [
    (dict(eo=NULL), moe.MOE_ERR_ARG),
    (dict(y=NULL), moe.MOE_ERR_ARG),
    (dict(w=NULL), moe.MOE_ERR_ARG),
    (dict(stride=14320), moe.MOE_ERR_ARG),
    (dict(rows=-1), moe.MOE_ERR_ARG),
    (dict(stride=14344), moe.MOE_ERR_ALIGN),
    (dict(eo=A + 4), moe.MOE_ERR_ALIGN),
    (dict(y=A + 8), moe.MOE_ERR_ALIGN),
    (dict(w=A + 2), moe.MOE_ERR_ALIGN),
    (dict(H=7176), moe.MOE_ERR_UNSUPPORTED),
    (dict(K=0), moe.MOE_ERR_ARG),
])
def test_combine_validation(kw, err):
    assert combine_call(**kw) == err


def unpack_call(win=A, nbytes=None, num=A, S=64, K=8, H=7168, quant=0, ex=A, sc=A, idx=A):
    if nbytes is None:
        nbytes = S * K * 14848
    return moe._lib.moe_unpack(win, nbytes, num, S, K, H, quant, ex, sc, idx, None)


@pytest.mark.parametrize("kw,err", [
    (dict(win=NULL), moe.MOE_ERR_ARG),
    (dict(num=NULL), moe.MOE_ERR_ARG),
    (dict(ex=NULL), moe.MOE_ERR_ARG),
    (dict(idx=NULL), moe.MOE_ERR_ARG),
    (dict(quant=1, sc=NULL), moe.MOE_ERR_ARG),
    (dict(quant=4), moe.MOE_ERR_ARG),
    (dict(K=17), moe.MOE_ERR_ARG),
    (dict(H=7160), moe.MOE_ERR_UNSUPPORTED),
    (dict(win=A + 64), moe.MOE_ERR_ALIGN),
    (dict(ex=A + 8), moe.MOE_ERR_ALIGN),
    (dict(num=A + 2), moe.MOE_ERR_ALIGN),
    (dict(quant=1, sc=NULL), moe.MOE_ERR_ARG),
    (dict(quant=-1), moe.MOE_ERR_ARG),
    (dict(nbytes=64 * 8 * 14848 - 512), moe.MOE_ERR_WINDOW),
])
def test_unpack_validation(kw, err):
    assert unpack_call(**kw) == err


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(moe.moe_status_string(s), str) and moe.moe_status_string(s)
    assert "window" in moe.moe_status_string(moe.MOE_ERR_WINDOW)


def test_python_errors_map_to_value_error():
    with pytest.raises(ValueError):
        moe.moe_slot_bytes(1000)
    with pytest.raises(ValueError):
        moe.moe_slot_offsets(7168, 5)
    assert moe.moe_slot_offsets(7168, moe.MOE_QUANT_INT8_DYN) == moe.moe_slot_offsets(7168, 1)


def unpack_padded_call(win=A, nbytes=None, esb=A, E=256, S=64, K=8, H=7168, quant=0, align=16,
                       rows=1024, ex=A, sc=A, idx=A, base=A, st=A):
    if nbytes is None:
        nbytes = S * K * 14848
    return moe._lib.moe_unpack_padded(win, nbytes, esb, E, S, K, H, quant, align, rows, ex, sc, idx,
                                      base, st, None)


@pytest.mark.parametrize("kw,err", [
    (dict(win=NULL), moe.MOE_ERR_ARG),
    (dict(esb=NULL), moe.MOE_ERR_ARG),
    (dict(base=NULL), moe.MOE_ERR_ARG),
    (dict(st=NULL), moe.MOE_ERR_ARG),
    (dict(quant=2, sc=NULL), moe.MOE_ERR_ARG),
    (dict(E=0), moe.MOE_ERR_ARG),
    (dict(E=513), moe.MOE_ERR_ARG),
    (dict(align=0), moe.MOE_ERR_ARG),
    (dict(align=65537), moe.MOE_ERR_ARG),
    (dict(rows=0), moe.MOE_ERR_ARG),
    (dict(rows=1048577), moe.MOE_ERR_ARG),
    (dict(H=7160), moe.MOE_ERR_UNSUPPORTED),
    (dict(ex=A + 8), moe.MOE_ERR_ALIGN),
    (dict(esb=A + 2), moe.MOE_ERR_ALIGN),
    (dict(st=A + 1), moe.MOE_ERR_ALIGN),
    (dict(nbytes=64 * 8 * 14848 - 512), moe.MOE_ERR_WINDOW),
])
def test_unpack_padded_validation(kw, err):
    assert unpack_padded_call(**kw) == err


def scatter_call(eo=A, stride=14336, rows=512, idx=A, num=A, S=64, K=8, H=7168, stg=A,
                 sstride=14336, sbytes=None):
    if sbytes is None:
        sbytes = S * K * sstride
    return moe._lib.moe_combine_scatter(eo, stride, rows, idx, num, S, K, H, stg, sstride, sbytes, None)


@pytest.mark.parametrize("kw,err", [
    (dict(eo=NULL), moe.MOE_ERR_ARG),
    (dict(idx=NULL), moe.MOE_ERR_ARG),
    (dict(num=NULL), moe.MOE_ERR_ARG),
    (dict(stg=NULL), moe.MOE_ERR_ARG),
    (dict(rows=-1), moe.MOE_ERR_ARG),
    (dict(rows=1048577), moe.MOE_ERR_ARG),
    (dict(stride=14320), moe.MOE_ERR_ARG),
    (dict(sstride=14320, sbytes=10**9), moe.MOE_ERR_ARG),
    (dict(sstride=14344, sbytes=10**9), moe.MOE_ERR_ALIGN),
    (dict(stg=A + 8), moe.MOE_ERR_ALIGN),
    (dict(idx=A + 2), moe.MOE_ERR_ALIGN),
    (dict(sbytes=(64 * 8 - 1) * 14336 + 2 * 7168 - 1), moe.MOE_ERR_WINDOW),
    (dict(H=7176), moe.MOE_ERR_UNSUPPORTED),
    (dict(K=17), moe.MOE_ERR_ARG),
])
def test_combine_scatter_validation(kw, err):
    assert scatter_call(**kw) == err


def staged_call(stg=A, sstride=14336, sbytes=None, slot=A, w=A, S=64, H=7168, K=8, y=A):
    if sbytes is None:
        sbytes = S * K * sstride
    return moe._lib.moe_combine_staged(stg, sstride, sbytes, slot, w, S, H, K, y, None)


@pytest.mark.parametrize("kw,err", [
    (dict(stg=NULL), moe.MOE_ERR_ARG),
    (dict(y=NULL), moe.MOE_ERR_ARG),
    (dict(sstride=14000), moe.MOE_ERR_ARG),
    (dict(sstride=14344), moe.MOE_ERR_ALIGN),
    (dict(y=A + 8), moe.MOE_ERR_ALIGN),
    (dict(w=A + 1), moe.MOE_ERR_ALIGN),
    (dict(S=0), moe.MOE_ERR_ARG),
    (dict(sbytes=(64 * 8 - 1) * 14336 + 2 * 7168 - 1), moe.MOE_ERR_WINDOW),
    (dict(sbytes=-1), moe.MOE_ERR_WINDOW),
    (dict(sstride=2**62, sbytes=2**63 - 1), moe.MOE_ERR_WINDOW),
])
def test_combine_staged_validation(kw, err):
    assert staged_call(**kw) == err


def layout_ex_call(path, topk=A, S=64, K=8, E=256, P=8, C=16):
    return moe._lib.moe_layout_ex(topk, S, K, E, P, C, *([A] * 9), path, None)


@pytest.mark.parametrize("kw,err", [
    (dict(path=3), moe.MOE_ERR_ARG),
    (dict(path=-1), moe.MOE_ERR_ARG),
    (dict(path=moe.MOE_LAYOUT_SINGLE, S=513), moe.MOE_ERR_UNSUPPORTED),
    (dict(path=moe.MOE_LAYOUT_SINGLE, S=2048, K=2, E=16, P=4, C=1025), moe.MOE_ERR_UNSUPPORTED),
    (dict(path=moe.MOE_LAYOUT_MULTI, topk=NULL), moe.MOE_ERR_ARG),
    (dict(path=moe.MOE_LAYOUT_MULTI, E=250), moe.MOE_ERR_UNSUPPORTED),
])
def test_layout_ex_validation(kw, err):
    assert layout_ex_call(**kw) == err


def test_layout_dispatch_ex_validation():
    nb = 513 * 8 * 14848
    lib = moe._lib
    assert lib.moe_layout_dispatch_ex(A, 513, 8, 256, 8, 16, *([A] * 9), A, 7168, 0, 0, A, nb,
                                      moe.MOE_LAYOUT_SINGLE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_layout_dispatch_ex(A, 64, 8, 256, 8, 16, *([A] * 9), A, 7168, 0, 0, A, nb, 7,
                                      None) == moe.MOE_ERR_ARG
    assert lib.moe_layout_dispatch_ex(A, 64, 8, 256, 8, 16, *([A] * 9), A, 7168, 0, 0, A, 0,
                                      moe.MOE_LAYOUT_MULTI, None) == moe.MOE_ERR_WINDOW


def test_layout_dispatch_workspace_bytes():
    """0 for tables the single kernel takes; otherwise, each part rounded up to 256 bytes but the last:
    the plan (in bf16 from 8192 entries on: 8 lists of ceil(groups / 8) groups of 1024 records when a
    channel holds at most 1024 entries, else the plan kernel's size), colexcl [E, C], bucket [S*K],
    chan [2C]."""
    r = lambda v: (v + 255) // 256 * 256
    f = moe.moe_layout_dispatch_workspace_bytes
    assert f(64, 8, 256, 8, 16) == 0
    assert f(64, 8, 256, 8, 16, path=moe.MOE_LAYOUT_MULTI) == r(256 * 16 * 4) + r(512 * 4) + 2 * 16 * 4
    scratch = r(256 * 128 * 4) + r(4096 * 8 * 4) + 2 * 128 * 4
    assert f(4096, 8, 256, 8, 128) == 8 * 4 * 1024 * 8 + scratch  # 4 channels a group, 32 groups
    assert f(4096, 8, 256, 8, 128, moe.MOE_QUANT_FP8_E4M3_DYN) == scratch
    scratch16 = r(256 * 16 * 4) + r(4096 * 8 * 4) + 2 * 16 * 4
    assert f(4096, 8, 256, 8, 16) == moe.moe_dispatch_workspace_bytes(4096, 8) + scratch16
    scratch_s = r(256 * 4096 * 4) + r(4096 * 8 * 4) + 2 * 4096 * 4
    assert f(4096, 8, 256, 8, 4096) == 8 * 4 * 1024 * 8 + scratch_s  # 128 channels a group
    lib = moe._lib
    assert lib.moe_layout_dispatch_workspace_bytes(0, 8, 256, 8, 1, 0, 0) == moe.MOE_ERR_ARG
    assert lib.moe_layout_dispatch_workspace_bytes(64, 8, 250, 8, 1, 0, 0) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_layout_dispatch_workspace_bytes(64, 8, 256, 8, 65, 0, 0) == moe.MOE_ERR_ARG
    assert lib.moe_layout_dispatch_workspace_bytes(64, 8, 256, 8, 16, 3, 0) == moe.MOE_ERR_ARG
    assert lib.moe_layout_dispatch_workspace_bytes(64, 8, 256, 8, 16, 0, 9) == moe.MOE_ERR_ARG
    assert lib.moe_layout_dispatch_workspace_bytes(513, 8, 256, 8, 16, 0, 2) == moe.MOE_ERR_UNSUPPORTED


def test_layout_dispatch_ws_validation():
    """The checks of moe_layout_dispatch_ex, then the workspace: NULL, misaligned or short."""
    lib = moe._lib
    S, K, E, P, C, H = 4096, 8, 256, 8, 128, 7168
    nb = S * K * 14848
    wsb = moe.moe_layout_dispatch_workspace_bytes(S, K, E, P, C)

    def call(ws=A, wsb=wsb, nbytes=nb, x=A, path=0, quant=0):
        return lib.moe_layout_dispatch_ws(A, S, K, E, P, C, *([A] * 9), x, H, quant, 0, A, nbytes, path, ws, wsb,
                                          None)

    assert call(ws=NULL) == moe.MOE_ERR_ARG
    assert call(ws=A + 8) == moe.MOE_ERR_ALIGN
    assert call(wsb=wsb - 1) == moe.MOE_ERR_WINDOW
    assert call(nbytes=nb - 1) == moe.MOE_ERR_WINDOW
    assert call(x=NULL) == moe.MOE_ERR_ARG
    assert call(x=A + 8) == moe.MOE_ERR_ALIGN
    assert call(path=moe.MOE_LAYOUT_SINGLE) == moe.MOE_ERR_UNSUPPORTED
    assert call(path=5) == moe.MOE_ERR_ARG
    assert call(quant=4) == moe.MOE_ERR_ARG


def test_layout_ws_and_dispatch_planned_validation():
    lib = moe._lib
    S, K, E, P, C, H = 4096, 8, 256, 8, 128, 7168
    wsb = moe.moe_layout_dispatch_workspace_bytes(S, K, E, P, C)
    plan = 8 * 4 * 1024 * 8

    def layout(ws=A, nbytes=wsb, quant=0, path=0, S=S, C=C):
        return lib.moe_layout_ws(A, S, K, E, P, C, *([A] * 9), quant, path, ws, nbytes, None)

    assert layout(ws=NULL) == moe.MOE_ERR_ARG
    assert layout(ws=A + 4) == moe.MOE_ERR_ALIGN
    assert layout(nbytes=wsb - 1) == moe.MOE_ERR_WINDOW
    assert layout(quant=3) == moe.MOE_ERR_ARG
    assert layout(path=moe.MOE_LAYOUT_SINGLE) == moe.MOE_ERR_UNSUPPORTED
    assert layout(C=0) == moe.MOE_ERR_ARG

    def dispatch(ws=A, nbytes=plan, C=C, x=A, quant=0, win=S * K * 14848):
        return lib.moe_dispatch_planned(x, A, S, H, K, C, quant, 0, A, win, ws, nbytes, None)

    assert dispatch(ws=NULL) == moe.MOE_ERR_ARG
    assert dispatch(ws=A + 8) == moe.MOE_ERR_ALIGN
    assert dispatch(nbytes=plan - 1) == moe.MOE_ERR_WINDOW
    assert dispatch(C=0) == moe.MOE_ERR_ARG
    assert dispatch(C=S + 1) == moe.MOE_ERR_ARG
    assert dispatch(C=4097) == moe.MOE_ERR_ARG
    assert dispatch(x=NULL) == moe.MOE_ERR_ARG
    assert dispatch(win=S * K * 14848 - 1) == moe.MOE_ERR_WINDOW
    assert dispatch(quant=5) == moe.MOE_ERR_ARG


def test_dedup_window_bytes():
    assert moe.moe_dedup_window_bytes(4096, 8, 8, 7168) == 4096 * 8 * 14848
    assert moe.moe_dedup_window_bytes(128, 8, 4, 7168) == 128 * 4 * 14848
    assert moe._lib.moe_dedup_window_bytes(16, 8, 0, 7168) == moe.MOE_ERR_ARG
    assert moe._lib.moe_dedup_window_bytes(16, 8, 4, 1000) == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,err", [
    (dict(topk=NULL), moe.MOE_ERR_ARG),
    (dict(E=250, P=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(C=0), moe.MOE_ERR_ARG),
    (dict(C=65), moe.MOE_ERR_ARG),
    (dict(K=0), moe.MOE_ERR_ARG),
    (dict(out=A + 2), moe.MOE_ERR_ALIGN),
])
def test_rank_rows_validation(kw, err):
    a = dict(topk=A, S=64, K=8, E=256, P=8, C=16, out=A)
    a.update(kw)
    assert moe._lib.moe_rank_rows(a["topk"], a["S"], a["K"], a["E"], a["P"], a["C"], A, A, a["out"], A,
                                  None) == err


@pytest.mark.parametrize("kw,err", [
    (dict(x=NULL), moe.MOE_ERR_ARG),
    (dict(P=0), moe.MOE_ERR_ARG),
    (dict(E=12, P=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(H=7160), moe.MOE_ERR_UNSUPPORTED),
    (dict(x=A + 8), moe.MOE_ERR_ALIGN),
    (dict(win=A + 256), moe.MOE_ERR_ALIGN),
    (dict(quant=3), moe.MOE_ERR_ARG),
    (dict(nbytes=64 * 8 * 14848 - 1), moe.MOE_ERR_WINDOW),
])
def test_dispatch_dedup_validation(kw, err):
    a = dict(x=A, S=64, H=7168, K=8, E=256, P=8, quant=0, win=A, nbytes=64 * 8 * 14848)
    a.update(kw)
    assert moe._lib.moe_dispatch_dedup(a["x"], A, A, a["S"], a["H"], a["K"], a["E"], a["P"], a["quant"], 0,
                                       a["win"], a["nbytes"], None) == err


@pytest.mark.parametrize("kw,err", [
    (dict(rr=NULL), moe.MOE_ERR_ARG),
    (dict(num=NULL), moe.MOE_ERR_ARG),
    (dict(P=0), moe.MOE_ERR_ARG),
    (dict(num=A + 2), moe.MOE_ERR_ALIGN),
    (dict(quant=1, sc=NULL), moe.MOE_ERR_ARG),
    (dict(quant=-1), moe.MOE_ERR_ARG),
    (dict(ex=A + 4), moe.MOE_ERR_ALIGN),
    (dict(nbytes=100), moe.MOE_ERR_WINDOW),
])
def test_expand_dedup_validation(kw, err):
    a = dict(rr=A, num=A, S=64, K=8, P=8, H=7168, quant=0, ex=A, sc=A, nbytes=64 * 8 * 14848)
    a.update(kw)
    assert moe._lib.moe_expand_dedup(A, a["nbytes"], a["rr"], A, a["num"], a["S"], a["K"], a["P"], a["H"],
                                     a["quant"], a["ex"], a["sc"], A, None) == err
